// dcn_dsample.hip -- single-scale deformable sampling (the DCNv3 operator).
//
// Page 5 (deformops README, "Single-scale deformable sampling"): the
// deformable convolution's sampling and aggregation without its spatial
// weight.  The C channels are G groups of D; for output pixel (ho, wo) and
// channel c of group g
//   out = sum_k a_{g,k} * bilinear(x[:, :, c], ho - ph + i_k + dy_{g,k}, wo - pw + j_k + dx_{g,k})
// with the convolution's sampling point and per-corner zero fill (the corner
// stage of dcn_device.h), and a_{g,k} the aggregation weight as given or a
// softmax over the K taps.
//
// There is no contraction, so this is a gather: per pixel, G*K*4 corner
// slices of D channels come through the vector L1 and are blended into
// fp32 accumulators that stay in registers over all taps.  A workgroup owns
// 64 pixels x CT = NV * VEC channels (VEC channels = one 16-byte vector):
//   * per tap, its corner table (four byte offsets, four weights x a) for
//     every (pixel, group) the tile touches is built once into LDS by one
//     thread per entry from coalesced offset / weight loads (64 consecutive
//     pixels of one plane), the loads of the next tap in flight meanwhile;
//   * every thread owns NV/4 (pixel, vector) units; consecutive lanes take
//     consecutive vectors of one pixel, so the lanes of one group's corner
//     read one contiguous D*e-byte run; all units' corner loads are issued
//     before any blend;
//   * the output is written NHWC (16-byte stores, consecutive lanes
//     contiguous) or NCHW through an LDS transpose (64-pixel runs).

#include <type_traits>

#include "dcn_device.h"
#include "dcn_launch.h"

namespace dcn {

namespace {

template <class T>
__device__ __forceinline__ void blend_acc(float* acc, float w, u32x4 v);
template <>
__device__ __forceinline__ void blend_acc<float>(float* acc, float w, u32x4 v) {
#pragma unroll
  for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(w, __uint_as_float(v[e]), acc[e]);
}
template <>
__device__ __forceinline__ void blend_acc<__bf16>(float* acc, float w, u32x4 v) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    acc[2 * q] = __builtin_fmaf(w, __uint_as_float(v[q] << 16), acc[2 * q]);
    acc[2 * q + 1] = __builtin_fmaf(w, __uint_as_float(v[q] & 0xffff0000u), acc[2 * q + 1]);
  }
}

}  // namespace

// GT: the most groups one channel tile can touch -- NV + 1 in general (groups
// of one 16-byte vector, misaligned), 8 for a launch whose groups are wide
// enough (fewer table entries per thread, fewer registers, more workgroups
// per CU).
template <class T, int NV, bool NHWC, int GT>
__global__ __launch_bounds__(256) void dsample_kernel(DsArgs a) {
  constexpr int E = sizeof(T);
  constexpr int VEC = 16 / E;           // channels per 16-byte vector
  constexpr int CT = NV * VEC;          // channels per workgroup
  constexpr int M = 64;                 // pixels per workgroup
  constexpr int U = M * NV / 256;       // (pixel, vector) units per thread
  constexpr int GTM = GT;               // most groups one channel tile touches
  constexpr int EPT = (GTM * M + 255) / 256;  // table entries per thread
  constexpr int TAB_BYTES = GTM * M * 32;
  constexpr int TR_BYTES = NHWC ? 0 : CT * (M + 1) * 4;
  constexpr int SMEM = TAB_BYTES > TR_BYTES ? TAB_BYTES : TR_BYTES;
  static_assert(U >= 1 && (M * NV) % 256 == 0, "units per thread");

  __shared__ __attribute__((aligned(16))) char smem[SMEM];
  f32x4* const Cw = reinterpret_cast<f32x4*>(smem);              // [gl][m]
  u32x4* const Co = reinterpret_cast<u32x4*>(smem + GTM * M * 16);

  const int tid = threadIdx.x;
  const int logical = xcd_logical_block(blockIdx.x, gridDim.x);
  const int ctile = logical % a.n_ctiles;
  const int t2 = logical / a.n_ctiles;
  const int tile = t2 % a.tiles_per_img;
  const int b = t2 / a.tiles_per_img;
  const int hw0 = tile * M;
  const int C = a.G * a.D;
  const int c0 = ctile * CT;
  const int g_first = c0 / a.D;
  const int g_last = (min(C, c0 + CT) - 1) / a.D;
  const int n_ent = (g_last - g_first + 1) * M;
  const uint32_t row_bytes = (uint32_t)C * E;

  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, a.x_bytes);
  const __amdgpu_buffer_rsrc_t offr = make_rsrc(a.offset, a.offset_bytes);
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(a.weights, a.weights_bytes);

  // ---- table entries owned by this thread: (group g_first + gl, pixel m)
  int e_g[EPT], e_hw[EPT], e_ho[EPT], e_wo[EPT];
  bool e_live[EPT], e_in[EPT];
#pragma unroll
  for (int r = 0; r < EPT; ++r) {
    const int e = tid + 256 * r;
    e_live[r] = e < n_ent;
    const int gl = e_live[r] ? e / M : 0, m = e % M;
    e_g[r] = g_first + gl;
    e_hw[r] = hw0 + m;
    e_in[r] = e_live[r] && e_hw[r] < a.HoWo;
    e_ho[r] = e_hw[r] / a.Wo;
    e_wo[r] = e_hw[r] - e_ho[r] * a.Wo;
  }
  // byte offsets of (g, k)'s dy plane and weight plane at the entry's pixel
  auto off_at = [&](int r, int k) {
    return ((uint32_t)((b * a.G + e_g[r]) * 2 * a.K + 2 * k) * (uint32_t)a.HoWo +
            (uint32_t)e_hw[r]) * E;
  };
  auto w_at = [&](int r, int k) {
    return ((uint32_t)((b * a.G + e_g[r]) * a.K + k) * (uint32_t)a.HoWo + (uint32_t)e_hw[r]) * E;
  };

  // softmax over the K taps of each entry: running maximum and sum (fp32)
  float s_max[EPT], s_inv[EPT];
#pragma unroll
  for (int r = 0; r < EPT; ++r) {
    s_max[r] = 0.0f;
    s_inv[r] = 1.0f;
  }
  if (a.softmax) {
    // the logits of up to KB taps are loaded at once (one memory latency per
    // KB taps instead of one per tap), then reduced from registers
    constexpr int KB = 9;
#pragma unroll
    for (int r = 0; r < EPT; ++r) {
      if (!e_in[r]) continue;
      float mx = -INFINITY, sum = 0.0f;
      for (int k0 = 0; k0 < a.K; k0 += KB) {
        float lg[KB];
#pragma unroll
        for (int q = 0; q < KB; ++q)
          lg[q] = k0 + q < a.K ? load_scalar<T>(wr, w_at(r, k0 + q)) : -INFINITY;
        float cm = mx;
#pragma unroll
        for (int q = 0; q < KB; ++q) cm = fmaxf(cm, lg[q]);
        sum *= expf(mx - cm);  // rescale the running sum to the new maximum
#pragma unroll
        for (int q = 0; q < KB; ++q)
          if (k0 + q < a.K) sum += expf(lg[q] - cm);
        mx = cm;
      }
      s_max[r] = mx;
      s_inv[r] = 1.0f / sum;
    }
  }

  float n_dy[EPT], n_dx[EPT], n_w[EPT];
  auto t_load = [&](int k) {
#pragma unroll
    for (int r = 0; r < EPT; ++r) {
      const uint32_t ob = e_in[r] ? off_at(r, k) : 0u;
      n_dy[r] = load_scalar<T>(offr, ob);
      n_dx[r] = load_scalar<T>(offr, ob + (uint32_t)a.HoWo * E);
      n_w[r] = load_scalar<T>(wr, e_in[r] ? w_at(r, k) : 0u);
    }
  };
  auto t_build = [&](int k) {
    const int i = k / a.kw, j = k - (k / a.kw) * a.kw;
#pragma unroll
    for (int r = 0; r < EPT; ++r) {
      if (!e_live[r]) continue;
      const TapCorners t = tap_corners((float)(e_ho[r] - a.ph + i), (float)(e_wo[r] - a.pw + j),
                                       n_dy[r], n_dx[r], a.H, a.W);
      const float aw = a.softmax ? expf(n_w[r] - s_max[r]) * s_inv[r] : n_w[r];
      const float hy = 1.0f - t.p.ly, hx = 1.0f - t.p.lx;
      const float wv[4] = {hy * hx, hy * t.p.lx, t.p.ly * hx, t.p.ly * t.p.lx};
      const uint32_t base =
          ((uint32_t)((b * a.H + t.y0) * a.W + t.x0)) * row_bytes + (uint32_t)(e_g[r] * a.D) * E;
      f32x4 w4;
      u32x4 o4;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bool ok = e_in[r] && ((t.valid >> q) & 1u);
        w4[q] = ok ? wv[q] * aw : 0.0f;
        o4[q] = ok ? base + (uint32_t)((q >> 1) * a.W + (q & 1)) * row_bytes : kNoCorner;
      }
      const int e = tid + 256 * r;
      Cw[e] = w4;
      Co[e] = o4;
    }
  };

  // ---- units: L = u * 256 + tid -> pixel m = L / NV, vector v = L % NV
  int u_ent[U];
  uint32_t u_cb[U];
  bool u_ok[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int L = u * 256 + tid;
    const int m = L / NV, v = L % NV;
    const int ch = c0 + v * VEC;
    u_ok[u] = ch < C;
    const int g = u_ok[u] ? ch / a.D : g_first;
    u_ent[u] = (g - g_first) * M + m;
    u_cb[u] = (uint32_t)(ch - g * a.D) * E;  // the vector's byte offset inside its group
  }
  float acc[U][VEC];
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[u][e] = 0.0f;

  t_load(0);
  for (int k = 0; k < a.K; ++k) {
    __syncthreads();  // the previous tap's gather is done with the table
    t_build(k);
    if (k + 1 < a.K) t_load(k + 1);
    __syncthreads();
    u32x4 cv[U][4];
    f32x4 cw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const u32x4 off = Co[u_ent[u]];
      cw[u] = Cw[u_ent[u]];
#pragma unroll
      for (int q = 0; q < 4; ++q) cv[u][q] = load16(xr, u_ok[u] ? off[q] + u_cb[u] : kNoCorner);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int q = 0; q < 4; ++q) blend_acc<T>(acc[u], cw[u][q], cv[u][q]);
  }

  // ---- store (fp32)
  if constexpr (NHWC) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int L = u * 256 + tid;
      const int m = L / NV, v = L % NV;
      const int hw = hw0 + m;
      if (!u_ok[u] || hw >= a.HoWo) continue;
      float* dst = a.out + ((size_t)b * a.HoWo + hw) * C + c0 + v * VEC;
#pragma unroll
      for (int h = 0; h < VEC / 4; ++h)
        *reinterpret_cast<f32x4*>(dst + 4 * h) =
            f32x4{acc[u][4 * h], acc[u][4 * h + 1], acc[u][4 * h + 2], acc[u][4 * h + 3]};
    }
  } else {
    __syncthreads();  // the table is dead; its LDS becomes the transpose tile
    float* tr = reinterpret_cast<float*>(smem);  // [CT][M + 1]
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int L = u * 256 + tid;
      const int m = L / NV, v = L % NV;
#pragma unroll
      for (int e = 0; e < VEC; ++e) tr[(v * VEC + e) * (M + 1) + m] = acc[u][e];
    }
    __syncthreads();
    for (int e = tid; e < CT * M; e += 256) {
      const int c = e / M, m = e % M;
      const int hw = hw0 + m;
      if (c0 + c >= C || hw >= a.HoWo) continue;
      a.out[((size_t)b * C + c0 + c) * a.HoWo + hw] = tr[c * (M + 1) + m];
    }
  }
}

namespace {
template <class T, int NV>
hipError_t launch_ds_nv(const DsArgs& a, bool nhwc, int64_t nblk, hipStream_t s) {
  const dim3 grid((unsigned)nblk), block(256);
  constexpr int VEC = 16 / (int)sizeof(T);
  // groups a tile of NV * VEC channels can touch: one more than it holds
  const bool wide = (NV * VEC + a.D - 1) / a.D + 1 <= 8 && NV + 1 > 8;
  if (wide && nhwc) hipLaunchKernelGGL((dsample_kernel<T, NV, true, 8>), grid, block, 0, s, a);
  else if (wide) hipLaunchKernelGGL((dsample_kernel<T, NV, false, 8>), grid, block, 0, s, a);
  else if (nhwc) hipLaunchKernelGGL((dsample_kernel<T, NV, true, NV + 1>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((dsample_kernel<T, NV, false, NV + 1>), grid, block, 0, s, a);
  return hipGetLastError();
}
template <class T>
hipError_t launch_ds_t(const DsArgs& a, int nv, bool nhwc, int64_t nblk, hipStream_t s) {
  switch (nv) {
    case 4: return launch_ds_nv<T, 4>(a, nhwc, nblk, s);
    case 8: return launch_ds_nv<T, 8>(a, nhwc, nblk, s);
    case 16: return launch_ds_nv<T, 16>(a, nhwc, nblk, s);
    default: return hipErrorInvalidValue;
  }
}
}  // namespace

int dsample_vectors_per_tile(int C, int bf16) {
  const int vec = bf16 ? 8 : 4;
  const int nvec = (C + vec - 1) / vec;
  return nvec >= 16 ? 16 : nvec > 4 ? 8 : 4;
}

hipError_t launch_dsample(const DsArgs& a, int bf16, int nhwc, hipStream_t s) {
  const int nv = dsample_vectors_per_tile(a.G * a.D, bf16);
  const int64_t nblk = (int64_t)a.B * a.tiles_per_img * a.n_ctiles;
  if (nblk <= 0) return hipSuccess;
  if (nblk > 0x7fffffff) return hipErrorInvalidConfiguration;
  return bf16 ? launch_ds_t<__bf16>(a, nv, nhwc, nblk, s)
              : launch_ds_t<float>(a, nv, nhwc, nblk, s);
}

}  // namespace dcn
