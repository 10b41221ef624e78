// dcn_msda.hip -- multi-scale deformable attention sampling (fp32 or bf16
// operands, fp32 accumulation and output).
//
// Page 5 (deformops README, "Multi-scale deformable attention"): value
// (B, sum_l H_l W_l, G, D) holds L flattened feature maps, locations
// (B, Q, G, L, K, 2) are normalised (x, y) in [0, 1], weights (B, Q, G, L*K)
// are used as given or normalised by a softmax over levels and points; the
// output (B, Q, G*D) is the attention-weighted sum of the bilinear samples.
// This is the deformable convolution's gather (coordinate stage, corner
// gather, weighted blend) without the dense contraction, so it is bound by
// the corner traffic, not by matrix math.
//
// A normalised location maps to pixel coordinates with the half-pixel
// convention, p = (x * W - 0.5, y * H - 0.5), each product and difference
// rounded to fp32 (no fused multiply-add); corners outside the level count as
// zero.
//
// One workgroup handles NP (b, q, g) pairs (32 for fp32, 64 for bf16, so
// that the gather's D/VEC lanes per pair fill the workgroup either way):
//   (a) coefficient stage: every (pair, point) gets its four corner weights
//       (attention x bilinear x validity) and corner byte offsets in an LDS
//       table (the softmax, when asked for, is reduced over the 256/NP
//       threads of a pair first);
//   (b) gather: D/VEC lanes per pair each own 16 bytes (VEC = 4 fp32 or 8
//       bf16 channels) of the head's D channels; per point they read the
//       table entry (a broadcast), issue the four 16-byte corner loads
//       (buffer loads: an outside corner reads zero) and accumulate in fp32;
//       one or two 16-byte fp32 stores per lane.
// bf16 operands (page 5: half precision throughout) are widened exactly to
// fp32; nothing is rounded back to bf16.

#include "dcn_device.h"
#include "dcn_launch.h"

namespace dcn {

template <class T>
__device__ __forceinline__ void msda_acc(float* acc, float w, u32x4 v);
template <>
__device__ __forceinline__ void msda_acc<float>(float* acc, float w, u32x4 v) {
#pragma unroll
  for (int c = 0; c < 4; ++c) acc[c] = __builtin_fmaf(w, __uint_as_float(v[c]), acc[c]);
}
template <>
__device__ __forceinline__ void msda_acc<__bf16>(float* acc, float w, u32x4 v) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    acc[2 * q] = __builtin_fmaf(w, __uint_as_float(v[q] << 16), acc[2 * q]);
    acc[2 * q + 1] = __builtin_fmaf(w, __uint_as_float(v[q] & 0xffff0000u), acc[2 * q + 1]);
  }
}

template <class T, int NPAIR>
__global__ __launch_bounds__(256) void msda_kernel(MsdaArgs a) {
  constexpr int TPP = 256 / NPAIR;  // coefficient threads per pair
  constexpr int MAXLK = kMsdaMaxLevels * kMsdaMaxPoints;
  constexpr int E = sizeof(T);
  constexpr int VEC = 16 / E;  // channels per 16-byte lane load
  const T* const wts = static_cast<const T*>(a.weights);
  const T* const locs = static_cast<const T*>(a.locations);
  // the table, sized by the launch for this problem's L * K points per pair
  // (a smaller table leaves room for more workgroups per CU):
  // Cw [NPAIR * LK] corner weights, then Co [NPAIR * LK] corner byte offsets
  extern __shared__ __attribute__((aligned(16))) char msda_smem[];
  __shared__ int lv[kMsdaMaxLevels][3];  // H, W, start

  const int tid = threadIdx.x;
  const int LK = a.L * a.K;
  f32x4* const Cw = reinterpret_cast<f32x4*>(msda_smem);
  u32x4* const Co = reinterpret_cast<u32x4*>(msda_smem + (size_t)NPAIR * LK * 16);
  if (tid < a.L) {
    lv[tid][0] = a.H[tid];
    lv[tid][1] = a.W[tid];
    lv[tid][2] = a.start[tid];
  }
  __syncthreads();
  const int logical = xcd_logical_block(blockIdx.x, gridDim.x);
  const int64_t n0 = (int64_t)logical * NPAIR;

  // ---- (a) coefficients: thread -> pair tid / TPP, points e = tid % TPP + TPP * r
  {
    const int pl = tid / TPP, sub = tid % TPP;
    const int64_t n = n0 + pl;
    const bool pin = n < a.npairs;
    const int npt = (LK + TPP - 1) / TPP;  // points per thread (<= MAXLK / TPP)
    float logit[MAXLK / TPP];
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < MAXLK / TPP; ++r) {
      const int e = sub + TPP * r;
      logit[r] = (r < npt && e < LK && pin) ? to_f32<T>(wts[n * LK + e]) : -INFINITY;
      mx = fmaxf(mx, logit[r]);
    }
    float sum = 0.f;
    if (a.softmax) {
#pragma unroll
      for (int sh = TPP / 2; sh >= 1; sh >>= 1) mx = fmaxf(mx, __shfl_xor(mx, sh, TPP));
#pragma unroll
      for (int r = 0; r < MAXLK / TPP; ++r)
        if (logit[r] != -INFINITY) sum += expf(logit[r] - mx);
#pragma unroll
      for (int sh = TPP / 2; sh >= 1; sh >>= 1) sum += __shfl_xor(sum, sh, TPP);
    }
    const int64_t g = pin ? n % a.G : 0;
    const int64_t b = pin ? n / ((int64_t)a.Q * a.G) : 0;
#pragma unroll
    for (int r = 0; r < MAXLK / TPP; ++r) {
      const int e = sub + TPP * r;
      if (r >= npt || e >= LK) continue;
      const int l = e / a.K;
      const int H = lv[l][0], W = lv[l][1], st = lv[l][2];
      f32x4 w4 = {0.f, 0.f, 0.f, 0.f};
      u32x4 o4 = {kNoCorner, kNoCorner, kNoCorner, kNoCorner};
      if (pin) {
        const float att = a.softmax ? expf(logit[r] - mx) / sum : logit[r];
        const float x = to_f32<T>(locs[(n * LK + e) * 2]);
        const float y = to_f32<T>(locs[(n * LK + e) * 2 + 1]);
        const float px = __fsub_rn(__fmul_rn(x, (float)W), 0.5f);
        const float py = __fsub_rn(__fmul_rn(y, (float)H), 0.5f);
        const float x0 = floorf(px), y0 = floorf(py);
        const float fx = __fsub_rn(px, x0), fy = __fsub_rn(py, y0);
        const float wv[4] = {(1.f - fy) * (1.f - fx), (1.f - fy) * fx, fy * (1.f - fx), fy * fx};
        const int ix = (int)fminf(fmaxf(x0, -1.0f), (float)W);
        const int iy = (int)fminf(fmaxf(y0, -1.0f), (float)H);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float yy = __fadd_rn(y0, (float)(q >> 1)), xx = __fadd_rn(x0, (float)(q & 1));
          const bool ok = yy >= 0.f && yy <= (float)(H - 1) && xx >= 0.f && xx <= (float)(W - 1);
          if (ok) {
            w4[q] = att * wv[q];
            const int64_t pix = (int64_t)st + (int64_t)(iy + (q >> 1)) * W + ix + (q & 1);
            o4[q] = (uint32_t)(((b * a.S + pix) * a.G + g) * a.D * E);
          }
        }
      }
      Cw[pl * LK + e] = w4;
      Co[pl * LK + e] = o4;
    }
  }
  __syncthreads();

  // ---- (b) gather: lanes per pair = D / VEC
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(a.value, a.value_bytes);
  const int lpp = a.D / VEC;
  const int ppp = 256 / lpp;  // pairs per pass
  const int pr = tid / lpp, sl = tid - (tid / lpp) * lpp;
  for (int p0 = 0; p0 < NPAIR; p0 += ppp) {
    const int pl = p0 + pr;
    if (pr >= ppp || pl >= NPAIR) continue;
    const int64_t n = n0 + pl;
    if (n >= a.npairs) continue;
    float acc[VEC];
#pragma unroll
    for (int c = 0; c < VEC; ++c) acc[c] = 0.f;
    const uint32_t lb = (uint32_t)sl * 16u;
    int e = 0;
    for (; e + 4 <= LK; e += 4) {  // four points (16 loads) in flight
      u32x4 v[4][4];
      f32x4 w[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const u32x4 o = Co[pl * LK + e + u];
        w[u] = Cw[pl * LK + e + u];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[u][q] = load16(vr, o[q] + lb);  // kNoCorner + lb stays outside
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int q = 0; q < 4; ++q) msda_acc<T>(acc, w[u][q], v[u][q]);
    }
    for (; e < LK; ++e) {
      const u32x4 o = Co[pl * LK + e];
      const f32x4 w = Cw[pl * LK + e];
#pragma unroll
      for (int q = 0; q < 4; ++q) msda_acc<T>(acc, w[q], load16(vr, o[q] + lb));
    }
    float* dst = a.out + n * a.D + VEC * sl;
#pragma unroll
    for (int h = 0; h < VEC / 4; ++h)
      *reinterpret_cast<f32x4*>(dst + 4 * h) =
          f32x4{acc[4 * h], acc[4 * h + 1], acc[4 * h + 2], acc[4 * h + 3]};
  }
}

hipError_t launch_msda(const MsdaArgs& a, int bf16, hipStream_t s) {
  const int LK = a.L * a.K;
  // 64 pairs for bf16 when the table (64 * LK * 32 bytes) stays within 64 KB
  const int NPAIR = bf16 && LK <= 32 ? 64 : 32;
  const int64_t nblk = (a.npairs + NPAIR - 1) / NPAIR;
  if (nblk <= 0) return hipSuccess;
  if (nblk > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (LK < 1 || LK > kMsdaMaxLevels * kMsdaMaxPoints) return hipErrorInvalidValue;
  if (bf16 && NPAIR == 64)
    hipLaunchKernelGGL((msda_kernel<__bf16, 64>), dim3((unsigned)nblk), dim3(256),
                       (size_t)NPAIR * LK * 32, s, a);
  else if (bf16)
    hipLaunchKernelGGL((msda_kernel<__bf16, 32>), dim3((unsigned)nblk), dim3(256),
                       (size_t)NPAIR * LK * 32, s, a);
  else
    hipLaunchKernelGGL((msda_kernel<float, 32>), dim3((unsigned)nblk), dim3(256),
                       (size_t)NPAIR * LK * 32, s, a);
  return hipGetLastError();
}

}  // namespace dcn
