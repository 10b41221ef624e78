// dcn_wsk.hip -- fp32 fused DCNv2 forward with the k-axis split across waves.
//
// Same operator as dcn_kernels.hip (page 1, "deform_conv.py": sample the input
// bilinearly at (h - pad + i + dy, w - pad + j + dx), corners outside count as
// zero, times the mask, contract over (tap, channel) with the weight, + bias).
// This variant serves fp32 problems with up to 128 output channels (the
// BiRefNet-decoder-like 64 -> 64, 7x7 shape), where one workgroup's output
// tile is small enough for each wave to own all of it:
//
//  * a workgroup = 4 waves = M output pixels x NO output channels; every k-block
//    is one tap x 64 input channels, and wave w owns channels [16w, 16w+16) of
//    each block: it gathers only those, keeps its own LDS column tile and
//    coefficient table, and loads its own quarter of the weight block straight
//    into registers in MFMA fragment order;
//  * so the main loop has no workgroup barrier: the waves never wait for each
//    other, and the two waves a SIMD holds (two workgroups per CU) overlap one
//    wave's corner-load latency with the other's MFMAs;
//  * each wave accumulates a partial [M x NO] over its channel quarter; the four
//    partials are summed once through LDS at the end, then bias and store.
//
// Per step kb (one tap, one 64-channel chunk) a wave issues, in this order,
// the weight fragments of kb+1, the corner loads of kb+1 and the offset/mask
// loads of a tap three steps ahead; runs the MFMAs of kb; turns the offsets
// loaded one step earlier into corner weights/offsets; and blends the corners
// of kb+1 into its idle column buffer.  The loads are branch-free (outside
// corners are buffer offsets past the end, which read as zero), so every wait
// is only for what is older than the loads still in flight.

#include <type_traits>

#include "dcn_device.h"
#include "dcn_launch.h"

namespace dcn {

template <int M, int NO, bool NHWC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void fused_wsk_kernel(FusedArgs a) {
  constexpr int CB = 64;          // channels per k-block
  constexpr int NPASS = M / 16;   // gather passes: 16 pixels x 4 channel quads each
  constexpr int MT = M / 16, NT = NO / 16;
  constexpr int A_FLOATS = M * 16;                       // one wave's column tile
  constexpr int MAIN_BYTES = 4 * 2 * A_FLOATS * 4 + 4 * 2 * M * 32;
  constexpr int RST = M + 4;                             // reduction row stride
  constexpr int RED_BYTES = 4 * NO * RST * 4;
  constexpr int SMEM = MAIN_BYTES > RED_BYTES ? MAIN_BYTES : RED_BYTES;
  static_assert(M == 32 || M == 64, "tile rows");
  static_assert(NO % 16 == 0, "tile columns");

  __shared__ __attribute__((aligned(16))) char smem[SMEM];
  float* const As = reinterpret_cast<float*>(smem);                       // [w][2][M][16]
  f32x4* const Cw = reinterpret_cast<f32x4*>(smem + 4 * 2 * A_FLOATS * 4);  // [w][2][M]
  u32x4* const Co = reinterpret_cast<u32x4*>(smem + 4 * 2 * A_FLOATS * 4 + 4 * 2 * M * 16);
  float* const red = reinterpret_cast<float*>(smem);                      // [w][NO][RST]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  const int logical = xcd_logical_block(blockIdx.x, gridDim.x);
  const int otile = logical % a.n_otiles;
  const int t2 = logical / a.n_otiles;
  const int tile = t2 % a.tiles_per_img;
  const int b = t2 / a.tiles_per_img;
  const int hw0 = tile * M;
  const int NKB = a.K * a.nchunk;

  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, a.x_bytes);
  const float* maskp = static_cast<const float*>(a.mask);
  const bool has_mask = maskp != nullptr;
  const __amdgpu_buffer_rsrc_t offr = make_rsrc(a.offset, a.offset_bytes);
  const __amdgpu_buffer_rsrc_t mskr =
      make_rsrc(has_mask ? a.mask : a.offset, has_mask ? a.mask_bytes : 0u);
  const float* wblocks = static_cast<const float*>(a.wpack) +
                         (size_t)otile * a.K * a.nchunk * (CB * NO);
  const uint32_t row_bytes = (uint32_t)a.C * 4;

  // ---- (a) coefficients: lane m computes pixel m's four corners for a tap
  float c_dy[2], c_dx[2], c_mk[2];
  auto coef_load = [&](int kt, auto set_tag) {
    constexpr int S = decltype(set_tag)::value;
    const uint32_t hw = (uint32_t)(hw0 + lane);
    const uint32_t ob = ((uint32_t)(b * 2 * a.K + 2 * kt) * (uint32_t)a.HoWo + hw) * 4;
    const uint32_t mb = ((uint32_t)(b * a.K + kt) * (uint32_t)a.HoWo + hw) * 4;
    c_dy[S] = load_scalar<float>(offr, ob);
    c_dx[S] = load_scalar<float>(offr, ob + (uint32_t)a.HoWo * 4);
    c_mk[S] = load_scalar<float>(mskr, mb);
  };
  auto coef_finish = [&](int kt, auto set_tag) {
    constexpr int S = decltype(set_tag)::value;
    const int slot = kt & 1;
    const int i = kt / a.kw;
    const int j = kt - i * a.kw;
    const int hw = hw0 + lane;
    const int ho = hw / a.Wo;
    const int wo = hw - ho * a.Wo;
    const TapPoint t = tap_point(c_dy[S], c_dx[S], ho - a.ph + i, wo - a.pw + j, a.H, a.W);
    const float mk = has_mask ? c_mk[S] : 1.0f;
    const float hy = 1.0f - t.ly, hx = 1.0f - t.lx;
    const float wv[4] = {hy * hx, hy * t.lx, t.ly * hx, t.ly * t.lx};
    const bool in_tile = hw < a.HoWo;
    const int y0 = (int)fminf(fmaxf(t.y0, -1.0f), (float)a.H);
    const int x0 = (int)fminf(fmaxf(t.x0, -1.0f), (float)a.W);
    f32x4 w4;
    u32x4 o4;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const bool ok = in_tile && ((t.valid >> c) & 1u);
      w4[c] = ok ? wv[c] * mk : 0.0f;
      o4[c] = ok ? (uint32_t)((b * a.H + y0 + (c >> 1)) * a.W + x0 + (c & 1)) * row_bytes
                 : kNoCorner;
    }
    if (lane < M) {
      Cw[(wave * 2 + slot) * M + lane] = w4;
      Co[(wave * 2 + slot) * M + lane] = o4;
    }
  };

  // ---- (b) corners: lane = (pixel of the pass, channel quad of the wave's 16)
  const int pp = lane >> 2;
  const int q4 = lane & 3;
  u32x4 gv[NPASS][4];
  uint32_t goff[NPASS][4];  // byte offsets of the next block's corner loads
  auto gather_offsets = [&](int kb) {
    const int kt = kb / a.nchunk;
    const int cc = kb - kt * a.nchunk;
    const int ch = cc * CB + wave * 16 + q4 * 4;
    const bool chan_ok = ch < a.C;
    const uint32_t cbyte = (uint32_t)ch * 4;
    const u32x4* co = Co + (wave * 2 + (kt & 1)) * M;
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
      const u32x4 off = co[ps * 16 + pp];
#pragma unroll
      for (int c = 0; c < 4; ++c) goff[ps][c] = chan_ok ? off[c] + cbyte : kNoCorner;
    }
  };
  // Column tile row p holds the wave's 16 channels as 4 quads; quad q sits at
  // position q ^ ((p >> 2) & 3) so that both the blend writes (16 lanes = 4
  // pixels x 4 quads) and the MFMA reads (16 lanes = 16 pixels, one quad) hit
  // 64 distinct banks.
  auto a_index = [](int p, int q) { return p * 16 + ((q ^ ((p >> 2) & 3)) << 2); };
  auto finish_gather = [&](int kb, int buf) {
    const int kt = kb / a.nchunk;
    const f32x4* cw = Cw + (wave * 2 + (kt & 1)) * M;
    float* A = As + (wave * 2 + buf) * A_FLOATS;
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
      const int p = ps * 16 + pp;
      const u32x4 r = Ops<float>::blend(cw[p], gv[ps][0], gv[ps][1], gv[ps][2], gv[ps][3]);
      *reinterpret_cast<u32x4*>(&A[a_index(p, q4)]) = r;
    }
  };

  // ---- weight fragments: block kb is [wave][nt][g][col][e] in the packed
  // layout, channel 16*wave + 4g + e, column 16*nt + col; lane (col, g) of
  // wave w reads its NT 16-byte pieces, one coalesced 1 KB run per nt.
  const int rl = lane & 15;
  const int g = lane >> 4;
  f32x4 bw[2][NT];
  auto b_src = [&](int kb) {
    return wblocks + (size_t)kb * (CB * NO) + (size_t)wave * (NT * 256) + (g * 16 + rl) * 4;
  };

  // ---- (c) MFMA: k-slot g of step e is channel 16*wave + 4g + e, on both sides
  f32x4 acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- prologue: coefficients of taps 0 and 1, registers for the tap the
  // first step turns into coefficients, weight and column tile of block 0
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  const int k1 = a.K > 1 ? 1 : 0;
  coef_load(0, S0{});
  coef_finish(0, S0{});
  coef_load(k1, S1{});
  coef_finish(k1, S1{});
  {
    const int t = 2 / a.nchunk;
    coef_load(t < a.K ? t : a.K - 1, S0{});
  }
  {
    const float* src = b_src(0);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) bw[0][nt] = *reinterpret_cast<const f32x4*>(src + nt * 256);
  }
  gather_offsets(0);
#pragma unroll
  for (int ps = 0; ps < NPASS; ++ps)
#pragma unroll
    for (int c = 0; c < 4; ++c) gv[ps][c] = load16(xr, goff[ps][c]);
  finish_gather(0, 0);

  // One step = block kb's MFMAs with the loads for later blocks threaded
  // through them: the texture-address queue is shared by all waves of a CU,
  // and a burst of loads would stall the wave at issue, before its MFMAs.
  // Load order: corners of kb+1 (needed at the end of this step), weight
  // fragments of kb+1 (next step), offsets/mask of a tap three steps ahead
  // (turned into coefficients next step); one load after every second MFMA.
  constexpr int NG = NPASS * 4;       // corner loads
  constexpr int NLOAD = NG + NT + 3;  // + weight fragments + dy, dx, mask
  constexpr int NMFMA = 4 * MT * NT;
  static_assert(2 * NLOAD <= NMFMA, "every load rides behind two MFMAs");
  auto step = [&](int kb, auto par) {
    constexpr int P = decltype(par)::value;  // kb & 1
    using SP = std::integral_constant<int, P>;
    const int kn = kb + 1 < NKB ? kb + 1 : NKB - 1;
    const int tl = (kb + 3) / a.nchunk;
    const int tload = tl < a.K ? tl : a.K - 1;
    gather_offsets(kn);
    const float* bsrc = b_src(kn);
    const uint32_t c_hw = (uint32_t)(hw0 + lane);
    const uint32_t c_ob = ((uint32_t)(b * 2 * a.K + 2 * tload) * (uint32_t)a.HoWo + c_hw) * 4;
    const uint32_t c_mb = ((uint32_t)(b * a.K + tload) * (uint32_t)a.HoWo + c_hw) * 4;
    const float* A = As + (wave * 2 + P) * A_FLOATS;
    f32x4 af[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      af[mt] = *reinterpret_cast<const f32x4*>(&A[a_index(mt * 16 + rl, g)]);
    __builtin_amdgcn_sched_barrier(0);
    static_for<NMFMA>([&](auto I) {
      constexpr int idx = decltype(I)::value;
      constexpr int e = idx / (MT * NT), mt = (idx / NT) % MT, nt = idx % NT;
      acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[mt][e], bw[P][nt][e], acc[mt][nt], 0,
                                                         0, 0);
      if constexpr (idx % 2 == 1 && idx / 2 < NLOAD) {
        constexpr int L = idx / 2;
        if constexpr (L < NG) {
          gv[L / 4][L % 4] = load16(xr, goff[L / 4][L % 4]);
        } else if constexpr (L < NG + NT) {
          bw[P ^ 1][L - NG] = *reinterpret_cast<const f32x4*>(bsrc + (L - NG) * 256);
        } else if constexpr (L == NG + NT) {
          c_dy[P ^ 1] = load_scalar<float>(offr, c_ob);
        } else if constexpr (L == NG + NT + 1) {
          c_dx[P ^ 1] = load_scalar<float>(offr, c_ob + (uint32_t)a.HoWo * 4);
        } else {
          c_mk[P ^ 1] = load_scalar<float>(mskr, c_mb);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    const int tc = (kb + 2) / a.nchunk;
    if (tc * a.nchunk == kb + 2 && tc < a.K) coef_finish(tc, SP{});
    finish_gather(kn, P ^ 1);
  };
  int kb = 0;
  for (; kb + 1 < NKB; kb += 2) {
    step(kb, S0{});
    step(kb + 1, S1{});
  }
  if (kb < NKB) step(kb, S0{});

  // ---- epilogue: sum the four waves' partial tiles through LDS, + bias, store
  __syncthreads();  // every wave is done with the column tiles and coefficients
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      *reinterpret_cast<f32x4*>(&red[(wave * NO + nt * 16 + rl) * RST + mt * 16 + g * 4]) =
          acc[mt][nt];
  __syncthreads();
  if constexpr (!NHWC) {
    constexpr int PER = M / 4;  // float4 runs per output channel
    for (int e = tid; e < NO * PER; e += 256) {
      const int col = e / PER;
      const int r4 = e - col * PER;
      const int o = otile * NO + col;
      if (o >= a.O) continue;
      f32x4 v = *reinterpret_cast<const f32x4*>(&red[col * RST + r4 * 4]);
#pragma unroll
      for (int w = 1; w < 4; ++w) v += *reinterpret_cast<const f32x4*>(&red[(w * NO + col) * RST + r4 * 4]);
      v += a.bias ? static_cast<const float*>(a.bias)[o] : 0.0f;
      const int hw = hw0 + r4 * 4;
      float* dst = a.out + ((size_t)b * a.O + o) * a.HoWo + hw;
      if (a.vec_store && hw + 3 < a.HoWo) {
        *reinterpret_cast<f32x4*>(dst) = v;
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (hw + r < a.HoWo) dst[r] = v[r];
      }
    }
  } else {
    for (int e = tid; e < NO * M; e += 256) {
      const int col = e % NO;
      const int row = e / NO;
      const int o = otile * NO + col;
      const int hw = hw0 + row;
      if (o >= a.O || hw >= a.HoWo) continue;
      float v = red[col * RST + row];
#pragma unroll
      for (int w = 1; w < 4; ++w) v += red[(w * NO + col) * RST + row];
      v += a.bias ? static_cast<const float*>(a.bias)[o] : 0.0f;
      a.out[((size_t)b * a.HoWo + hw) * a.O + o] = v;
    }
  }
}

namespace {
template <int M, int NO, bool NHWC>
hipError_t launch_wsk_variant(const KernelConfig& kc, const FusedArgs& a, hipStream_t s) {
  const int64_t nblk = (int64_t)a.B * kc.tiles_per_img * kc.n_otiles;
  if (nblk <= 0) return hipSuccess;
  if (nblk > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fused_wsk_kernel<M, NO, NHWC>), dim3((unsigned)nblk), dim3(256), 0, s, a);
  return hipGetLastError();
}
}  // namespace

bool wsk_supported(const KernelConfig& kc) {
  return !kc.bf16 && kc.CB == 64 && ((kc.NO == 64 && kc.M == 64) || (kc.NO == 128 && kc.M == 32));
}

hipError_t launch_fused_wsk(const KernelConfig& kc, const FusedArgs& a, hipStream_t s) {
  if (kc.NO == 64 && kc.M == 64)
    return kc.nhwc ? launch_wsk_variant<64, 64, true>(kc, a, s)
                   : launch_wsk_variant<64, 64, false>(kc, a, s);
  if (kc.NO == 128 && kc.M == 32)
    return kc.nhwc ? launch_wsk_variant<32, 128, true>(kc, a, s)
                   : launch_wsk_variant<32, 128, false>(kc, a, s);
  return hipErrorInvalidValue;
}

}  // namespace dcn
