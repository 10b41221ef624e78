// dcn_bf16.hip -- bf16 fused DCNv2 forward for wide outputs (256 output
// channels per workgroup).
//
// Same operator as the other kernels (page 1, "deform_conv.py": sample the
// input bilinearly at (h - pad + i + dy, w - pad + j + dx), corners outside
// count as zero, times the mask, contract over (tap, channel) with the
// weight, + bias), here for bf16 operands with fp32 accumulation (page 5,
// deformops README: accumulation in float32 for every operand dtype).
//
// Shape of the work: at 256 output channels the texture-address unit, the
// LDS and the vector ALUs all carry more per MFMA than in the fp32 kernels.
// One workgroup of 4 waves (one per SIMD) owns 128 output pixels x 256 output
// channels -- the accumulators of a whole CU, in AGPRs -- so each weight is
// fetched once per 128 pixels.  Wave w owns output channels [64w, 64w + 64)
// of all 128 pixels and fetches exactly its own weight fragments straight
// from memory (L2) into registers, so weights never pass through LDS; LDS
// holds only the double-buffered column tile and the corner tables.  A
// k-block is one tap x CB channels (CB up to 256: one barrier per tap).
//
// The blend multiplies bf16 pairs: the corner weight (bilinear x validity x
// mask, formed in fp32) is rounded once to bf16, and the bf16 pair dot
// product with (w, 0) / (0, w) scales the low / high channel of each loaded
// dword into an fp32 accumulator -- one instruction per channel and corner
// instead of a widening plus an FMA.  The blended sample is rounded once to
// bf16 for the column tile.
//
// Per k-block step s (one barrier): the MFMAs of block s are interleaved
// one-for-one with the blend of block s+1 into the idle column buffer.  The
// blend walks CB/16 passes (32 pixels x 64 channels each); the corner loads
// run up to four passes ahead of it, across the step boundary, and the weight
// fragments two k-steps ahead of the MFMAs.  Once per tap the corner table of
// tap (s+3)/nchunk is formed from offsets loaded at the top of the step.

#include <type_traits>

#include "dcn_device.h"
#include "dcn_launch.h"

namespace dcn {

template <int CB, bool NHWC, bool FULLC, class Src>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void
fused_bf16_kernel(Src src) {
  int logical;
  const FusedArgs& a = resolve_args(src, logical);
  constexpr int M = 128;              // output pixels per workgroup
  constexpr int NO = 256;             // output channels per workgroup
  constexpr int NQ = CB / 32;         // MFMA k-steps per block
  constexpr int MT = M / 16;          // 16-row tiles
  constexpr int NTW = 4;              // 16-column tiles per wave
  constexpr int ROWB = CB * 2;        // column-tile row bytes
  constexpr int A_BYTES = M * ROWB;
  constexpr int NCK = CB / 64;        // 64-channel chunks per block
  constexpr int NP = 4 * NCK;         // blend passes per block (32 pixels x 64 channels)
  constexpr int NSL = NQ * MT * NTW;  // MFMA slots per block
  constexpr int SPP = NSL / NP;       // slots per pass
  constexpr int NSLOT = 3;            // corner-table ring
  static_assert(SPP == 16, "one blend unit per MFMA slot");
  constexpr int LAG = NP >= 8 ? 4 : 2;  // corner loads run LAG passes ahead of the blend
  static_assert(NP % LAG == 0, "corner registers rotate over LAG passes");

  __shared__ __attribute__((aligned(16))) char As[2][A_BYTES];
  __shared__ f32x4 Cw[NSLOT][M];  // corner weights (bilinear x validity x mask), bf16-rounded
  __shared__ u32x4 Co[NSLOT][M];  // corner byte offsets in x (kNoCorner: outside)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  const int otile = logical % a.n_otiles;
  const int t2 = logical / a.n_otiles;
  const int tile = t2 % a.tiles_per_img;
  const int b = t2 / a.tiles_per_img;
  const int hw0 = tile * M;
  const int NKB = a.K * a.nchunk;
  auto clampb = [&](int kb) { return kb < NKB ? kb : NKB - 1; };
  auto clampt = [&](int kt) { return kt < a.K ? kt : a.K - 1; };

  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, a.x_bytes);
  const bool has_mask = a.mask != nullptr;
  const __amdgpu_buffer_rsrc_t offr = make_rsrc(a.offset, a.offset_bytes);
  const __amdgpu_buffer_rsrc_t mskr =
      make_rsrc(has_mask ? a.mask : a.offset, has_mask ? a.mask_bytes : 0u);
  // this wave's weight fragments: block kb, k-step q, tile k' at
  // wfrag + (kb * NQ + q) * 16 * 64 + k' * 64 (u32x4 units)
  const u32x4* wfrag = reinterpret_cast<const u32x4*>(
                           static_cast<const __bf16*>(a.wpack) +
                           (size_t)otile * a.K * a.nchunk * (CB * NO)) +
                       wave * NTW * 64 + lane;
  const uint32_t row_bytes = (uint32_t)a.C * 2;

  // ---- (a) corner table: thread -> pixel tid & 127, corner row a = tid >> 7
  // (corners (a, 0), (a, 1)).  Offsets and mask are bf16, widened exactly.
  const int c_px = tid & (M - 1);
  const int c_pair = tid >> 7;
  const int c_hw = hw0 + c_px;
  const bool c_in = c_hw < a.HoWo;
  const int c_ho = c_hw / a.Wo;
  const int c_wo = c_hw - c_ho * a.Wo;
  float c_dy, c_dx, c_mk;
  auto coef_load = [&](int kt) {
    const uint32_t ob = ((uint32_t)(b * 2 * a.K + 2 * kt) * (uint32_t)a.HoWo + (uint32_t)c_hw) * 2;
    const uint32_t mb = ((uint32_t)(b * a.K + kt) * (uint32_t)a.HoWo + (uint32_t)c_hw) * 2;
    c_dy = load_scalar<__bf16>(offr, ob);
    c_dx = load_scalar<__bf16>(offr, ob + (uint32_t)a.HoWo * 2);
    c_mk = load_scalar<__bf16>(mskr, mb);
  };
  auto coef_finish = [&](int kt) {
    const int slot = kt % NSLOT;
    const int i = kt / a.kw;
    const int j = kt - i * a.kw;
    const SamplePoint p =
        sample_point((float)(c_ho - a.ph + i), (float)(c_wo - a.pw + j), c_dy, c_dx);
    const CornerRow cr = corner_row(p, c_pair, a.H, a.W);
    const float mk = has_mask ? c_mk : 1.0f;
    const float wy = c_pair ? p.ly : 1.0f - p.ly;
    const uint32_t base = (uint32_t)((b * a.H + cr.ry) * a.W + cr.ix) * row_bytes;
    const bool ok0 = c_in && cr.ok0;
    const bool ok1 = c_in && cr.ok1;
    const float w0 = static_cast<float>(static_cast<__bf16>(wy * (1.0f - p.lx) * mk));
    const float w1 = static_cast<float>(static_cast<__bf16>(wy * p.lx * mk));
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const f32x2 w2 = {ok0 ? w0 : 0.0f, ok1 ? w1 : 0.0f};
    const u32x2 o2 = {ok0 ? base : kNoCorner, ok1 ? base + row_bytes : kNoCorner};
    if (a.dbg_corner != nullptr && c_in) {
      const size_t e = (((size_t)b * a.K + kt) * a.HoWo + c_hw) * 4 + 2 * c_pair;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        a.dbg_corner[e + q] = o2[q] == kNoCorner ? -1 : (int32_t)(o2[q] / row_bytes);
        a.dbg_weight[e + q] = w2[q];
      }
    }
    *reinterpret_cast<f32x2*>(reinterpret_cast<float*>(&Cw[slot][c_px]) + 2 * c_pair) = w2;
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint32_t*>(&Co[slot][c_px]) + 2 * c_pair) = o2;
  };

  // ---- (b) corners.  Pass pi of a block: pixel group pg = pi / NCK (32
  // pixels), chunk ck = pi % NCK (64 channels); thread -> pixel 32 pg + pp,
  // 16-byte slice ck * 8 + sl.  Eight lanes cover one corner's 128-byte run.
  const int sl = tid & 7;
  const int pp = tid >> 3;
  u32x4 gv[LAG][4];  // corner vectors of LAG consecutive passes
  auto cbyte_of = [&](int kb, int ck, bool& ok) {
    const int kt = kb / a.nchunk;
    const int ch = (kb - kt * a.nchunk) * CB + ck * 64 + sl * 8;
    ok = FULLC || ch < a.C;
    return (uint32_t)ch * 2;
  };
  auto slot_of = [&](int kb) { return (kb / a.nchunk) % NSLOT; };
  // Column tile: row r (pixel), 16-byte chunk k (channels 8k .. 8k+7) at
  // r * ROWB + 16 * (k ^ x(r)); the XOR spreads both the eight-lane row writes
  // and the sixteen-row fragment reads over all banks.
  auto a_off = [](int r, int k) {
    if constexpr (ROWB == 128) return r * 128 + 16 * (k ^ ((r >> 1) & 7));
    else return r * ROWB + 16 * (k ^ (((r & 1) << 3) | ((r >> 1) & 7)));
  };

  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  auto dot2 = [](uint32_t v, uint32_t w, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, v),
                                          __builtin_bit_cast(bf16x2, w), acc, false);
  };

  // ---- (c) MFMA.  k-step q of a block covers its channels [32q, 32q + 32);
  // lane group g (lane / 16) supplies channels 32q + 8g + e.  Weight block
  // layout [q][16 column tiles][64 lanes][8].
  const int rl = lane & 15;
  const int g = lane >> 4;
  f32x4 acc[MT][NTW];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  u32x4 af[3];        // column-tile fragments, sequence u = 8q + mt
  u32x4 bw[4][NTW];   // weight fragments, ring over the global k-step index
  auto a_frag = [&](const char* A, int u) {
    const int q = u / MT, mt = u % MT;
    return *reinterpret_cast<const u32x4*>(A + a_off(mt * 16 + rl, 4 * q + g));
  };
  auto b_load = [&](int kb, int q, int k) { return wfrag[((size_t)kb * NQ + q) * 1024 + k * 64]; };

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;

  // ---- prologue: corner tables of taps 0..2; block 0 blended into As[0];
  // the corner loads of block 1 passes 0 .. LAG-1 and the weights of block 0
  // k-steps 0, 1 in flight.
#pragma unroll
  for (int t = 0; t < 3; ++t) {
    coef_load(clampt(t));
    coef_finish(clampt(t));
  }
  __syncthreads();
  {
#pragma unroll
    for (int q = 0; q < 2 && q < NQ; ++q)
#pragma unroll
      for (int k = 0; k < NTW; ++k) bw[q][k] = b_load(0, q, k);
    const int s0 = slot_of(0);
    for (int pi = 0; pi < NP; ++pi) {
      const int pg = pi / NCK, ck = pi % NCK;
      bool ok;
      const uint32_t cb = cbyte_of(0, ck, ok);
      const u32x4 off = Co[s0][32 * pg + pp];
      u32x4 v[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) v[c] = load16(xr, ok ? off[c] + cb : kNoCorner);
      const u32x4 w = __builtin_bit_cast(u32x4, Cw[s0][32 * pg + pp]);
      float r[8];
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          r[2 * d] = dot2(v[c][d], w[c] >> 16, c == 0 ? 0.0f : r[2 * d]);
          r[2 * d + 1] = dot2(v[c][d], w[c], c == 0 ? 0.0f : r[2 * d + 1]);
        }
      bf16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = static_cast<__bf16>(r[e]);
      *reinterpret_cast<u32x4*>(&As[0][a_off(32 * pg + pp, ck * 8 + sl)]) =
          __builtin_bit_cast(u32x4, o);
    }
#pragma unroll
    for (int f = 0; f < LAG; ++f) {  // flattened pass f after block 0
      const int kb = clampb(1 + f / NP), pi = f % NP;
      const int pg = pi / NCK, ck = pi % NCK;
      bool ok;
      const uint32_t cb = cbyte_of(kb, ck, ok);
      const u32x4 off = Co[slot_of(kb)][32 * pg + pp];
#pragma unroll
      for (int c = 0; c < 4; ++c) gv[f][c] = load16(xr, ok ? off[c] + cb : kNoCorner);
    }
  }
  // Corner-table entries in registers, by pixel-group parity: blend weights
  // of block s+1, load offsets of the pass the loads reach.
  u32x4 wt[2], ot[2];

  // ---- one step s.  Slot j (0..NSL-1) holds MFMA (q, mt, nt) = (j / 32,
  // (j / 4) % 8, j % 4) and, pinned beside it:
  //   * blend unit (pass j / 16, corner (j / 4) % 4, dword j % 4) of block
  //     s+1: two pair dot products; after a corner's last unit, that
  //     corner's load for the pass LAG ahead (block s+1, or s+2 at the end);
  //     after a pass's last unit, the bf16 rounding and the column-tile write;
  //   * at the first slot of a 16-row tile: the column-tile fragment two
  //     tiles ahead; at slots 4k of k-step q: weight fragment k of k-step
  //     q+2 (next block past the end);
  //   * corner-table entries of the pixel group the blend / the loads reach
  //     next, read one pass ahead.
  auto step = [&](int s, auto par) {
    constexpr int P = decltype(par)::value;  // s & 1: column buffers, weight ring
    const int n1 = clampb(s + 1), n2 = clampb(s + 2);
    const int sl_1 = slot_of(n1), sl_2 = slot_of(n2);
    const int tc = (s + 3) / a.nchunk;
    const bool coef_due = tc * a.nchunk == s + 3 && tc < a.K;
    const char* A = As[P];
    char* An = As[P ^ 1];

    __syncthreads();  // block s in As[P]; every wave done with block s-1
    coef_load(clampt(tc));
    af[0] = a_frag(A, 0);
    af[1] = a_frag(A, 1);
    wt[0] = __builtin_bit_cast(u32x4, Cw[sl_1][pp]);
    float r[8];
    __builtin_amdgcn_sched_barrier(0);

    static_for<NSL>([&](auto J) {
      constexpr int j = decltype(J)::value;
      constexpr int q = j / 32, mt = (j / 4) % MT, nt = j % 4;
      constexpr int u = q * MT + mt;
      constexpr int gq = P * NQ + q;  // global k-step index mod 4 (NQ even or P-split)
      acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          __builtin_bit_cast(bf16x8, af[u % 3]), __builtin_bit_cast(bf16x8, bw[gq % 4][nt]),
          acc[mt][nt], 0, 0, 0);
      if constexpr (nt == 0 && u + 2 < NQ * MT) af[(u + 2) % 3] = a_frag(A, u + 2);
      if constexpr (mt == 0) {
        // weight fragment nt of k-step q+2
        if constexpr (q + 2 < NQ) bw[(gq + 2) % 4][nt] = b_load(s, q + 2, nt);
        else bw[(gq + 2) % 4][nt] = b_load(n1, q + 2 - NQ, nt);
      }
      constexpr int pi = j / SPP, c = (j / 4) % 4, d = j % 4;
      constexpr int pg = pi / NCK, ck = pi % NCK;
      {
        const uint32_t wh = wt[pg & 1][c];
        const uint32_t v = gv[pi % LAG][c][d];
        r[2 * d] = dot2(v, wh >> 16, c == 0 ? 0.0f : r[2 * d]);
        r[2 * d + 1] = dot2(v, wh, c == 0 ? 0.0f : r[2 * d + 1]);
      }
      if constexpr (d == 3) {
        // corner c of pass pi consumed: load it for pass pi + LAG
        constexpr int pn = pi + LAG < NP ? pi + LAG : pi + LAG - NP;
        constexpr int pgn = pn / NCK, ckn = pn % NCK;
        bool ok;
        const uint32_t cb = cbyte_of(pi + LAG < NP ? n1 : n2, ckn, ok);
        gv[pi % LAG][c] = load16(xr, ok ? ot[pgn & 1][c] + cb : kNoCorner);
      }
      if constexpr (c == 3 && d == 3) {
        bf16x8 o;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = static_cast<__bf16>(r[e]);
        *reinterpret_cast<u32x4*>(&An[a_off(32 * pg + pp, ck * 8 + sl)]) =
            __builtin_bit_cast(u32x4, o);
      }
      // table entries one pass ahead: blend weights of pass pi+1, load
      // offsets of pass pi+LAG+1 (block s+2 past the end)
      if constexpr (c == 2 && d == 0 && pi + 1 < NP && (pi + 1) % NCK == 0)
        wt[((pi + 1) / NCK) & 1] = __builtin_bit_cast(u32x4, Cw[sl_1][32 * ((pi + 1) / NCK) + pp]);
      if constexpr (c == 2 && d == 1) {
        constexpr int p3 = pi + LAG + 1 < NP ? pi + LAG + 1 : pi + LAG + 1 - NP;
        if constexpr (p3 % NCK == 0)
          ot[(p3 / NCK) & 1] = Co[pi + LAG + 1 < NP ? sl_1 : sl_2][32 * (p3 / NCK) + pp];
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    if (coef_due) coef_finish(tc);
  };
  // The loop's first loads are flattened pass LAG after block 0: its table
  // entry, as the previous step would have left it.
  {
    constexpr int fp = LAG % NP;
    ot[(fp / NCK) & 1] = Co[slot_of(clampb(1 + LAG / NP))][32 * (fp / NCK) + pp];
  }
  int s = 0;
  for (; s + 1 < NKB; s += 2) {
    step(s, S0{});
    step(s + 1, S1{});
  }
  if (s < NKB) step(s, S0{});

  // ---- epilogue: + bias, fp32 store straight from the accumulators.
  // MFMA 16x16 result layout: lane l, register r -> row 4(l/16) + r,
  // column l % 16.
  const __bf16* biasp = static_cast<const __bf16*>(a.bias);
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    const int o = otile * NO + wave * 64 + nt * 16 + rl;
    if (o >= a.O) continue;
    const float bo = biasp ? static_cast<float>(biasp[o]) : 0.0f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int hw = hw0 + mt * 16 + 4 * g;
      const f32x4 v = acc[mt][nt] + bo;
      if constexpr (!NHWC) {
        float* dst = a.out + ((size_t)b * a.O + o) * a.HoWo + hw;
        if (a.vec_store && hw + 3 < a.HoWo) {
          *reinterpret_cast<f32x4*>(dst) = v;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (hw + e < a.HoWo) dst[e] = v[e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (hw + e < a.HoWo) a.out[((size_t)b * a.HoWo + hw + e) * a.O + o] = v[e];
      }
    }
  }
}

bool bf16w_supported(const KernelConfig& kc) {
  return kc.bf16 && (kc.CB == 64 || kc.CB == 128 || kc.CB == 256) && kc.NO == 256 &&
         kc.M == 128;
}

namespace {
template <int CB, class Src>
hipError_t launch_cb_bf16w(const Src& src, int C, bool nhwc, dim3 grid, hipStream_t s) {
  const bool fullc = C % CB == 0;
  const dim3 block(256);
  if (nhwc) {
    if (fullc) hipLaunchKernelGGL((fused_bf16_kernel<CB, true, true, Src>), grid, block, 0, s, src);
    else hipLaunchKernelGGL((fused_bf16_kernel<CB, true, false, Src>), grid, block, 0, s, src);
  } else {
    if (fullc) hipLaunchKernelGGL((fused_bf16_kernel<CB, false, true, Src>), grid, block, 0, s, src);
    else hipLaunchKernelGGL((fused_bf16_kernel<CB, false, false, Src>), grid, block, 0, s, src);
  }
  return hipGetLastError();
}

template <class Src>
hipError_t launch_bf16w_src(const KernelConfig& kc, const Src& src, int C, int64_t nblk,
                            hipStream_t s) {
  if (nblk <= 0) return hipSuccess;
  if (nblk > 0x7fffffff || !bf16w_supported(kc)) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)nblk);
  switch (kc.CB) {
    case 64: return launch_cb_bf16w<64>(src, C, kc.nhwc, grid, s);
    case 128: return launch_cb_bf16w<128>(src, C, kc.nhwc, grid, s);
    default: return launch_cb_bf16w<256>(src, C, kc.nhwc, grid, s);
  }
}
}  // namespace

hipError_t launch_fused_bf16w(const KernelConfig& kc, const FusedArgs& a, hipStream_t s) {
  return launch_bf16w_src(kc, a, a.C, (int64_t)a.B * kc.tiles_per_img * kc.n_otiles, s);
}

hipError_t launch_fused_bf16w_multi(const KernelConfig& kc, const MultiArgs& m, hipStream_t s) {
  return launch_bf16w_src(kc, m, m.a[0].C, m.start[m.n], s);
}

}  // namespace dcn
