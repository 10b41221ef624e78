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

template <int M, int NO, bool NHWC, class Src>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void
fused_wsk_kernel(Src src) {
  int logical;
  const FusedArgs& a = resolve_args(src, logical);
  constexpr int CB = 64;          // channels per k-block
  constexpr int MT = M / 16;      // row groups = gather passes (16 pixels x 4 quads each)
  constexpr int NT = NO / 16;
  constexpr int NSLOT = 3;        // coefficient ring: taps whose tables are live at once
  constexpr int A_FLOATS = M * 16;                       // one wave's column tile
  constexpr int MAIN_BYTES = 4 * A_FLOATS * 4 + 4 * NSLOT * M * 32;
  constexpr int RST = M + 4;                             // reduction row stride
  constexpr int RED_BYTES = 4 * NO * RST * 4;
  constexpr int SMEM = MAIN_BYTES > RED_BYTES ? MAIN_BYTES : RED_BYTES;
  static_assert(M == 32 || M == 64, "tile rows");
  static_assert(NO % 16 == 0, "tile columns");

  __shared__ __attribute__((aligned(16))) char smem[SMEM];
  float* const As = reinterpret_cast<float*>(smem);                          // [w][M][16]
  f32x4* const Cw = reinterpret_cast<f32x4*>(smem + 4 * A_FLOATS * 4);       // [w][slot][M]
  u32x4* const Co = reinterpret_cast<u32x4*>(smem + 4 * A_FLOATS * 4 + 4 * NSLOT * M * 16);
  float* const red = reinterpret_cast<float*>(smem);                         // [w][NO][RST]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  const int otile = logical % a.n_otiles;
  const int t2 = logical / a.n_otiles;
  const int tile = t2 % a.tiles_per_img;
  const int b = t2 / a.tiles_per_img;
  const int hw0 = tile * M;
  const int NKB = a.K * a.nchunk;

  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, a.x_bytes);
  const bool has_mask = a.mask != nullptr;
  const __amdgpu_buffer_rsrc_t offr = make_rsrc(a.offset, a.offset_bytes);
  const __amdgpu_buffer_rsrc_t mskr =
      make_rsrc(has_mask ? a.mask : a.offset, has_mask ? a.mask_bytes : 0u);
  const float* wblocks = static_cast<const float*>(a.wpack) +
                         (size_t)otile * a.K * a.nchunk * (CB * NO);
  const uint32_t row_bytes = (uint32_t)a.C * 4;
  float* const Aw = As + wave * A_FLOATS;
  f32x4* const Cww = Cw + wave * NSLOT * M;
  u32x4* const Cow = Co + wave * NSLOT * M;

  // ---- (a) coefficients.  Lane m owns pixel m of the tile (all four
  // corners); the pixel's grid position is fixed, so it is computed once.
  const int c_hw = hw0 + lane;
  const bool c_in = c_hw < a.HoWo && lane < M;
  const int c_ho = c_hw / a.Wo;
  const int c_wo = c_hw - c_ho * a.Wo;
  float c_dy[2], c_dx[2], c_mk[2];
  auto coef_addr = [&](int kt, uint32_t& ob, uint32_t& mb) {
    ob = ((uint32_t)(b * 2 * a.K + 2 * kt) * (uint32_t)a.HoWo + (uint32_t)c_hw) * 4;
    mb = ((uint32_t)(b * a.K + kt) * (uint32_t)a.HoWo + (uint32_t)c_hw) * 4;
  };
  auto coef_finish = [&](int kt, auto set_tag) {
    constexpr int S = decltype(set_tag)::value;
    const int slot = kt % NSLOT;
    const int i = kt / a.kw;
    const int j = kt - i * a.kw;
    const TapCorners t = tap_corners((float)(c_ho - a.ph + i), (float)(c_wo - a.pw + j), c_dy[S],
                                     c_dx[S], a.H, a.W);
    const float mk = has_mask ? c_mk[S] : 1.0f;
    const float hy = 1.0f - t.p.ly, hx = 1.0f - t.p.lx;
    const float wv[4] = {hy * hx, hy * t.p.lx, t.p.ly * hx, t.p.ly * t.p.lx};
    const uint32_t base = (uint32_t)((b * a.H + t.y0) * a.W + t.x0) * row_bytes;
    f32x4 w4;
    u32x4 o4;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const bool ok = c_in && ((t.valid >> c) & 1u);
      w4[c] = ok ? wv[c] * mk : 0.0f;
      o4[c] = ok ? base + (uint32_t)((c >> 1) * a.W + (c & 1)) * row_bytes : kNoCorner;
    }
    if (a.dbg_corner != nullptr && c_in) {
      const size_t e = (((size_t)b * a.K + kt) * a.HoWo + c_hw) * 4;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        a.dbg_corner[e + c] = o4[c] == kNoCorner ? -1 : (int32_t)(o4[c] / row_bytes);
        a.dbg_weight[e + c] = w4[c];
      }
    }
    if (lane < M) {
      Cww[slot * M + lane] = w4;
      Cow[slot * M + lane] = o4;
    }
  };
  auto coef_now = [&](int kt, auto set_tag) {  // prologue: load and finish at once
    constexpr int S = decltype(set_tag)::value;
    uint32_t ob, mb;
    coef_addr(kt, ob, mb);
    c_dy[S] = load_scalar<float>(offr, ob);
    c_dx[S] = load_scalar<float>(offr, ob + (uint32_t)a.HoWo * 4);
    c_mk[S] = load_scalar<float>(mskr, mb);
    coef_finish(kt, set_tag);
  };

  // ---- (b) corners: lane = (pixel pp of a pass, channel quad q4 of the
  // wave's 16).  gv[p] holds pass p's four corners of one block.
  const int pp = lane >> 2;
  const int q4 = lane & 3;
  u32x4 gv[MT][4];
  // Byte offset of this lane's channel quad inside a corner's channel vector
  // for block kb, and whether that quad exists (C need not fill the block).
  auto gather_base = [&](int kb, uint32_t& cbyte, bool& chan_ok) {
    const int kt = kb / a.nchunk;
    const int ch = (kb - kt * a.nchunk) * CB + wave * 16 + q4 * 4;
    chan_ok = ch < a.C;
    cbyte = (uint32_t)ch * 4;
    return kt % NSLOT;
  };
  // Column tile row p holds the wave's 16 channels as 4 quads; quad q sits at
  // position q ^ ((p >> 2) & 3) so that both the blend writes (16 lanes = 4
  // pixels x 4 quads) and the MFMA reads (16 lanes = 16 pixels, one quad) hit
  // 64 distinct banks.
  auto a_index = [](int p, int q) { return p * 16 + ((q ^ ((p >> 2) & 3)) << 2); };

  // ---- weight fragments: block kb is [wave][nt][g][col][e] in the packed
  // layout (channel 16*wave + 4g + e, column 16*nt + col); lane (col, g)
  // reads NT 16-byte pieces, one coalesced 1 KB run per nt.
  const int rl = lane & 15;
  const int g = lane >> 4;
  f32x4 bw[2][NT];
  auto b_src = [&](int kb) {
    return wblocks + (size_t)kb * (CB * NO) + (size_t)wave * (NT * 256) + (g * 16 + rl) * 4;
  };

  // ---- (c) MFMA: k-slot g of step e is channel 16*wave + 4g + e, on both
  // sides; row group mt uses column-tile rows [16 mt, 16 mt + 16).
  f32x4 acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 af[MT];

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  auto clampb = [&](int kb) { return kb < NKB ? kb : NKB - 1; };
  auto clampt = [&](int kt) { return kt < a.K ? kt : a.K - 1; };

  // ---- prologue: coefficient tables of taps 0..2, offsets of the tap the
  // first step finishes, weights of block 0, all corners of block 0, pass 0
  // blended, pass 0 of block 1 in flight.
  coef_now(0, S0{});
  coef_now(clampt(1), S0{});
  coef_now(clampt(2), S0{});
  {
    uint32_t ob, mb;
    coef_addr(clampt(3 / a.nchunk), ob, mb);
    c_dy[0] = load_scalar<float>(offr, ob);
    c_dx[0] = load_scalar<float>(offr, ob + (uint32_t)a.HoWo * 4);
    c_mk[0] = load_scalar<float>(mskr, mb);
  }
  {
    const float* src = b_src(0);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) bw[0][nt] = *reinterpret_cast<const f32x4*>(src + nt * 256);
  }
  {
    uint32_t cb0;
    bool ok0;
    const int sl0 = gather_base(0, cb0, ok0);
#pragma unroll
    for (int p = 0; p < MT; ++p) {
      const u32x4 off = Cow[sl0 * M + p * 16 + pp];
#pragma unroll
      for (int c = 0; c < 4; ++c) gv[p][c] = load16(xr, ok0 ? off[c] + cb0 : kNoCorner);
    }
    const f32x4 w = Cww[sl0 * M + pp];
    *reinterpret_cast<u32x4*>(&Aw[a_index(pp, q4)]) =
        Ops<float>::blend(w, gv[0][0], gv[0][1], gv[0][2], gv[0][3]);
    uint32_t cb1;
    bool ok1;
    const int sl1 = gather_base(clampb(1), cb1, ok1);
    const u32x4 off = Cow[sl1 * M + pp];
#pragma unroll
    for (int c = 0; c < 4; ++c) gv[0][c] = load16(xr, ok1 ? off[c] + cb1 : kNoCorner);
    af[0] = *reinterpret_cast<const f32x4*>(&Aw[a_index(rl, g)]);
  }

  // ---- one step = the MFMAs of block s, row group by row group.  Under the
  // MFMAs of row group q run: the blend of pass q+1 of block s (pass 0 of
  // block s+1 under the last group), the corner loads of the block after that
  // pass's block into the registers the blend just freed (one full step
  // before they are blended), the column-tile read for the next row group;
  // in group 0 the weight fragments of block s+1 and the offsets/mask of a
  // tap four steps ahead; in the last group the coefficient table of tap
  // (s+3)/nchunk (from offsets loaded one step earlier).  Each item is pinned
  // after a given MFMA, so the matrix pipe never waits for a burst of other
  // work, and every load has a static position, so each wait is exact.
  constexpr int NMF = 4 * NT;  // MFMAs per row group
  auto step = [&](int s, auto par) {
    constexpr int P = decltype(par)::value;  // s & 1: weight / offset register sets
    using SP = std::integral_constant<int, P>;
    const int tl = (s + 4) / a.nchunk;
    uint32_t c_ob, c_mb;
    coef_addr(clampt(tl), c_ob, c_mb);
    const float* bsrc = b_src(clampb(s + 1));
    static_for<MT>([&](auto Q) {
      constexpr int q = decltype(Q)::value;
      constexpr int p = (q + 1) % MT;           // pass blended under this group
      constexpr bool LAST = q + 1 == MT;
      const int blk = clampb(LAST ? s + 1 : s);  // block of that pass
      const int nblk = clampb(blk + 1);          // block whose pass-p corners load next
      uint32_t cb_b, cb_n;
      bool ok_b, ok_n;
      const int sl_b = gather_base(blk, cb_b, ok_b);
      const int sl_n = gather_base(nblk, cb_n, ok_n);
      (void)cb_b;
      (void)ok_b;
      f32x4 w;
      u32x4 off, r;
      constexpr int NACT = 12 + (q == 0 ? NT + 3 : 0) + (LAST ? 1 : 0);
      static_for<NMF>([&](auto J) {
        constexpr int j = decltype(J)::value;
        constexpr int e = j / NT, nt = j % NT;
        acc[q][nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[q][e], bw[P][nt][e], acc[q][nt], 0,
                                                          0, 0);
        static_for<NACT>([&](auto X) {
          constexpr int x = decltype(X)::value;
          if constexpr (x * NMF / NACT == j) {  // action x rides behind MFMA j
            if constexpr (x == 0) {
              w = Cww[sl_b * M + p * 16 + pp];
            } else if constexpr (x == 1) {
              off = Cow[sl_n * M + p * 16 + pp];
            } else if constexpr (x <= 5) {
              constexpr int c = x - 2;
              const f32x4 v = __builtin_bit_cast(f32x4, gv[p][c]);
              if constexpr (c == 0) {
                r = __builtin_bit_cast(u32x4, v * w[0]);
              } else {
                f32x4 t = __builtin_bit_cast(f32x4, r);
#pragma unroll
                for (int k = 0; k < 4; ++k) t[k] = __builtin_fmaf(w[c], v[k], t[k]);
                r = __builtin_bit_cast(u32x4, t);
              }
            } else if constexpr (x == 6) {
              *reinterpret_cast<u32x4*>(&Aw[a_index(p * 16 + pp, q4)]) = r;
            } else if constexpr (x == 7) {
              af[p] = *reinterpret_cast<const f32x4*>(&Aw[a_index(p * 16 + rl, g)]);
            } else if constexpr (x <= 11) {
              constexpr int c = x - 8;
              gv[p][c] = load16(xr, ok_n ? off[c] + cb_n : kNoCorner);
            } else if constexpr (q == 0 && x < 12 + NT) {
              bw[P ^ 1][x - 12] = *reinterpret_cast<const f32x4*>(bsrc + (x - 12) * 256);
            } else if constexpr (q == 0 && x == 12 + NT) {
              c_dy[P ^ 1] = load_scalar<float>(offr, c_ob);
            } else if constexpr (q == 0 && x == 13 + NT) {
              c_dx[P ^ 1] = load_scalar<float>(offr, c_ob + (uint32_t)a.HoWo * 4);
            } else if constexpr (q == 0 && x == 14 + NT) {
              c_mk[P ^ 1] = load_scalar<float>(mskr, c_mb);
            } else if constexpr (LAST) {
              const int tc = (s + 3) / a.nchunk;
              if (tc * a.nchunk == s + 3 && tc < a.K) coef_finish(tc, SP{});
            }
          }
        });
        __builtin_amdgcn_sched_barrier(0);
      });
    });
  };
  int s = 0;
  for (; s + 1 < NKB; s += 2) {
    step(s, S0{});
    step(s + 1, S1{});
  }
  if (s < NKB) step(s, S0{});

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
template <int M, int NO, bool NHWC, class Src>
hipError_t launch_wsk_variant(const Src& src, int64_t nblk, hipStream_t s) {
  if (nblk <= 0) return hipSuccess;
  if (nblk > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fused_wsk_kernel<M, NO, NHWC, Src>), dim3((unsigned)nblk), dim3(256), 0, s,
                     src);
  return hipGetLastError();
}

template <class Src>
hipError_t launch_wsk_src(const KernelConfig& kc, const Src& src, int64_t nblk, hipStream_t s) {
  if (kc.NO == 64 && kc.M == 64)
    return kc.nhwc ? launch_wsk_variant<64, 64, true>(src, nblk, s)
                   : launch_wsk_variant<64, 64, false>(src, nblk, s);
  if (kc.NO == 128 && kc.M == 32)
    return kc.nhwc ? launch_wsk_variant<32, 128, true>(src, nblk, s)
                   : launch_wsk_variant<32, 128, false>(src, nblk, s);
  return hipErrorInvalidValue;
}
}  // namespace

bool wsk_supported(const KernelConfig& kc) {
  return !kc.bf16 && kc.CB == 64 && ((kc.NO == 64 && kc.M == 64) || (kc.NO == 128 && kc.M == 32));
}

hipError_t launch_fused_wsk(const KernelConfig& kc, const FusedArgs& a, hipStream_t s) {
  return launch_wsk_src(kc, a, (int64_t)a.B * kc.tiles_per_img * kc.n_otiles, s);
}

hipError_t launch_fused_wsk_multi(const KernelConfig& kc, const MultiArgs& m, hipStream_t s) {
  return launch_wsk_src(kc, m, m.start[m.n], s);
}

}  // namespace dcn
