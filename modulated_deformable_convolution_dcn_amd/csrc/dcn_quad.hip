// dcn_quad.hip -- fp32 fused DCNv2 forward: each wave owns 32 pixels x 32
// channels of every k-block.
//
// Same operator as the other kernels (page 1, "deform_conv.py": sample the
// input bilinearly at (h - pad + i + dy, w - pad + j + dx), corners outside
// count as zero, times the mask, contract over (tap, channel) with the
// weight, + bias).  This kernel serves fp32 problems with up to 64 output
// channels -- the BiRefNet-decoder-like 64 -> 64, 7x7 shape.
//
// A workgroup is 4 waves = 64 consecutive output pixels x 64 output
// channels; every k-block is one tap x 64 input channels.  Wave (h, c) owns
// pixels [32h, 32h+32) and channels [32c, 32c+32) of each block:
//   * its corner loads are 8 lanes x 16 B = one 128-byte line per pixel
//     corner (as cheap for the texture-address unit as a full 256-byte
//     vector, half the cost of the 64-byte runs a 16-channel split needs);
//   * its column tile, coefficient table and weight fragments (loaded from
//     memory straight into registers in MFMA order) are private, so the
//     main loop has no workgroup barrier;
//   * it accumulates 32 x 64 partial outputs over its channel half; the two
//     halves are summed through LDS once at the end.
// The choice keeps the per-MFMA instruction mix small: on gfx950 every VALU
// op or LDS read issued beside the MFMAs costs matrix-pipe time, and this
// split needs 4 LDS fragment reads and 8 weight loads per 32x32x2 k-block
// of the wave (32 MFMAs of 2048 multiply-adds each).  The 32x32x2 fp32
// MFMA does the work of two 16x16x4 ones in one instruction: on this chip,
// with one VALU op per 1024 multiply-adds beside it, it takes about 9 % less
// time per multiply-add than the 16x16x4 form in isolation and 2 % less in
// this kernel on the 256 x 256, 64-channel 7 x 7 shape (the corner gather
// through the vector L1 bounds the rest).
//
// Software pipeline (two column-tile buffers per wave): step s runs the
// MFMAs of block s from buffer s & 1 while blending block s+1 into the other
// buffer, four passes of 8 pixels.  Each blended pass frees its corner
// registers, which immediately take the same pass of block s+2 (one full
// step before they are needed).
//
// Tap groups (WS = 2): for grids too small to hold two 4-wave workgroups per
// CU, a workgroup has 8 waves, two groups of four, each running the pipeline
// above over one half of the workgroup's taps; the four partial sums of each
// pixel meet in LDS at the end, so the chip holds two waves per SIMD with no
// partial outputs in memory.

#include <type_traits>

#include "dcn_device.h"
#include "dcn_launch.h"

namespace dcn {

typedef float f32x16 __attribute__((ext_vector_type(16)));

// NCH: the number of 64-channel chunks when it is known to be 1 (the
// 64-channel workloads), else 0 (read from the arguments): a compile-time 1
// removes the per-step divisions by it from the scalar instruction stream.
// WS: tap groups per workgroup (1: 4 waves, 2: 8 waves).
template <bool NHWC, bool FULLC, int NCH, int WS, class Src>
__global__ __launch_bounds__(256 * WS) __attribute__((amdgpu_waves_per_eu(2, 2))) void
fused_quad_kernel(Src src) {
  int logical;
  const FusedArgs& a = resolve_args(src, logical);
  const int nchunk = NCH > 0 ? NCH : a.nchunk;
  constexpr int M = 64;           // output pixels per workgroup
  constexpr int NO = 64;          // output channels per workgroup
  constexpr int CB = 64;          // channels per k-block
  constexpr int PW = 32;          // pixels per wave
  constexpr int AST = 32;         // column-tile row: 32 channels, 16-byte chunks XOR-swizzled
  constexpr int NSLOT = 3;        // coefficient ring
  constexpr int NWV = 4 * WS;     // waves
  constexpr int NTH = 64 * NWV;   // threads
  constexpr int A_FLOATS = PW * AST;  // one column tile
  constexpr int MAIN_BYTES = NWV * 2 * A_FLOATS * 4 + NWV * NSLOT * PW * 32;
  constexpr int RST = PW + 4;
  constexpr int RED_BYTES = NWV * NO * RST * 4;
  constexpr int SMEM = MAIN_BYTES > RED_BYTES ? MAIN_BYTES : RED_BYTES;

  __shared__ __attribute__((aligned(16))) char smem[SMEM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wq = WS == 1 ? 0 : wave >> 2;               // tap group
  const int wh = WS == 1 ? wave >> 1 : (wave >> 1) & 1;  // pixel half
  const int wc = wave & 1;   // channel half

  float* const Aw = reinterpret_cast<float*>(smem) + wave * 2 * A_FLOATS;  // [2][A_FLOATS]
  f32x4* const Cw = reinterpret_cast<f32x4*>(smem + NWV * 2 * A_FLOATS * 4) + wave * NSLOT * PW;
  u32x4* const Co =
      reinterpret_cast<u32x4*>(smem + NWV * 2 * A_FLOATS * 4 + NWV * NSLOT * PW * 16) +
      wave * NSLOT * PW;
  float* const red = reinterpret_cast<float*>(smem);  // [wave][NO][RST]
  // Column tile: row r (pixel), 16-byte chunk k (channels 4k .. 4k+3) at
  // float r * 32 + 4 * (k ^ ((r >> 1) & 7)): the eight-lane row writes of two
  // rows and the sixteen-row fragment reads both cover all banks.
  auto a_at = [](int r, int k) { return r * AST + 4 * (k ^ ((r >> 1) & 7)); };

  // workgroup -> (image, pixel tile, tap split, output tile); the splits of
  // one pixel tile are neighbours, so they share the XCD (and L2) that holds
  // its input rows.
  const int otile = logical % a.n_otiles;
  const int t1 = logical / a.n_otiles;
  const int split = t1 % a.nsplit;
  const int t2 = t1 / a.nsplit;
  const int tile = t2 % a.tiles_per_img;
  const int b = t2 / a.tiles_per_img;
  const int hw0 = tile * M + wh * PW;  // first pixel of this wave
  // taps [k0, k0 + kn) of this split and tap group (group 0 takes the first
  // ceil(n / 2) of the split's n taps, group 1 the rest: the host gives every
  // split at least WS taps); kt below counts from k0
  const int ks = split * a.kper;
  const int kns = min(a.kper, a.K - ks);
  const int khalf = WS == 1 ? kns : (kns + 1) >> 1;
  const int k0 = WS == 1 ? ks : ks + wq * khalf;
  const int kn = WS == 1 ? kns : (wq == 0 ? khalf : kns - khalf);
  const int NKB = kn * nchunk;
  auto clampb = [&](int kb) { return kb < NKB ? kb : NKB - 1; };
  auto clampt = [&](int kt) { return kt < kn ? kt : kn - 1; };

  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, a.x_bytes);
  const bool has_mask = a.mask != nullptr;
  const __amdgpu_buffer_rsrc_t offr = make_rsrc(a.offset, a.offset_bytes);
  const __amdgpu_buffer_rsrc_t mskr =
      make_rsrc(has_mask ? a.mask : a.offset, has_mask ? a.mask_bytes : 0u);
  const float* wblocks = static_cast<const float*>(a.wpack) +
                         ((size_t)otile * a.K + k0) * nchunk * (CB * NO);
  const uint32_t row_bytes = (uint32_t)a.C * 4;

  // ---- (a) coefficients: lane l -> pixel l & 31, corners 2(l>>5), 2(l>>5)+1
  const int c_px = lane & 31;
  const int c_pair = lane >> 5;
  const int c_hw = hw0 + c_px;
  const bool c_in = c_hw < a.HoWo;
  const int c_ho = c_hw / a.Wo;
  const int c_wo = c_hw - c_ho * a.Wo;
  float c_dy[2], c_dx[2], c_mk[2];
  auto coef_load = [&](int kt, float& dy, float& dx, float& mk) {
    const uint32_t ob =
        ((uint32_t)(b * 2 * a.K + 2 * (k0 + kt)) * (uint32_t)a.HoWo + (uint32_t)c_hw) * 4;
    const uint32_t mb = ((uint32_t)(b * a.K + k0 + kt) * (uint32_t)a.HoWo + (uint32_t)c_hw) * 4;
    dy = load_scalar<float>(offr, ob);
    dx = load_scalar<float>(offr, ob + (uint32_t)a.HoWo * 4);
    mk = load_scalar<float>(mskr, mb);
  };
  // The table entry of one tap, in four stages so that the step can spread
  // them over four MFMA slots: (0) the sampling point (sample_point), (1) the
  // lane's corner row and the validity of its two corners (corner_row),
  // (2) corner weights = bilinear weight x validity x mask, (3) the table
  // write (corner byte offsets, kNoCorner for an outside corner).
  const float c_gyb = (float)(c_ho - a.ph);  // exact: |values| < 2^24
  const float c_gxb = (float)(c_wo - a.pw);
  const float c_s = c_pair ? 1.0f : -1.0f, c_t = c_pair ? 0.0f : 1.0f;  // row weight ly*s + t
  const uint32_t c_img = (uint32_t)b * (uint32_t)a.H * (uint32_t)a.W;
  struct CoefState {
    SamplePoint p;
    CornerRow r;
    float w0, w1;
  } cs;
  auto coef_stage = [&](int stage, int kt, float dy, float dx, float mkr) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    if (stage == 0) {
      const int i = (k0 + kt) / a.kw, j = (k0 + kt) - ((k0 + kt) / a.kw) * a.kw;
      cs.p = sample_point(c_gyb + (float)i, c_gxb + (float)j, dy, dx);
    } else if (stage == 1) {
      cs.r = corner_row(cs.p, c_pair, a.H, a.W);
      cs.r.ok0 = c_in && cs.r.ok0;
      cs.r.ok1 = c_in && cs.r.ok1;
    } else if (stage == 2) {
      const float wy = __builtin_fmaf(cs.p.ly, c_s, c_t);  // 1 - ly or ly, exactly rounded
      const float wm = has_mask ? wy * mkr : wy;
      cs.w0 = cs.r.ok0 ? wm * (1.0f - cs.p.lx) : 0.0f;
      cs.w1 = cs.r.ok1 ? wm * cs.p.lx : 0.0f;
    } else {
      const int slot = kt % NSLOT;
      const uint32_t base = (c_img + (uint32_t)(cs.r.ry * a.W + cs.r.ix)) * row_bytes;
      const f32x2 w2 = {cs.w0, cs.w1};
      const u32x2 o2 = {cs.r.ok0 ? base : kNoCorner, cs.r.ok1 ? base + row_bytes : kNoCorner};
      if (a.dbg_corner != nullptr && c_in) {
        const size_t e = (((size_t)b * a.K + k0 + kt) * a.HoWo + c_hw) * 4 + 2 * c_pair;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          a.dbg_corner[e + q] = o2[q] == kNoCorner ? -1 : (int32_t)(o2[q] / row_bytes);
          a.dbg_weight[e + q] = w2[q];
        }
      }
      *reinterpret_cast<f32x2*>(reinterpret_cast<float*>(&Cw[slot * PW + c_px]) + 2 * c_pair) = w2;
      *reinterpret_cast<u32x2*>(reinterpret_cast<uint32_t*>(&Co[slot * PW + c_px]) + 2 * c_pair) =
          o2;
    }
  };
  auto coef_finish = [&](int kt, float dy, float dx, float mkr) {
#pragma unroll
    for (int st = 0; st < 4; ++st) coef_stage(st, kt, dy, dx, mkr);
  };

  // ---- (b) corners: lane = (pixel pp of an 8-pixel pass, 16-byte slice sl
  // of the wave's 32 channels); pass p covers the wave's pixels 8p .. 8p+7.
  const int pp = lane >> 3;
  const int sl = lane & 7;
  u32x4 gv[4][4];
  auto chan = [&](int kb, uint32_t& cbyte) {
    const int kt = kb / nchunk;
    const int ch = (kb - kt * nchunk) * CB + wc * 32 + sl * 4;
    cbyte = (uint32_t)ch * 4;
    return FULLC || ch < a.C;
  };
  auto slot_of = [&](int kb) { return (kb / nchunk) % NSLOT; };
  // the modulated sample of pass p: 4 corner slices times their weights
  auto blend = [&](const f32x4& w, int p) {
    f32x4 r = __builtin_bit_cast(f32x4, gv[p][0]) * w[0];
#pragma unroll
    for (int c = 1; c < 4; ++c) {
      const f32x4 v = __builtin_bit_cast(f32x4, gv[p][c]);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) r[kk] = __builtin_fmaf(w[c], v[kk], r[kk]);
    }
    return r;
  };

  // ---- (c) MFMA 32x32x2 (fp32): A row i = pixel (lane % 32), B column j =
  // output (lane % 32) of a 32-output half n; lane half hh = lane / 32 takes
  // k = hh of each k-step.  K-step t (0 .. 15) of the wave's 32 channels is
  // channel 16 hh + t for lane half hh, so fragment read q of a lane holds
  // channels 16 hh + 4q + [0, 4) of its pixel = k-steps 4q .. 4q+3.
  // Weight block layout [channel half wc][n][q][lane][e] (channel
  // 32 wc + 16 (lane / 32) + 4q + e, output 32 n + lane % 32): each of the
  // wave's 8 fragments is one 1 KB run.
  const int rl = lane & 31;
  const int hh = lane >> 5;
  f32x16 acc[2];
#pragma unroll
  for (int n = 0; n < 2; ++n)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[n][r] = 0.0f;
  f32x4 af[4];          // A fragments (q) of one block
  f32x4 bw[2][8];       // [set][n * 4 + q]
  auto b_src = [&](int kb) {
    return wblocks + (size_t)kb * (CB * NO) + (size_t)wc * (2 * 4 * 256) + lane * 4;
  };
  auto a_frag = [&](int buf, int q) {
    return *reinterpret_cast<const f32x4*>(&Aw[buf * A_FLOATS + a_at(rl, 4 * hh + q)]);
  };

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;

  // ---- prologue: tables of taps 0 .. 2, block 0 blended into tile buffer 0,
  // the corners of block 1 and the weights of block 0 in flight
  {
    float dy, dx, mk;
#pragma unroll
    for (int t = 0; t < 3; ++t) {
      coef_load(clampt(t), dy, dx, mk);
      coef_finish(clampt(t), dy, dx, mk);
    }
  }
  coef_load(clampt(3 / nchunk), c_dy[0], c_dx[0], c_mk[0]);
  coef_load(clampt(4 / nchunk), c_dy[1], c_dx[1], c_mk[1]);
  {
    const float* src = b_src(0);
#pragma unroll
    for (int k = 0; k < 8; ++k) bw[0][k] = *reinterpret_cast<const f32x4*>(src + k * 256);
  }
  {
    uint32_t cb0, cb1;
    const bool ok0 = chan(0, cb0);
    const bool ok1 = chan(clampb(1), cb1);
    const int s0 = slot_of(0), s1 = slot_of(clampb(1));
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const u32x4 off = Co[s0 * PW + p * 8 + pp];
#pragma unroll
      for (int c = 0; c < 4; ++c) gv[p][c] = load16(xr, ok0 ? off[c] + cb0 : kNoCorner);
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const f32x4 r = blend(Cw[s0 * PW + p * 8 + pp], p);
      *reinterpret_cast<f32x4*>(&Aw[a_at(p * 8 + pp, sl)]) = r;
      const u32x4 off = Co[s1 * PW + p * 8 + pp];
#pragma unroll
      for (int c = 0; c < 4; ++c) gv[p][c] = load16(xr, ok1 ? off[c] + cb1 : kNoCorner);
    }
#pragma unroll
    for (int q = 0; q < 3; ++q) af[q] = a_frag(0, q);
  }

  // ---- one step s: the 32 MFMAs of block s (tile buffer P = s & 1), with
  // one or two actions pinned after each, in this order: fragment 3 of block
  // s; per pass p of block s+1 (into buffer P ^ 1) the table reads, the four
  // blend terms, the tile write, the pass's corner loads for block s+2 and
  // two of block s+1's weight fragments; fragments 0 .. 2 of block s+1 (after
  // the MFMAs that read those registers for block s: fragment q serves MFMAs
  // 8q .. 8q+7); the coefficient table of tap (s+3)/nchunk in four stages from
  // offsets loaded two steps ago; the offsets of tap (s+5)/nchunk.
  constexpr int NMF = 32;  // MFMAs per step
  constexpr int NPA = 13;  // actions per pass
  constexpr int NACT = 1 + 4 * NPA + 3 + 4 + 1;
  auto step = [&](int s, auto par) {
    constexpr int P = decltype(par)::value;  // s & 1
    const int n1 = clampb(s + 1), n2 = clampb(s + 2);
    const int sl_1 = slot_of(n1), sl_2 = slot_of(n2);
    uint32_t cb2;
    const bool ok2 = chan(n2, cb2);
    const float* bsrc = b_src(n1);
    const int tc = (s + 3) / nchunk;
    const bool coef_due = tc * nchunk == s + 3 && tc < kn;
    const int tl = clampt((s + 5) / nchunk);
    f32x4 w;
    u32x4 off;
    f32x4 r;
    auto act = [&](auto X) {
      constexpr int x = decltype(X)::value;
      if constexpr (x == 0) {
        af[3] = a_frag(P, 3);
      } else if constexpr (x < 1 + 4 * NPA) {
        constexpr int p = (x - 1) / NPA, y = (x - 1) % NPA;
        if constexpr (y == 0) {
          w = Cw[sl_1 * PW + p * 8 + pp];
        } else if constexpr (y == 1) {
          off = Co[sl_2 * PW + p * 8 + pp];
        } else if constexpr (y < 6) {
          constexpr int c = y - 2;
          const f32x4 v = __builtin_bit_cast(f32x4, gv[p][c]);
          if constexpr (c == 0) {
            r = v * w[0];
          } else {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) r[kk] = __builtin_fmaf(w[c], v[kk], r[kk]);
          }
        } else if constexpr (y == 6) {
          *reinterpret_cast<f32x4*>(&Aw[(P ^ 1) * A_FLOATS + a_at(p * 8 + pp, sl)]) = r;
        } else if constexpr (y < 11) {
          constexpr int c = y - 7;
          gv[p][c] = load16(xr, ok2 ? off[c] + cb2 : kNoCorner);
        } else {
          constexpr int k = 2 * p + (y - 11);
          bw[P ^ 1][k] = *reinterpret_cast<const f32x4*>(bsrc + k * 256);
        }
      } else if constexpr (x < 4 + 4 * NPA) {
        af[x - 1 - 4 * NPA] = a_frag(P ^ 1, x - 1 - 4 * NPA);
      } else if constexpr (x < 8 + 4 * NPA) {
        if (coef_due) coef_stage(x - 4 - 4 * NPA, tc, c_dy[P], c_dx[P], c_mk[P]);
      } else {
        coef_load(tl, c_dy[P], c_dx[P], c_mk[P]);
      }
    };
    static_for<NMF>([&](auto J) {
      constexpr int jj = decltype(J)::value;
      constexpr int n = jj & 1, q = jj >> 3, e = (jj >> 1) & 3;  // k-step 4q + e
      acc[n] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[q][e], bw[P][n * 4 + q][e], acc[n], 0,
                                                     0, 0);
      // actions x with x * NMF / NACT == jj: x in [x0, x1)
      constexpr int x0 = (jj * NACT + NMF - 1) / NMF, x1 = ((jj + 1) * NACT + NMF - 1) / NMF;
      static_for<x1 - x0>([&](auto D) { act(std::integral_constant<int, x0 + decltype(D)::value>{}); });
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  int s = 0;
  for (; s + 1 < NKB; s += 2) {
    step(s, S0{});
    step(s + 1, S1{});
  }
  if (s < NKB) step(s, S0{});

  // ---- epilogue: sum the two channel halves (and tap groups) of each pixel
  // half, + bias, store: (g0 c0 + g0 c1) + (g1 c0 + g1 c1).  MFMA 32x32
  // result layout: lane l, register r -> row (pixel) 8 (r / 4) + 4 (l / 32) +
  // r % 4, column (output of half n) l % 32.
  __syncthreads();  // every wave is done with its column tiles and tables
#pragma unroll
  for (int n = 0; n < 2; ++n)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
      *reinterpret_cast<f32x4*>(&red[(wave * NO + n * 32 + rl) * RST + 8 * r4 + 4 * hh]) =
          f32x4{acc[n][4 * r4], acc[n][4 * r4 + 1], acc[n][4 * r4 + 2], acc[n][4 * r4 + 3]};
  __syncthreads();
  const float* biasp = static_cast<const float*>(a.bias);  // NULL for a split
  float* const outp = a.out + (size_t)split * a.split_stride;
  const int base_hw = tile * M;
  if constexpr (!NHWC) {
    // thread -> (pixel half, output channel, run of 4 pixels)
    for (int e = tid; e < 2 * NO * (PW / 4); e += NTH) {
      const int h = e / (NO * (PW / 4));
      const int rem = e - h * NO * (PW / 4);
      const int col = rem / (PW / 4);
      const int r4 = rem - col * (PW / 4);
      const int o = otile * NO + col;
      if (o >= a.O) continue;
      const int w0 = h * 2;  // waves (h, 0) and (h, 1) of tap group 0
      f32x4 v = *reinterpret_cast<const f32x4*>(&red[(w0 * NO + col) * RST + r4 * 4]);
      v += *reinterpret_cast<const f32x4*>(&red[((w0 + 1) * NO + col) * RST + r4 * 4]);
      if constexpr (WS == 2) {
        f32x4 u = *reinterpret_cast<const f32x4*>(&red[((w0 + 4) * NO + col) * RST + r4 * 4]);
        u += *reinterpret_cast<const f32x4*>(&red[((w0 + 5) * NO + col) * RST + r4 * 4]);
        v += u;
      }
      v += biasp ? biasp[o] : 0.0f;
      const int hw = base_hw + h * PW + r4 * 4;
      float* dst = outp + ((size_t)b * a.O + o) * a.HoWo + hw;
      if (a.vec_store && hw + 3 < a.HoWo) {
        *reinterpret_cast<f32x4*>(dst) = v;
      } else {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          if (hw + rr < a.HoWo) dst[rr] = v[rr];
      }
    }
  } else {
    for (int e = tid; e < M * NO; e += NTH) {
      const int col = e % NO;
      const int px = e / NO;
      const int h = px / PW, row = px - h * PW;
      const int o = otile * NO + col;
      const int hw = base_hw + px;
      if (o >= a.O || hw >= a.HoWo) continue;
      float v = red[(2 * h * NO + col) * RST + row] + red[((2 * h + 1) * NO + col) * RST + row];
      if constexpr (WS == 2)
        v += red[((2 * h + 4) * NO + col) * RST + row] + red[((2 * h + 5) * NO + col) * RST + row];
      v += biasp ? biasp[o] : 0.0f;
      outp[((size_t)b * a.HoWo + hw) * a.O + o] = v;
    }
  }
}

bool quad_supported(const KernelConfig& kc) {
  return !kc.bf16 && kc.CB == 64 && kc.NO == 64 && kc.M == 64;
}

namespace {
template <bool NHWC, int NCH, int WS, class Src>
void launch_quad_fc(bool fullc, dim3 grid, hipStream_t s, const Src& src) {
  const dim3 block(256 * WS);
  if (fullc) hipLaunchKernelGGL((fused_quad_kernel<NHWC, true, NCH, WS, Src>), grid, block, 0, s, src);
  else hipLaunchKernelGGL((fused_quad_kernel<NHWC, false, NCH, WS, Src>), grid, block, 0, s, src);
}

template <int WS, class Src>
void launch_quad_ws(bool nhwc, bool one_chunk, bool fullc, dim3 grid, hipStream_t s,
                    const Src& src) {
  if (nhwc) {
    if (one_chunk) launch_quad_fc<true, 1, WS>(fullc, grid, s, src);
    else launch_quad_fc<true, 0, WS>(fullc, grid, s, src);
  } else {
    if (one_chunk) launch_quad_fc<false, 1, WS>(fullc, grid, s, src);
    else launch_quad_fc<false, 0, WS>(fullc, grid, s, src);
  }
}
}  // namespace

hipError_t launch_fused_quad(const KernelConfig& kc, const FusedArgs& a, hipStream_t s) {
  // every split needs at least one tap, and with two tap groups two
  if (a.nsplit < 1 || a.kper < a.wsplit || (a.wsplit != 1 && a.wsplit != 2) ||
      (int64_t)(a.nsplit - 1) * a.kper >= a.K || a.K - (int64_t)(a.nsplit - 1) * a.kper < a.wsplit)
    return hipErrorInvalidValue;
  const int64_t nblk = (int64_t)a.B * kc.tiles_per_img * a.nsplit * kc.n_otiles;
  if (nblk <= 0) return hipSuccess;
  if (nblk > 0x7fffffff || !quad_supported(kc)) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)nblk);
  const bool fullc = a.C % 64 == 0, one_chunk = a.nchunk == 1;
  if (a.wsplit == 2) launch_quad_ws<2>(kc.nhwc, one_chunk, fullc, grid, s, a);
  else launch_quad_ws<1>(kc.nhwc, one_chunk, fullc, grid, s, a);
  return hipGetLastError();
}

namespace {
// Sum of the tap splits plus bias.  Thread -> 4 consecutive elements (16-B
// loads and store when the count is a multiple of 4; the buffers are 16-B
// aligned and the split stride is a multiple of 4 floats).
__global__ __launch_bounds__(256) void split_reduce_kernel(const float* __restrict__ part,
                                                           int nsplit, uint32_t stride,
                                                           const float* __restrict__ bias,
                                                           float* __restrict__ out, int64_t n,
                                                           int O, int HoWo, int nhwc) {
  const int64_t n4 = n / 4;
  for (int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x; v < (n + 3) / 4;
       v += (int64_t)gridDim.x * 256) {
    const int64_t i0 = v * 4;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (v < n4) {
      for (int s = 0; s < nsplit; ++s)
        acc += *reinterpret_cast<const f32x4*>(part + (size_t)s * stride + i0);
    } else {
      for (int s = 0; s < nsplit; ++s)
        for (int e = 0; e < 4; ++e)
          if (i0 + e < n) acc[e] += part[(size_t)s * stride + i0 + e];
    }
    if (bias) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t i = i0 + e;
        const int o = nhwc ? (int)(i % O) : (int)((i / HoWo) % O);
        if (i < n) acc[e] += bias[o];
      }
    }
    if (v < n4) {
      *reinterpret_cast<f32x4*>(out + i0) = acc;
    } else {
      for (int e = 0; e < 4; ++e)
        if (i0 + e < n) out[i0 + e] = acc[e];
    }
  }
}
}  // namespace

hipError_t launch_split_reduce(const float* part, int nsplit, uint32_t stride, const float* bias,
                               float* out, int B, int O, int HoWo, int nhwc, hipStream_t s) {
  const int64_t n = (int64_t)B * O * HoWo;
  if (n <= 0) return hipSuccess;
  if (nsplit < 1 || stride % 4 != 0 || (int64_t)stride < n) return hipErrorInvalidValue;
  const int64_t want = ((n + 3) / 4 + 255) / 256;
  const unsigned nblk = (unsigned)(want < 4096 ? want : 4096);
  hipLaunchKernelGGL(split_reduce_kernel, dim3(nblk), dim3(256), 0, s, part, nsplit, stride, bias,
                     out, n, O, HoWo, nhwc);
  return hipGetLastError();
}

hipError_t launch_fused_quad_multi(const KernelConfig& kc, const MultiArgs& m, hipStream_t s) {
  if (m.n < 1) return hipSuccess;
  bool one_chunk = true;
  const int ws = m.a[0].wsplit;
  for (int i = 0; i < m.n; ++i) {
    one_chunk = one_chunk && m.a[i].nchunk == 1;
    // one tap-group count per launch, never a split into runs
    if (m.a[i].wsplit != ws || (ws != 1 && ws != 2) || m.a[i].nsplit != 1 ||
        m.a[i].K < ws)
      return hipErrorInvalidValue;
  }
  const int64_t nblk = m.start[m.n];
  if (nblk <= 0) return hipSuccess;
  if (nblk > 0x7fffffff || !quad_supported(kc)) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)nblk);
  if (ws == 2) launch_quad_ws<2>(kc.nhwc, one_chunk, m.a[0].C % 64 == 0, grid, s, m);
  else launch_quad_ws<1>(kc.nhwc, one_chunk, m.a[0].C % 64 == 0, grid, s, m);
  return hipGetLastError();
}

}  // namespace dcn
