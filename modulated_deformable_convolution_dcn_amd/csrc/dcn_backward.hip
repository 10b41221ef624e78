// dcn_backward.hip -- fp32 backward of the modulated deformable conv2d.
//
// The forward (page 1, "deform_conv.py": sample the NHWC input bilinearly at
// (h - pad + i + dy, w - pad + j + dx), corners outside count as zero, times
// mask_k, contract over (tap, channel) with the weight, + bias), differentiated
// term by term.  With g = dL/dout, for output pixel p and tap k (floor cell
// (y0, x0), fractions (ly, lx), corner weights w_ab, mask m):
//   gs[c]        = sum_o g[p, o] W[o, c, k]          (an MFMA contraction)
//   dL/dx_ab[c] += gs[c] m w_ab                        (scatter: atomics)
//   dL/dm       += sum_c gs[c] su[c],  su[c] = sum_ab w_ab x_ab[c]
//   dL/ddy      += m sum_c gs[c] sum_ab (dw_ab/dly) x_ab[c]   (and dx)
//   dL/dW[o,c,k]+= g[p, o] m su[c]                     (an MFMA contraction)
//   dL/dbias[o] += g[p, o]
// Page 5 notes that the gradient scatter of these operators needs atomic
// adds into fp32 accumulators; the input gradient here is exactly that.
//
// Three kernels after zero-filling the outputs:
//   bwd_data   one workgroup per 8 x 8 block of output pixels: the g tile
//              stays in LDS, per (tap, 64-channel chunk) gs comes from MFMA
//              against the re-packed weight, then each thread takes one
//              pixel's 4-channel slice: corner loads, input-gradient adds
//              (into an LDS window around the block, flushed once per chunk;
//              far corners straight to memory), and the mask / offset sums
//              reduced over the 16 lanes of the pixel;
//   bwd_weight one workgroup per (tap, chunk, image, run of pixel tiles):
//              MFMA accumulates dW over the run in registers, then one
//              atomic add per weight element; up to 64 outputs each wave
//              feeds its blended samples to the MFMA straight from
//              registers (bwd_weight2), wider outputs go through LDS tiles
//              (bwd_weight);
//   bwd_bias   a per-output sum of g.

#include <type_traits>

#include "dcn_device.h"
#include "dcn_launch.h"

namespace dcn {

namespace {

constexpr int TILE = 64;   // output pixels per tile
constexpr int GPAD = 4;    // LDS row padding (floats)

__device__ __forceinline__ void atomic_add(float* p, float v) { unsafeAtomicAdd(p, v); }

// Per (pixel, tap): the sampling point and the validity-masked corner
// weights, their derivatives and the corner pixel indices (row-major in the
// image) -- from the forward's corner stage (tap_corners).
struct TapTerms {
  float w[4], dwy[4], dwx[4];
  int pix[4];
  int y0, x0;  // corner (0, 0), clamped to [-2, H] x [-2, W]
  bool ok[4];
};

__device__ __forceinline__ TapTerms tap_terms(const BwdArgs& a, int b, int ho, int wo, int k) {
  const int i = k / a.kw, j = k - (k / a.kw) * a.kw;
  const size_t ob = ((size_t)(b * 2 * a.K + 2 * k) * a.HoWo) + (size_t)ho * a.Wo + wo;
  const float dy = a.offset[ob], dx = a.offset[ob + a.HoWo];
  const TapCorners t =
      tap_corners((float)(ho - a.ph + i), (float)(wo - a.pw + j), dy, dx, a.H, a.W);
  const float ly = t.p.ly, lx = t.p.lx;
  const float hy = 1.0f - ly, hx = 1.0f - lx;
  const float wv[4] = {hy * hx, hy * lx, ly * hx, ly * lx};
  const float vy[4] = {-hx, -lx, hx, lx};
  const float vx[4] = {-hy, hy, -ly, ly};
  const int y0 = t.y0;
  const int x0 = t.x0;
  TapTerms r;
  r.y0 = y0;
  r.x0 = x0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    r.ok[q] = (t.valid >> q) & 1u;
    r.w[q] = r.ok[q] ? wv[q] : 0.0f;
    r.dwy[q] = r.ok[q] ? vy[q] : 0.0f;
    r.dwx[q] = r.ok[q] ? vx[q] : 0.0f;
    r.pix[q] = (b * a.H + y0 + (q >> 1)) * a.W + x0 + (q & 1);
  }
  return r;
}

// Sum over each row of 16 lanes, the result in every lane of the row (DPP:
// swap neighbours, swap pairs, mirror halves of 8, mirror the row).
__device__ __forceinline__ float row16_sum(float v) {
  auto dpp = [](float x, auto CTRL) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                           decltype(CTRL)::value, 0xF, 0xF, false));
  };
  v += dpp(v, std::integral_constant<int, 0xB1>{});   // quad_perm [1, 0, 3, 2]
  v += dpp(v, std::integral_constant<int, 0x4E>{});   // quad_perm [2, 3, 0, 1]
  v += dpp(v, std::integral_constant<int, 0x141>{});  // row_half_mirror
  v += dpp(v, std::integral_constant<int, 0x140>{});  // row_mirror
  return v;
}

__device__ __forceinline__ float gout_at(const BwdArgs& a, int b, int o, int hw) {
  return a.nhwc_g ? a.gout[((size_t)b * a.HoWo + hw) * a.O + o]
                  : a.gout[((size_t)b * a.O + o) * a.HoWo + hw];
}

}  // namespace

// ---------------------------------------------------------------- data grads
// LDS budget of the input-gradient window, per padded output count (with the
// g tile, the gs tile, the tables and the scatter lists the kernel uses
// <= 160 KB of LDS).
constexpr int bwd_window_floats(int OP) {
  return OP <= 64 ? 28480 : OP <= 128 ? 24384 : 15872;
}
constexpr int WSTR = 64;  // floats per window position: the chunk's 64 channels

// One workgroup = an 8 x 8 block of output pixels of one image.  Its
// sampling points cluster around the block, so the input gradient of the
// window [wy0, wy0 + WH) x [wx0, wx0 + WW) (the block's footprint grown by R
// on every side) is accumulated in LDS and flushed to memory once per
// 64-channel chunk; corners outside the window (far offsets) go straight to
// memory with atomics.  R < 0: no window.
//
// Per 64-channel chunk the taps run as a two-stage pipeline, one barrier
// pair per tap: the MFMAs form gs = g W^T of tap k; after the second barrier
// every thread issues the corner loads of tap k + 1 (and, for up to 64
// outputs, its weight fragments) before it works on tap k with the corners
// loaded one tap earlier.  The sampling tables of tap k sit in slot k % 3:
// wave 0 builds those of tap k + 2 after its own scatter of tap k, in the
// time the other waves' scatter leaves it before the next barrier.
//
// Tap k's work has two layouts.  The mask / offset sums need the corner
// values: 16 lanes per pixel, 4 channels each (one 16-byte load per corner),
// reduced over the 16 lanes and staged in LDS for one wave to write at the
// next tap.  The input-gradient scatter needs none: each window position
// belongs to one wave, which adds 16 lanes x 4 channels per item with plain
// LDS read-add-writes (see step (2b)).
template <int OP>  // padded output channels: 16, 64, 128 or 256
__global__ __launch_bounds__(512) void bwd_data_kernel(BwdArgs a, int R, int tiles_x,
                                                       int tiles_per_img) {
  constexpr int GST = OP + GPAD;     // g tile row stride
  constexpr int SST = 64 + GPAD;     // gs tile row stride
  constexpr bool WPRE = OP <= 64;    // next tap's weight fragments held in registers
  constexpr int NW = 8;              // waves: two per SIMD
  constexpr int NT = 64 * NW;        // threads
  constexpr int NPASS = TILE * 16 / NT;  // sum passes (16 lanes per pixel)
  constexpr int NQ = OP / 16;
  // up to 64 outputs the g^T fragments stay in registers and the gs tile has
  // two buffers: one barrier per tap, and a wave done with its scatter of
  // tap k goes on to the MFMAs of tap k + 1 while others still scatter
  constexpr bool ONEBAR = OP <= 64;
  __shared__ __attribute__((aligned(16))) float Gs[ONEBAR ? 4 : TILE * GST];
  __shared__ __attribute__((aligned(16))) float gsT[(ONEBAR ? 2 : 1) * TILE * SST];
  // the window, then 64 floats that take the scatter's discarded adds
  constexpr int SINK = bwd_window_floats(OP);
  __shared__ __attribute__((aligned(16))) float win[SINK + 64];
  // three sets of tables of the block's 64 sampling points (written by wave 0):
  //   Tf {ly, lx, mask, validity bits as an int}
  //   Si {window offset of corner (0,0), corner flags, image pixel of (0,0),
  //       byte offset of corner (0,0) in x}
  //   Sf {mask x corner weight, 0 for an invalid corner}
  // corner flags: bit q = in the window, bit 4 + q = valid but outside it,
  // bits 8-9 = window column of corner (0,0) mod 4, bits 10-12 = its window
  // row mod 8
  __shared__ f32x4 Tf[3][TILE];
  __shared__ int4 Si[3][TILE];
  __shared__ f32x4 Sf[3][TILE];
  const float* const Sfl = reinterpret_cast<const float*>(&Sf[0][0]);  // [3][TILE][4]
  __shared__ float red[2][3][TILE];  // mask, dy, dx sums of a tap
  __shared__ int ilist[NW][2 * TILE];  // per wave: scatter items of one corner pair

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // MFMA: wave -> pixel rows 32 mr .. 32 mr + 31, channels 16 mh .. 16 mh + 15
  // (one weight fragment per k-step shared by two pixel tiles)
  const int mr = wave & 1, mh = wave >> 1;
  const int logical = xcd_logical_block(blockIdx.x, gridDim.x);
  const int tile = logical % tiles_per_img, b = logical / tiles_per_img;
  const int ty = tile / tiles_x, tx = tile - (tile / tiles_x) * tiles_x;
  // the input gradient is optional: without it there is no window, no
  // scatter and no flush (only the mask / offset sums run)
  const bool want_gx = a.gx != nullptr;
  const bool use_win = R >= 0 && want_gx;
  const int WH = 8 + a.kh + 2 * R, WW = 8 + a.kw + 2 * R;
  const int wy0 = 8 * ty - a.ph - R, wx0 = 8 * tx - a.pw - R;
  // pixel px of the block -> output (8ty + px / 8, 8tx + px % 8)
  auto px_hw = [&](int px, int& hw) {
    const int ho = 8 * ty + (px >> 3), wo = 8 * tx + (px & 7);
    hw = ho * a.Wo + wo;
    return ho < a.Ho && wo < a.Wo;
  };

  // g tile [64 pixels][OP outputs], zero outside
  if constexpr (!ONEBAR) {
    for (int e = tid; e < TILE * OP; e += NT) {
      const int o = e / TILE, px = e % TILE;
      int hw;
      const bool in = px_hw(px, hw);
      Gs[px * GST + o] = (o < a.O && in) ? gout_at(a, b, o, hw) : 0.0f;
    }
  }

  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, a.x_bytes);
  const int rl = lane & 15, g = lane >> 4;
  // the same g values as MFMA A fragments of this wave's two pixel tiles:
  // ga[q][pt][e] = g[pixel 32 mr + 16 pt + rl][output 16 q + 4 g + e]
  f32x4 ga[ONEBAR ? NQ : 1][2];
  if constexpr (ONEBAR) {
#pragma unroll
    for (int pt = 0; pt < 2; ++pt) {
      int hw;
      const bool in = px_hw(32 * mr + 16 * pt + rl, hw);
#pragma unroll
      for (int q = 0; q < NQ; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int o = 16 * q + 4 * g + e;
          ga[q][pt][e] = (in && o < a.O) ? gout_at(a, b, o, hw) : 0.0f;
        }
    }
  }
  const int sl = tid & 15;  // 4-channel slice of the 64-channel chunk (sum layout)
  const int nwin = use_win ? WH * WW : 0;

  // wave 0: the offsets / mask of a tap, loaded a tap before its tables
  int t_hw = 0;
  const bool t_in = tid < TILE && px_hw(tid, t_hw);
  const int t_ho = t_hw / a.Wo, t_wo = t_hw - (t_hw / a.Wo) * a.Wo;
  float n_dy = 0.f, n_dx = 0.f, n_m = 1.f;
  auto t_load = [&](int k) {
    if (!t_in) return;
    const size_t ob = (size_t)(b * 2 * a.K + 2 * k) * a.HoWo + t_hw;
    n_dy = a.offset[ob];
    n_dx = a.offset[ob + a.HoWo];
    n_m = a.mask ? a.mask[(size_t)(b * a.K + k) * a.HoWo + t_hw] : 1.0f;
  };
  auto t_build = [&](int slot, int k) {  // tid < TILE
    const int i = k / a.kw, j = k - (k / a.kw) * a.kw;
    const TapCorners tp =
        tap_corners((float)(t_ho - a.ph + i), (float)(t_wo - a.pw + j), n_dy, n_dx, a.H, a.W);
    const int y0 = tp.y0;
    const int x0 = tp.x0;
    const uint32_t v4 = t_in ? tp.valid : 0u;
    // corner (0,0)'s byte offset; the other corners are a uniform step away
    // (used only for valid corners, whose offsets are exact and in range)
    const uint32_t b00 = (uint32_t)((b * a.H + y0) * a.W + x0) * ((uint32_t)a.C * 4u);
    Tf[slot][tid] = f32x4{tp.p.ly, tp.p.lx, n_m, __int_as_float((int)v4)};
    const float hy = 1.0f - tp.p.ly, hx = 1.0f - tp.p.lx;
    const float wv[4] = {hy * hx, hy * tp.p.lx, tp.p.ly * hx, tp.p.ly * tp.p.lx};
    f32x4 cf;
    int flags = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bool ok = (v4 >> q) & 1u;
      cf[q] = ok ? n_m * wv[q] : 0.0f;
      const int wy = y0 + (q >> 1) - wy0, wx = x0 + (q & 1) - wx0;
      const bool inwin = use_win && wy >= 0 && wy < WH && wx >= 0 && wx < WW;
      if (ok) flags |= inwin ? (1 << q) : (16 << q);
    }
    flags |= ((x0 - wx0) & 3) << 8;          // window column mod 4 (scatter classes)
    flags |= ((y0 - wy0) & (NW - 1)) << 10;  // window row mod 8 (owner wave of the row)
    Si[slot][tid] = make_int4(((y0 - wy0) * WW + (x0 - wx0)) * WSTR, flags,
                              (b * a.H + y0) * a.W + x0, (int)b00);
    Sf[slot][tid] = cf;
  };
  // wave 1: the mask / offset gradients of tap k from the staged sums.  Every
  // (pixel, tap) element belongs to this workgroup alone, so the first chunk
  // stores it (the outputs need no zero fill) and later chunks add to it.
  auto sums_store = [&](int slot, int k, bool first) {
    int hw;
    if (!px_hw(lane, hw)) return;
    auto put = [&](float* d, float v) {
      if (first) *d = v;
      else atomic_add(d, v);
    };
    if (a.gmask) put(a.gmask + (size_t)(b * a.K + k) * a.HoWo + hw, red[slot][0][lane]);
    if (a.goff) {
      put(a.goff + (size_t)(b * 2 * a.K + 2 * k) * a.HoWo + hw, red[slot][1][lane]);
      put(a.goff + (size_t)(b * 2 * a.K + 2 * k + 1) * a.HoWo + hw, red[slot][2][lane]);
    }
  };

  // corner values of the sum passes x 4 corners, one buffer per table slot
  u32x4 cv[2][NPASS][4];
  f32x4 bw[WPRE ? NQ : 1];
  auto w_load = [&](int kb) {
    if constexpr (WPRE) {
      const float* wt = a.wt + (size_t)kb * OP * 64;
#pragma unroll
      for (int q = 0; q < NQ; ++q)
        bw[q] = *reinterpret_cast<const f32x4*>(&wt[((4 * q + g) * 64 + 16 * mh + rl) * 4]);
    }
  };

  // byte steps from corner (0,0) to corners (0,1), (1,0), (1,1) in x
  const uint32_t row_b = (uint32_t)a.C * 4u;
  const uint32_t corner_step[4] = {0u, row_b, (uint32_t)a.W * row_b, (uint32_t)(a.W + 1) * row_b};

  for (int chunk = 0; chunk < a.nchunk; ++chunk) {
    for (int e = tid; e < nwin * WSTR; e += NT) win[e] = 0.0f;
    const int ch = chunk * 64 + 4 * sl;
    const bool chan_ok = ch < a.C;            // sum layout

    // corner loads of the tap in table slot ts into register buffer BUF
    auto c_issue = [&](auto BUF, int ts) {
      constexpr int S = decltype(BUF)::value;
#pragma unroll
      for (int p = 0; p < NPASS; ++p) {
        const int4 si = Si[ts][(NT / 16) * p + (tid >> 4)];
        const uint32_t base = (uint32_t)si.w + (uint32_t)ch * 4u;
        const int v4 = si.y | (si.y >> 4);  // in the window or not
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const bool ok = chan_ok && ((v4 >> q) & 1);
          cv[S][p][q] = load16(xr, ok ? base + corner_step[q] : kNoCorner);
        }
      }
    };

    // prologue: tables of taps 0 and 1, offsets of tap 2, corners and
    // weights of tap 0.  Tap k's tables live in slot k % 3; wave 0 builds
    // those of tap k + 2 after its own scatter of tap k.
    if (tid < TILE) {
      t_load(0);
      t_build(0, 0);
      if (a.K > 1) {
        t_load(1);
        t_build(1, 1);
      }
      t_load(a.K > 2 ? 2 : 0);
    }
    __syncthreads();  // tables of taps 0, 1 visible; window zeroed
    c_issue(std::integral_constant<int, 0>{}, 0);
    w_load(chunk);

    // (1) gs[px, c] = sum_o g[px, o] W[o, c, tap] into tile gt: wave w ->
    // pixel rows 32 (w % 2) .., channels 16 (w / 2) ..
    auto mfma_tap = [&](int kb, float* gt) {
      f32x4 acc[2];
#pragma unroll
      for (int pt = 0; pt < 2; ++pt) acc[pt] = f32x4{0.f, 0.f, 0.f, 0.f};
      const float* wt = a.wt + (size_t)kb * OP * 64;
#pragma unroll 4
      for (int q = 0; q < NQ; ++q) {
        f32x4 af[2];
#pragma unroll
        for (int pt = 0; pt < 2; ++pt) {
          if constexpr (ONEBAR)
            af[pt] = ga[q][pt];
          else
            af[pt] = *reinterpret_cast<const f32x4*>(
                &Gs[(32 * mr + 16 * pt + rl) * GST + 16 * q + 4 * g]);
        }
        f32x4 bf;
        if constexpr (WPRE)
          bf = bw[q];
        else
          bf = *reinterpret_cast<const f32x4*>(&wt[((4 * q + g) * 64 + 16 * mh + rl) * 4]);
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int pt = 0; pt < 2; ++pt)
            acc[pt] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[pt][e], bf[e], acc[pt], 0, 0, 0);
      }
      // MFMA 16x16 layout: lane l, register r -> row 4(l/16) + r, column l % 16
#pragma unroll
      for (int pt = 0; pt < 2; ++pt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          gt[(32 * mr + 16 * pt + 4 * g + r) * SST + 16 * mh + rl] = acc[pt][r];
    };
    if constexpr (ONEBAR) mfma_tap(chunk, gsT);  // tap 0 into buffer 0

    auto step = [&](int k, int ts, auto PAR) {
      constexpr int P = decltype(PAR)::value;  // k & 1: corner buffer and sums of tap k
      const int ts1 = ts == 2 ? 0 : ts + 1, ts2 = ts1 == 2 ? 0 : ts1 + 1;  // slots of k + 1, k + 2
      const int kb = k * a.nchunk + chunk;
      const bool more = k + 1 < a.K;
      float* const gt = gsT + (ONEBAR ? P * TILE * SST : 0);  // gs tile of tap k
      // two barriers: step k-1 is done with the gs tile and its sums, then
      // the MFMAs of tap k; one barrier: the MFMAs of tap k were the end of
      // every wave's step k-1
      __syncthreads();
      if (wave == 1 && k > 0) sums_store(P ^ 1, k - 1, chunk == 0);
      if constexpr (!ONEBAR) {
        mfma_tap(kb, gt);
        __syncthreads();  // gs tile visible
      }

      // (2) weights and corner loads of tap k + 1, then tap k's sums and scatter
      if (more) {
        w_load(kb + a.nchunk);
        c_issue(std::integral_constant<int, P ^ 1>{}, ts1);
      }
      // (2a) sums: pass p -> pixel (NT / 16) p + tid / 16, 4 channels per lane
#pragma unroll
      for (int p = 0; p < NPASS; ++p) {
        const int px = (NT / 16) * p + (tid >> 4);
        const f32x4 tf = Tf[ts][px];
        float sm = 0.f, sdy = 0.f, sdx = 0.f;
        if (__float_as_int(tf[3]) != 0 && chan_ok) {  // any valid corner
          const float ly = tf[0], lx = tf[1], hy = 1.0f - ly, hx = 1.0f - lx;
          const float wv[4] = {hy * hx, hy * lx, ly * hx, ly * lx};
          const float vy[4] = {-hx, -lx, hx, lx};
          const float vx[4] = {-hy, hy, -ly, ly};
          const f32x4 gs = *reinterpret_cast<const f32x4*>(&gt[px * SST + 4 * sl]);
#pragma unroll
          for (int q = 0; q < 4; ++q) {  // an outside corner was loaded as zeros: no terms
            const f32x4 v = __builtin_bit_cast(f32x4, cv[P][p][q]);
            float t = gs[0] * v[0];
#pragma unroll
            for (int e = 1; e < 4; ++e) t = __builtin_fmaf(gs[e], v[e], t);
            sm = __builtin_fmaf(wv[q], t, sm);
            sdy = __builtin_fmaf(vy[q], t, sdy);
            sdx = __builtin_fmaf(vx[q], t, sdx);
          }
        }
        // sum over the 16 lanes of the pixel (one DPP row)
        sm = row16_sum(sm);
        sdy = row16_sum(sdy);
        sdx = row16_sum(sdx);
        if (sl == 0) {
          red[P][0][px] = sm;
          red[P][1][px] = tf[2] * sdy;
          red[P][2][px] = tf[2] * sdx;
        }
      }
      // (2b) scatter.  Window row wy belongs to wave wy mod 8, so no two waves
      // ever update one position and the updates are plain LDS read-add-writes
      // (float atomics cost far more).  An item is one pixel's corner pair
      // (h, 0), (h, 1): two neighbouring positions of one row, so one owner.
      // The wave lists its items (position, in-window bits, pixel, pair) in
      // LDS, grouped by window column mod 4, and takes one of each group at a
      // time: 16 lanes per item, 4 channels per lane; the gs slice is read
      // once, then position (h, 0) and position (h, 1) each get one 16-byte
      // read, 4 FMAs and one 16-byte write per lane, in that order.  Equal
      // pairs fall in one group, so a batch never names a position twice in
      // one of its two updates, and a pair's second position met as another
      // group's first is updated after it.  Far corners of the wave's 8
      // pixels go to memory with atomics.
      if (want_gx) {
        const int4 si = Si[ts][lane];  // lane = pixel
        const f32x4 sf = Sf[ts][lane];
        const int grp = lane >> 4, sub = lane & 15;
        static_for<4>([&](auto Q) {
          constexpr int q = decltype(Q)::value;
          // the corner weight as a scalar first: taking the bits of a vector
          // element directly reads element 0 with this compiler
          const float sfq = sf[q];
          const bool far = ((si.y >> (4 + q)) & 1) && (lane >> 3) == wave;
          uint64_t m_far = __ballot(far);
          while (m_far) {
            const int p = __builtin_ctzll(m_far);
            m_far &= m_far - 1;
            const int pix = __builtin_amdgcn_readlane(si.z, p) + (q >> 1) * a.W + (q & 1);
            const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sfq), p));
            if (chunk * 64 + lane < a.C)  // lanes past C would reach the next pixel
              atomic_add(a.gx + (size_t)pix * a.C + chunk * 64 + lane, gt[p * SST + lane] * c);
          }
        });
        // position classes (window column mod 4): a class's items are listed
        // together, and batch j takes the j-th item of each class (lane
        // group g <- class g)
        const int cls = (si.y >> 8) & 3;
        const int row8 = (si.y >> 10) & (NW - 1);
        bool own[2];
        int ent[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int inw = (si.y >> (2 * h)) & 3;  // corners (h, 0), (h, 1) in the window
          own[h] = inw != 0 && ((row8 + h) & (NW - 1)) == wave;
          // list entry: window position index of (h, 0), in-window bits,
          // pixel, pair (the corner weights are read back from the table)
          ent[h] = (((si.x >> 6) + h * WW) << 9) | (inw << 7) | (lane << 1) | h;
        }
        // wave-uniform: class bits and owners as masks; per class and pair
        // the bucket sizes, packed one byte per class (every count is at most
        // 128): bucket starts of pair 0 and pair 1 items, class sizes
        const uint64_t X = __ballot(cls & 1), Y = __ballot(cls & 2);
        const uint64_t O0 = __ballot(own[0]), O1 = __ballot(own[1]);
        uint32_t st0 = 0, st1 = 0, szs = 0;
        int nb = 0;
        {
          int acc = 0;
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const uint64_t cm = ((g & 1) ? X : ~X) & ((g & 2) ? Y : ~Y);
            const int n0 = __builtin_popcountll(O0 & cm), n1 = __builtin_popcountll(O1 & cm);
            st0 |= (uint32_t)acc << (8 * g);
            st1 |= (uint32_t)(acc + n0) << (8 * g);
            szs |= (uint32_t)(n0 + n1) << (8 * g);
            acc += n0 + n1;
            nb = max(nb, n0 + n1);
          }
        }
        // lanes of another class than this lane's
        const uint64_t other = (X ^ ((cls & 1) ? ~0ull : 0ull)) | (Y ^ ((cls & 2) ? ~0ull : 0ull));
#pragma unroll
        for (int h = 0; h < 2; ++h)
          if (own[h]) {
            const uint64_t mm = (h ? O1 : O0) & ~other;
            const int idx = (int)__builtin_amdgcn_ubfe(h ? st1 : st0, 8 * cls, 8) +
                            (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mm >> 32),
                                                           __builtin_amdgcn_mbcnt_lo((uint32_t)mm, 0));
            ilist[wave][idx] = ent[h];
          }
        const int my_n = (int)__builtin_amdgcn_ubfe(szs, 8 * grp, 8);
        const int my_base = (int)__builtin_amdgcn_ubfe(st0, 8 * grp, 8);
        // software pipeline: while batch j updates the window, the weights
        // and gs slice of batch j + 1 and the list entry of batch j + 2 are
        // in flight
        auto entry = [&](int j) { return ilist[wave][j < my_n ? my_base + j : 0]; };
        int e_next = entry(1), pa, pb;
        float2 c;
        f32x4 g4;
        auto fetch = [&](int j, int it) {
          const bool valid = j < my_n;
          const int p0 = (it >> 9) * WSTR;
          pa = valid && ((it >> 7) & 1) ? p0 : SINK;
          pb = valid && ((it >> 8) & 1) ? p0 + WSTR : SINK;
          c = *reinterpret_cast<const float2*>(&Sfl[ts * TILE * 4 + ((it & 127) << 1)]);
          g4 = *reinterpret_cast<const f32x4*>(&gt[((it >> 1) & 63) * SST + 4 * sub]);
        };
        fetch(0, entry(0));
        for (int j = 0; j < nb; ++j) {
          float* da = &win[pa + 4 * sub];
          float* db = &win[pb + 4 * sub];
          f32x4 w4 = *reinterpret_cast<const f32x4*>(da);
          const float2 cj = c;
          const f32x4 gj = g4;
          {  // the last batch fetches entry 0 and the sink: harmless
            const int e = e_next;
            e_next = entry(j + 2);
            fetch(j + 1, e);
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) w4[e] = __builtin_fmaf(gj[e], cj.x, w4[e]);
          *reinterpret_cast<f32x4*>(da) = w4;
          f32x4 v4 = *reinterpret_cast<const f32x4*>(db);
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = __builtin_fmaf(gj[e], cj.y, v4[e]);
          *reinterpret_cast<f32x4*>(db) = v4;
        }
      }
      // (2c) wave 0, in the time the other waves' scatter leaves it: tables of
      // tap k + 2 into the slot of tap k - 1 (unused since this step's first
      // barrier), then the offsets of tap k + 3
      if (wave == 0 && k + 2 < a.K) {
        t_build(ts2, k + 2);
        t_load(k + 3 < a.K ? k + 3 : 0);
      }
      // (2d) one barrier per tap: the MFMAs of tap k + 1 into the other gs
      // buffer (last read in step k - 1, which every wave had finished before
      // this step's barrier)
      if constexpr (ONEBAR)
        if (more) mfma_tap(kb + a.nchunk, gsT + (P ^ 1) * TILE * SST);
    };
    int k = 0, ts = 0;
    for (; k + 1 < a.K; k += 2) {
      step(k, ts, std::integral_constant<int, 0>{});
      ts = ts == 2 ? 0 : ts + 1;
      step(k + 1, ts, std::integral_constant<int, 1>{});
      ts = ts == 2 ? 0 : ts + 1;
    }
    if (k < a.K) step(k, ts, std::integral_constant<int, 0>{});

    // (3) the last tap's sums, then flush the window's input gradient of this chunk
    __syncthreads();
    if (wave == 1) sums_store((a.K - 1) & 1, a.K - 1, chunk == 0);
    for (int e = tid; e < nwin * 64; e += NT) {
      const int pos = e >> 6, c = e & 63;
      const int y = wy0 + pos / WW, xx = wx0 + pos % WW;
      const float v = win[pos * WSTR + c];
      if (v != 0.0f && y >= 0 && y < a.H && xx >= 0 && xx < a.W && chunk * 64 + c < a.C)
        atomic_add(a.gx + ((size_t)(b * a.H + y) * a.W + xx) * a.C + chunk * 64 + c, v);
    }
    __syncthreads();  // flush and sums done before the next chunk reuses window and tables
  }
}

// ---------------------------------------------------------------- weight grad
// Weight gradient, wave-private pipeline (fp32).
// dW[o, c, k] = sum over pixels of g[px, o] * s[px, k, c], s the modulated
// sample of the forward.  One workgroup per (output tile of OP, tap, chunk,
// image, run of 64-pixel tiles), output tiles fastest so that the tiles of
// one sample run meet its corners in the same L2; wave w owns pixels
// [16w, 16w + 16) of every tile and accumulates dW[the tile's o][chunk's
// 64 c] over them in registers, so the main
// loop has no barrier.  Per tile it blends its 16 samples x 64 channels in 4
// passes (corners loaded one tile ahead, 16 lanes per pixel, one 16-byte load
// per corner): pass p gives lane (sl, q) = (lane % 16, lane / 16) channels
// 4 sl .. 4 sl + 3 of pixel 4 q + p.  Those registers are the B operand of
// MFMA k-step p as they stand -- k = q, column n = sl of output tile u holds
// channel 4 n + u -- so the samples never go through LDS; A = g^T fragments
// (4 consecutive pixels of one output, one 16-byte load from an NCHW
// gradient; element p is pixel 4 q + p).  Tile u's column n is channel
// 4 n + u of the chunk, which the epilogue undoes.  The four waves' partial
// sums meet in LDS once per run, then one atomic add per weight element.
// The loop body has no branches: the next tile's table, corner loads and g
// fragments are issued unconditionally (past the run's end they read clamped
// offsets, zeros or in-range data that is never used), so the compiler keeps
// one register assignment and needs no copies at the loop's joins.
//   NTO: 16-output tiles (OP / 16: 1 or 4)
//   GV: NCHW g, Ho*Wo % 4 == 0 and one image of g below 2^31 bytes (16-byte
//       buffer loads of g^T fragments, two tiles ahead)
//   FULLC: C % 64 == 0 (every lane's channels exist)
template <int NTO, bool GV, bool FULLC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void
bwd_weight2_kernel(BwdArgs a, int n_otiles, int tiles_per_run, int runs_per_img) {
  constexpr int OP = 16 * NTO;
  constexpr int RST = 64 + 4;                   // epilogue row: 64 channels + 4
  constexpr int LOOP_BYTES = 4 * 2 * 16 * 32;   // per wave: tables of two tiles
  constexpr int RED_BYTES = 4 * OP * RST * 4;
  constexpr int SMEM = LOOP_BYTES > RED_BYTES ? LOOP_BYTES : RED_BYTES;
  __shared__ __attribute__((aligned(16))) char smem[SMEM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  f32x4* const Cw = reinterpret_cast<f32x4*>(smem) + wave * 32;  // [2][16]
  u32x4* const Co = reinterpret_cast<u32x4*>(smem + 4 * 32 * 16) + wave * 32;
  float* const red = reinterpret_cast<float*>(smem);  // [wave][o][RST]

  const int logical = xcd_logical_block(blockIdx.x, gridDim.x);
  // output tile, then (tap, chunk) fastest: the workgroups of one XCD share
  // pixel runs, so one run's corner reads (every output tile reads the same
  // ones, neighbouring taps nearly the same) meet in that XCD's L2
  const int otile = logical % n_otiles;
  const int t1 = logical / n_otiles;
  const int kb = t1 % (a.K * a.nchunk);
  const int t2 = t1 / (a.K * a.nchunk);
  const int run = t2 % runs_per_img;
  const int b = t2 / runs_per_img;
  const int k = kb / a.nchunk, chunk = kb - k * a.nchunk;
  const int ki = k / a.kw, kj = k - ki * a.kw;
  const int o0 = otile * OP;  // first output of the tile
  const int t_begin = run * tiles_per_run;
  const int t_end = min(t_begin + tiles_per_run, a.tiles_per_img);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, a.x_bytes);
  const uint32_t row_bytes = (uint32_t)a.C * 4;

  // ---- table of one tile: lanes 0..15 -> pixel 16 wave + lane (all lanes
  // load, so every wave issues the same memory operations)
  const int tl = lane & 15;
  float n_dy = 0.f, n_dx = 0.f, n_m = 0.f;
  auto t_load = [&](int tile) {
    const int hw = tile * 64 + 16 * wave + tl;
    const int hc = hw < a.HoWo ? hw : a.HoWo - 1;
    const size_t ob = (size_t)(b * 2 * a.K + 2 * k) * a.HoWo + hc;
    n_dy = a.offset[ob];
    n_dx = a.offset[ob + a.HoWo];
    const float mv = a.mask ? a.mask[(size_t)(b * a.K + k) * a.HoWo + hc] : 1.0f;
    n_m = hw < a.HoWo ? mv : 0.0f;
  };
  auto t_build = [&](int slot, int tile) {
    const int hw = tile * 64 + 16 * wave + tl;
    const int ho = hw / a.Wo, wo = hw - (hw / a.Wo) * a.Wo;
    const TapCorners tp =
        tap_corners((float)(ho - a.ph + ki), (float)(wo - a.pw + kj), n_dy, n_dx, a.H, a.W);
    const float hy = 1.0f - tp.p.ly, hx = 1.0f - tp.p.lx;
    const float wv[4] = {hy * hx, hy * tp.p.lx, tp.p.ly * hx, tp.p.ly * tp.p.lx};
    const int y0 = tp.y0;
    const int x0 = tp.x0;
    f32x4 w4;
    u32x4 o4;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bool ok = ((tp.valid >> q) & 1u) && n_m != 0.0f;
      w4[q] = ok ? n_m * wv[q] : 0.0f;
      const uint32_t pix = (uint32_t)((b * a.H + y0 + (q >> 1)) * a.W + x0 + (q & 1));
      o4[q] = ok ? pix * row_bytes : kNoCorner;
    }
    if (lane < 16) {
      Cw[slot * 16 + tl] = w4;
      Co[slot * 16 + tl] = o4;
    }
  };

  // ---- corners: pass p -> pixel 4 (lane / 16) + p, channels 4 (lane % 16) ..
  const int sl = lane & 15, pq = lane >> 4;
  const uint32_t cbyte = (uint32_t)(chunk * 64 + 4 * sl) * 4;
  const bool chan_ok = FULLC || chunk * 64 + 4 * sl < a.C;
  u32x4 cv[4][4];
  auto c_issue = [&](int slot, int p) {
    const u32x4 o4 = Co[slot * 16 + 4 * pq + p];
#pragma unroll
    for (int q = 0; q < 4; ++q) cv[p][q] = load16(xr, chan_ok ? o4[q] + cbyte : kNoCorner);
  };
  // the modulated sample of pass p: channels 4 sl .. 4 sl + 3 of pixel 4 pq + p
  auto blend = [&](int slot, int p) {
    const f32x4 w4 = Cw[slot * 16 + 4 * pq + p];
    f32x4 sv = __builtin_bit_cast(f32x4, cv[p][0]) * w4[0];
#pragma unroll
    for (int q = 1; q < 4; ++q) {
      const f32x4 v = __builtin_bit_cast(f32x4, cv[p][q]);
#pragma unroll
      for (int e = 0; e < 4; ++e) sv[e] = __builtin_fmaf(w4[q], v[e], sv[e]);
    }
    return sv;
  };

  // ---- g^T fragments: lane -> output 16t + lane % 16, pixels 4 (lane / 16) ..
  const int rl = lane & 15, g = lane >> 4;
  // gf[P]: fragments of the tile in slot P, loaded two tiles ahead
  f32x4 gf[2][NTO];
  // GV: one image of g through a buffer descriptor; output o's row starts at
  // byte o * Ho*Wo * 4, and a lane whose output or pixels fall outside reads
  // zeros (kNoCorner)
  const __amdgpu_buffer_rsrc_t gr =
      make_rsrc(a.gout + (size_t)b * a.O * a.HoWo, GV ? (uint32_t)a.O * a.HoWo * 4u : 0u);
  uint32_t g_row[NTO];
#pragma unroll
  for (int t = 0; t < NTO; ++t) {
    const int o = o0 + 16 * t + rl;
    g_row[t] = o < a.O ? (uint32_t)o * (uint32_t)a.HoWo * 4u : kNoCorner;
  }
  auto g_load = [&](f32x4* dst, int tile) {
    const int hw = tile * 64 + 16 * wave + 4 * g;
    if constexpr (GV) {
      const bool hw_ok = hw < a.HoWo;  // Ho*Wo % 4 == 0: all four pixels or none
#pragma unroll
      for (int t = 0; t < NTO; ++t)
        dst[t] = __builtin_bit_cast(
            f32x4, load16(gr, hw_ok ? g_row[t] + (uint32_t)hw * 4u : kNoCorner));
    } else {
#pragma unroll
      for (int t = 0; t < NTO; ++t) {
        const int o = o0 + 16 * t + rl;
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        if (o < a.O) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (hw + e < a.HoWo) v[e] = gout_at(a, b, o, hw + e);
        }
        dst[t] = v;
      }
    }
  };

  f32x4 acc[NTO][4];
#pragma unroll
  for (int t = 0; t < NTO; ++t)
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[t][u] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Tile `tile` (slot P): the table of tile + 1 into the other slot and the
  // offsets of tile + 2 first, then per pass the blend of this tile, the
  // corner loads of tile + 1 into the freed registers and the MFMAs; last the
  // g^T fragments of tile + 2 into this tile's buffer.  Past the run's end
  // (t_load clamps its pixel) the work is wasted but harmless.
  auto step = [&](int tile, auto PAR) {
    constexpr int P = decltype(PAR)::value;  // slot / buffer of this tile
    t_build(P ^ 1, tile + 1);
    t_load(tile + 2);
    // dW[o][c] += sum over the wave's 16 pixels: k-step p takes pixels
    // 4 q + p (q = lane / 16) -- the samples of pass p -- and column n of
    // tile u is channel 4 n + u
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const f32x4 sv = blend(P, p);
      c_issue(P ^ 1, p);
#pragma unroll
      for (int t = 0; t < NTO; ++t)
#pragma unroll
        for (int u = 0; u < 4; ++u)
          acc[t][u] =
              __builtin_amdgcn_mfma_f32_16x16x4f32(gf[P][t][p], sv[u], acc[t][u], 0, 0, 0);
    }
    g_load(gf[P], tile + 2);
  };

  if (t_begin < t_end) {
    t_load(t_begin);
    t_build(0, t_begin);
    t_load(t_begin + 1);
#pragma unroll
    for (int p = 0; p < 4; ++p) c_issue(0, p);
    g_load(gf[0], t_begin);
    g_load(gf[1], t_begin + 1);
    int tile = t_begin;
    for (; tile + 1 < t_end; tile += 2) {
      step(tile, std::integral_constant<int, 0>{});
      step(tile + 1, std::integral_constant<int, 1>{});
    }
    if (tile < t_end) step(tile, std::integral_constant<int, 0>{});
  }

  // ---- the four waves' partial sums, then one atomic add per element
  __syncthreads();  // every wave is done with its s^T tile and tables
  // MFMA 16x16 layout: lane l, register r -> row 4(l/16) + r (output), column
  // l % 16 (channel 4 (l % 16) + u of tile u)
#pragma unroll
  for (int t = 0; t < NTO; ++t)
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        red[(wave * OP + 16 * t + 4 * g + r) * RST + 4 * rl + u] = acc[t][u][r];
  __syncthreads();
  for (int e = tid; e < OP * 64; e += 256) {
    const int ol = e >> 6, c = e & 63;
    const int o = o0 + ol, cc = chunk * 64 + c;
    if (o >= a.O || cc >= a.C) continue;
    const float v = red[(0 * OP + ol) * RST + c] + red[(1 * OP + ol) * RST + c] +
                    red[(2 * OP + ol) * RST + c] + red[(3 * OP + ol) * RST + c];
    atomic_add(a.gw + (((size_t)o * a.C + cc) * a.kh + ki) * a.kw + kj, v);
  }
}

// ---------------------------------------------------------------- bias grad
// dL/dbias[o] = sum of g over images and pixels.  NCHW g: one workgroup per
// (output, image, pixel range), threads along the contiguous pixels, a tree
// sum in LDS, one atomic add.  NHWC g: one workgroup per (image, pixel
// range), thread t -> output t % 64 of rows t / 64, 4 rows ..., per-output
// sums in LDS, one atomic add per output.
constexpr int kBiasPixels = 4096;  // pixels per workgroup
__global__ __launch_bounds__(256) void bwd_bias_kernel(BwdArgs a, int nsplit) {
  __shared__ float red[256];
  const int tid = threadIdx.x;
  if (!a.nhwc_g) {
    const int split = blockIdx.x % nsplit, t2 = blockIdx.x / nsplit;
    const int o = t2 % a.O, b = t2 / a.O;
    const int h0 = split * kBiasPixels, h1 = min(h0 + kBiasPixels, a.HoWo);
    const float* src = a.gout + ((size_t)b * a.O + o) * a.HoWo;
    float s = 0.f;
    for (int hw = h0 + tid; hw < h1; hw += 256) s += src[hw];
    red[tid] = s;
    __syncthreads();
    for (int w = 128; w >= 1; w >>= 1) {
      if (tid < w) red[tid] += red[tid + w];
      __syncthreads();
    }
    if (tid == 0) atomic_add(a.gb + o, red[0]);
  } else {
    const int split = blockIdx.x % nsplit, b = blockIdx.x / nsplit;
    const int h0 = split * kBiasPixels, h1 = min(h0 + kBiasPixels, a.HoWo);
    for (int o0 = 0; o0 < a.O; o0 += 64) {
      const int o = o0 + (tid & 63);
      float s = 0.f;
      if (o < a.O)
        for (int hw = h0 + (tid >> 6); hw < h1; hw += 4)
          s += a.gout[((size_t)b * a.HoWo + hw) * a.O + o];
      red[tid] = s;
      __syncthreads();
      if (tid < 64 && o < a.O) atomic_add(a.gb + o, red[tid] + red[tid + 64] + red[tid + 128] + red[tid + 192]);
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------- helpers
__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ p, int64_t n) {
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256)
    p[e] = 0.0f;
}


// weight [O][C][kh][kw] -> per (tap, 64-channel chunk) block [OP/4][64][4]:
// element (o, c) at ((o / 4) * 64 + c % 64) * 4 + o % 4, so one 16-byte read
// gives a lane 4 consecutive outputs of one channel (4 MFMA k-steps).  One
// thread per packed element, padding (o >= O or c >= C) written as zero in
// the same pass.  The same launch zero-fills the weight and bias gradients
// (nw and nb elements of gw and gb; the weight and bias kernels add into
// them with atomics).
__global__ __launch_bounds__(256) void bwd_pack_kernel(const float* __restrict__ w,
                                                       float* __restrict__ wt, int O, int C,
                                                       int K, int OP, int nchunk,
                                                       float* __restrict__ gw, int64_t nw,
                                                       float* __restrict__ gb, int64_t nb) {
  const int64_t total = (int64_t)K * nchunk * OP * 64;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < nw + nb;
       e += (int64_t)gridDim.x * 256) {
    if (e < nw) gw[e] = 0.0f;
    else gb[e - nw] = 0.0f;
  }
  for (int64_t d = (int64_t)blockIdx.x * 256 + threadIdx.x; d < total;
       d += (int64_t)gridDim.x * 256) {
    const int64_t blk = d / (OP * 64);
    const int rem = (int)(d - blk * (OP * 64));
    const int o = (rem >> 8) * 4 + (rem & 3);
    const int c = (int)(blk % nchunk) * 64 + ((rem >> 2) & 63);
    const int tap = (int)(blk / nchunk);
    wt[d] = (o < O && c < C) ? w[((int64_t)o * C + c) * K + tap] : 0.0f;
  }
}

// bf16 -> fp32, exact: dst[i] = src[i] for i < n (8 elements per thread and
// step; src and dst 16-byte aligned, a tail of n % 8 element-wise).
__global__ __launch_bounds__(256) void widen_bf16_kernel(const uint16_t* __restrict__ src,
                                                         float* __restrict__ dst, int64_t n) {
  const int64_t n8 = n / 8;
  for (int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x; v < n8;
       v += (int64_t)gridDim.x * 256) {
    const u32x4 q = *reinterpret_cast<const u32x4*>(src + 8 * v);
    f32x4 lo, hi;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      lo[2 * e] = __uint_as_float(q[e] << 16);
      lo[2 * e + 1] = __uint_as_float(q[e] & 0xffff0000u);
      hi[2 * e] = __uint_as_float(q[2 + e] << 16);
      hi[2 * e + 1] = __uint_as_float(q[2 + e] & 0xffff0000u);
    }
    *reinterpret_cast<f32x4*>(dst + 8 * v) = lo;
    *reinterpret_cast<f32x4*>(dst + 8 * v + 4) = hi;
  }
  if (blockIdx.x == 0)
    for (int64_t i = n8 * 8 + threadIdx.x; i < n; i += 256)
      dst[i] = __uint_as_float((uint32_t)src[i] << 16);
}

namespace {
unsigned grid_of(int64_t n) {
  int64_t g = (n + 255) / 256;
  return (unsigned)(g < 1 ? 1 : g > 65535 ? 65535 : g);
}

hipError_t zero(float* p, int64_t n, hipStream_t s) {
  if (!p || n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(grid_of(n)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_widen_bf16(const void* src, float* dst, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(widen_bf16_kernel, dim3(grid_of((n + 7) / 8)), dim3(256), 0, s,
                     static_cast<const uint16_t*>(src), dst, n);
  return hipGetLastError();
}

int bwd_out_pad(int O) { return O <= 16 ? 16 : O <= 64 ? 64 : O <= 128 ? 128 : 256; }

int64_t bwd_workspace_floats(int O, int C, int K) {
  return (int64_t)K * ((C + 63) / 64) * bwd_out_pad(O) * 64;
}

hipError_t launch_backward(const BwdArgs& a0, const float* weight, float* ws, hipStream_t s) {
  BwdArgs a = a0;
  const int OP = bwd_out_pad(a.O);
  hipError_t e;
  // zero the outputs that atomics accumulate into: grad_x here, the weight
  // and bias gradients in the re-pack launch (the offset and mask gradients
  // are stored by their owning workgroup, the re-packed weight writes its own
  // padding)
  const int64_t nx = (int64_t)a.B * a.H * a.W * a.C;
  if ((e = zero(a.gx, nx, s)) != hipSuccess) return e;
  const int64_t nw = a.gw ? (int64_t)a.O * a.C * a.K : 0, nb = a.gb ? a.O : 0;
  const int64_t nws = bwd_workspace_floats(a.O, a.C, a.K);
  hipLaunchKernelGGL(bwd_pack_kernel, dim3(grid_of(nws > nw + nb ? nws : nw + nb)), dim3(256), 0,
                     s, weight, ws, a.O, a.C, a.K, OP, a.nchunk, a.gw, nw, a.gb, nb);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  a.wt = ws;
  if (a.gx || a.goff || a.gmask) {
    // 8 x 8 output blocks; window radius R: the largest that fits the LDS
    // budget (-1: none)
    const int tiles_x = (a.Wo + 7) / 8, tiles_y = (a.Ho + 7) / 8;
    const int tiles = tiles_x * tiles_y;
    const int64_t nblk = (int64_t)a.B * tiles;
    if (nblk > 0x7fffffff) return hipErrorInvalidConfiguration;
    const int budget = OP <= 16 ? bwd_window_floats(16) : OP <= 64 ? bwd_window_floats(64)
                       : OP <= 128 ? bwd_window_floats(128) : bwd_window_floats(256);
    int R = -1;
    for (int r = 0; r <= 8; ++r)
      if ((int64_t)(8 + a.kh + 2 * r) * (8 + a.kw + 2 * r) * WSTR <= budget) R = r;
    const dim3 grid((unsigned)nblk), block(512);
    switch (OP) {
      case 16: hipLaunchKernelGGL(bwd_data_kernel<16>, grid, block, 0, s, a, R, tiles_x, tiles); break;
      case 64: hipLaunchKernelGGL(bwd_data_kernel<64>, grid, block, 0, s, a, R, tiles_x, tiles); break;
      case 128: hipLaunchKernelGGL(bwd_data_kernel<128>, grid, block, 0, s, a, R, tiles_x, tiles); break;
      default: hipLaunchKernelGGL(bwd_data_kernel<256>, grid, block, 0, s, a, R, tiles_x, tiles); break;
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (a.gw) {
    // output tiles of 16 (O <= 16) or 64, and runs of pixel tiles: two
    // workgroups per CU, at most 512 workgroups when the units allow, so the
    // grid is about one round and each run's closing reduction is spread
    // over many tiles
    const int wop = OP <= 16 ? 16 : 64;
    const int n_ot = (a.O + wop - 1) / wop;
    const int64_t per_run_units = (int64_t)a.K * a.nchunk * a.B * n_ot;
    int64_t runs = 512 / per_run_units;
    if (runs > a.tiles_per_img) runs = a.tiles_per_img;
    if (runs < 1) runs = 1;
    const int tiles_per_run = (int)((a.tiles_per_img + runs - 1) / runs);
    const int runs_per_img = (a.tiles_per_img + tiles_per_run - 1) / tiles_per_run;
    const int64_t g = per_run_units * runs_per_img;
    if (g > 0x7fffffff) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)g), block(256);
    const bool gv = !a.nhwc_g && a.HoWo % 4 == 0 && (int64_t)a.O * a.HoWo * 4 < (1ll << 31);
    const bool fullc = a.C % 64 == 0;
#define DCN_W2(NTO, GV, FC) \
  hipLaunchKernelGGL((bwd_weight2_kernel<NTO, GV, FC>), grid, block, 0, s, a, n_ot, tiles_per_run, \
                     runs_per_img)
#define DCN_W2F(NTO)                          \
  if (gv && fullc) DCN_W2(NTO, true, true);   \
  else if (gv) DCN_W2(NTO, true, false);      \
  else if (fullc) DCN_W2(NTO, false, true);   \
  else DCN_W2(NTO, false, false)
    if (wop == 16) DCN_W2F(1);
    else DCN_W2F(4);
#undef DCN_W2F
#undef DCN_W2
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (a.gb) {
    const int nsplit = (a.HoWo + kBiasPixels - 1) / kBiasPixels;
    const int64_t nb = (a.nhwc_g ? (int64_t)a.B : (int64_t)a.B * a.O) * nsplit;
    if (nb > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(bwd_bias_kernel, dim3((unsigned)nb), dim3(256), 0, s, a, nsplit);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace dcn
