// dcn_bf16win.hip -- bf16 fused DCNv2 forward for wide outputs and 3 x 3
// kernels, with the corner gather served from an input window staged in LDS.
//
// Same operator as the other kernels (page 1, "deform_conv.py": sample the
// input bilinearly at (h - pad + i + dy, w - pad + j + dx), corners outside
// count as zero, times the mask, contract over (tap, channel) with the
// weight, + bias), for bf16 operands with fp32 accumulation (page 5,
// deformops README: float32 accumulation for every operand dtype), 3 x 3
// kernels and channel counts that are multiples of 64.
//
// Why a window: at 256 output channels every sampled corner feeds 256
// multiply-adds per channel, and fetching the four corner slices of every
// (pixel, tap) through the vector L1 takes longer than the bf16 MFMAs that
// consume them.  The corners of one tile and all its taps lie within a few
// pixels of the tile, so the workgroup copies that neighbourhood -- an input
// window of (8 + 2 + 2R + 1) x (16 + 2 + 2R + 1) pixels, R = 7 pixels of
// offset reach -- into LDS, 32 channels at a time, and blends from there.
// The window of the next 32 channels is loaded while the current ones are
// consumed (two window buffers), so the copy costs no time of its own after
// the first.  A tile with any inside-image corner beyond its window (an
// offset larger than R near the tile's edge: 1 of the detection workload's
// 256 tiles) runs the same pipeline with every corner fetched from memory
// instead, so the result never depends on R.  The choice is made once per
// tile: a load under a branch inside the pipelined slots would make the
// compiler wait for every load in flight.
//
// Work layout: one workgroup of 8 waves (two per SIMD: while one waits on
// LDS or memory the other issues) owns an 8 x 16 pixel tile x 256 output
// channels, accumulators in registers; wave w owns outputs [32w, 32w+32)
// and loads exactly its own weight fragments from L2.  The k-axis runs
// chunk-major: for each 32-channel chunk, the 9 taps.  The corner tables
// (weights and window or memory offsets of the 4 corners) of all 9 taps are
// built once per tile.  Per k-block step the 16 MFMAs of block s are
// interleaved with the blend of block s+1 into the idle LDS column tile, the
// corner fetches of block s+2 and a slice of the next window.  The blend
// pairs the two corners of a corner row channel by channel (a byte permute)
// and takes each pair's weighted sum with one bf16 dot product into an fp32
// accumulator (the products of two bf16 values are exact in fp32): two
// instructions per two multiply-adds, with no widening of the bf16 corner
// values; the sum is rounded to bf16 once.  On this chip VALU work beside
// the MFMAs is not hidden behind them, so the blend's instruction count is
// part of every step's time.

#include <type_traits>

#include "dcn_device.h"
#include "dcn_launch.h"

namespace dcn {

namespace {
constexpr int kWinTH = 8;   // tile rows
constexpr int kWinTW = 16;  // tile columns
constexpr int kWinR = 7;    // offset reach the window covers, pixels
constexpr int kWinK = 3;    // kernel height and width
}  // namespace

template <bool NHWC, class Src>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void
fused_bf16win_kernel(Src src) {
  int logical;
  const FusedArgs& a = resolve_args(src, logical);
  constexpr int TH = kWinTH, TW = kWinTW, M = TH * TW;  // 128 pixels
  constexpr int KT = kWinK * kWinK;   // 9 taps
  constexpr int NO = 256;             // output channels per workgroup
  constexpr int CB = 32;              // channels per k-block (one MFMA k-step)
  constexpr int MT = M / 16;          // 16-row tiles
  constexpr int NT = 512;             // threads
  constexpr int NTW = 2;              // 16-column tiles per wave
  constexpr int ROWB = CB * 2;        // column-tile and window row bytes
  constexpr int A_BYTES = M * ROWB;
  constexpr int NSL = MT * NTW;       // MFMA slots per block
  constexpr int AFD = 3;              // column-tile fragments read this many tiles ahead
  constexpr int WH = TH + kWinK - 1 + 2 * kWinR + 1;  // 25 window rows
  constexpr int WW = TW + kWinK - 1 + 2 * kWinR + 1;  // 33 window columns
  constexpr int WIN_PX = WH * WW;
  constexpr uint32_t ZERO_ROW = (uint32_t)WIN_PX * ROWB;  // a row of zeros after the window
  constexpr int WIN_BYTES = (WIN_PX + 1) * ROWB;
  constexpr int NFILL = WIN_PX * 4;                  // 16-byte window loads per chunk
  constexpr int FPT = (NFILL + NT - 1) / NT;         // ... per thread (7)
  constexpr int KPT = (KT + 1) / 2;                  // taps per table thread
  static_assert(NSL == 16, "one blend unit per MFMA slot");
  static_assert(FPT <= KT - 2, "the next window lands before its first fetch");

  __shared__ __attribute__((aligned(16))) char As[2][A_BYTES];
  __shared__ __attribute__((aligned(16))) char Win[2][WIN_BYTES];
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  __shared__ u32x2 Cw[KT][M];  // corner weights (bilinear x validity x mask) in bf16, corner
                               // row a: (a, 0) in the low half, (a, 1) in the high half
  __shared__ u32x4 Cx[KT][M];  // corner byte offsets: in the window (ZERO_ROW: outside)
                               // or, for a tile fetched from memory, in x (kNoCorner)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  const int otile = logical % a.n_otiles;
  const int t2 = logical / a.n_otiles;
  const int tile = t2 % a.tiles_per_img;
  const int b = t2 / a.tiles_per_img;
  const int ty0 = (tile / a.tiles_x) * TH;
  const int tx0 = (tile - (tile / a.tiles_x) * a.tiles_x) * TW;
  // the window: image rows [wy0, wy0 + WH) x columns [wx0, wx0 + WW)
  const int wy0 = ty0 - a.ph - kWinR;
  const int wx0 = tx0 - a.pw - kWinR;
  const int nch = a.nchunk * 2;  // 32-channel chunks (C is a multiple of 64)

  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, a.x_bytes);
  const bool has_mask = a.mask != nullptr;
  const __amdgpu_buffer_rsrc_t offr = make_rsrc(a.offset, a.offset_bytes);
  const __amdgpu_buffer_rsrc_t mskr =
      make_rsrc(has_mask ? a.mask : a.offset, has_mask ? a.mask_bytes : 0u);
  // the packed weight of this output tile: per (tap, 64-channel chunk), two
  // 32-channel k-steps of 1024 fragments (u32x4) each; this lane's fragment
  // of 16-column tile nt at wlane + nt * 64
  const u32x4* wtile = reinterpret_cast<const u32x4*>(static_cast<const __bf16*>(a.wpack) +
                                                      (size_t)otile * KT * a.nchunk * (64 * NO));
  const int wlane = wave * NTW * 64 + lane;
  const uint32_t row_bytes = (uint32_t)a.C * 2;

  // zero rows read by every outside corner
  if (tid < 2 * (ROWB / 16)) {
    char* z = Win[tid / (ROWB / 16)] + ZERO_ROW + (tid % (ROWB / 16)) * 16;
    *reinterpret_cast<u32x4*>(z) = u32x4{0u, 0u, 0u, 0u};
  }

  // ---- window loads: this thread's load u (0 .. FPT) of a chunk is element
  // e = u * NT + tid: window pixel e / 4, 16-byte slice e % 4 of the chunk's
  // 32 channels; its offset in x for chunk 0 (kNoCorner outside the image or
  // past the window: it stays past the end of x for every chunk)
  uint32_t fg[FPT];
#pragma unroll
  for (int u = 0; u < FPT; ++u) {
    const int e = u * NT + tid;
    const int px = e >> 2;
    const int y = wy0 + px / WW, x = wx0 + px % WW;
    const bool in = e < NFILL && (uint32_t)y < (uint32_t)a.H && (uint32_t)x < (uint32_t)a.W;
    fg[u] = in ? (uint32_t)((b * a.H + y) * a.W + x) * row_bytes + (uint32_t)(e & 3) * 16
               : kNoCorner;
  }
  auto fill_load = [&](int chunk, int u) {
    return load16(xr, fg[u] + (uint32_t)chunk * (CB * 2));
  };
  auto fill_store = [&](int buf, int u, const u32x4& v) {
    const int e = u * NT + tid;
    if (e < NFILL) *reinterpret_cast<u32x4*>(Win[buf] + e * 16) = v;
  };

  // ---- (a) corner tables: thread -> pixel tid & 127 (row m / 16, column
  // m % 16 of the tile), corner row a = (tid >> 7) & 1 (corners (a, 0),
  // (a, 1)), taps k = 2q + (tid >> 8).  The offsets and mask of all taps are
  // loaded at once, together with the first window.
  const int c_px = tid & (M - 1);
  const int c_pair = (tid >> 7) & 1;
  const int c_k0 = tid >> 8;
  const int c_ho = ty0 + c_px / TW;
  const int c_wo = tx0 + c_px % TW;
  const bool c_in = c_ho < a.Ho && c_wo < a.Wo;
  const int c_hw = c_ho * a.Wo + c_wo;
  float dy[KPT], dx[KPT], mk[KPT];
  {
    const uint32_t hw = c_in ? (uint32_t)c_hw : 0u;
#pragma unroll
    for (int q = 0; q < KPT; ++q) {
      const int k = 2 * q + c_k0 < KT ? 2 * q + c_k0 : KT - 1;
      const uint32_t ob = ((uint32_t)(b * 2 * KT + 2 * k) * (uint32_t)a.HoWo + hw) * 2;
      const uint32_t mb = ((uint32_t)(b * KT + k) * (uint32_t)a.HoWo + hw) * 2;
      dy[q] = load_scalar<__bf16>(offr, ob);
      dx[q] = load_scalar<__bf16>(offr, ob + (uint32_t)a.HoWo * 2);
      mk[q] = has_mask ? load_scalar<__bf16>(mskr, mb) : 1.0f;
    }
  }
  u32x4 w0v[FPT];
#pragma unroll
  for (int u = 0; u < FPT; ++u) w0v[u] = fill_load(0, u);

  // is every inside corner of every tap of this tile in the window?  (each
  // thread checks its corner row of its pixel; one vote)
  // the point of this thread's q-th tap k = 2q + c_k0
  auto point = [&](int q) {
    const int k = 2 * q + c_k0;
    return sample_point((float)(c_ho - a.ph + k / kWinK), (float)(c_wo - a.pw + k % kWinK), dy[q],
                        dx[q]);
  };
  bool tile_far;
  {
    bool far = false;
#pragma unroll
    for (int q = 0; q < KPT; ++q) {
      if (2 * q + c_k0 >= KT) break;
      const CornerRow cr = corner_row(point(q), c_pair, a.H, a.W);
      const int win_y = cr.ry - wy0, win_x = cr.ix - wx0;
      const bool row_in = (uint32_t)win_y < (uint32_t)WH;
      far |= c_in && cr.ok0 && !(row_in && (uint32_t)win_x < (uint32_t)WW);
      far |= c_in && cr.ok1 && !(row_in && (uint32_t)(win_x + 1) < (uint32_t)WW);
    }
    tile_far = __syncthreads_or(far) != 0;
  }

  typedef float f32x2 __attribute__((ext_vector_type(2)));
  // corner-table entries of tap k: window offsets (WIN) or offsets in x
  auto build_tables = [&](auto from_win) {
    constexpr bool WIN = decltype(from_win)::value;
#pragma unroll
    for (int q = 0; q < KPT; ++q) {
      const int k = 2 * q + c_k0;
      if (k >= KT) break;
      const SamplePoint p = point(q);
      const CornerRow cr = corner_row(p, c_pair, a.H, a.W);
      const float wy = c_pair ? p.ly : 1.0f - p.ly;
      const bool ok0 = c_in && cr.ok0;
      const bool ok1 = c_in && cr.ok1;
      const float w0 = static_cast<float>(static_cast<__bf16>(wy * (1.0f - p.lx) * mk[q]));
      const float w1 = static_cast<float>(static_cast<__bf16>(wy * p.lx * mk[q]));
      const f32x2 w2 = {ok0 ? w0 : 0.0f, ok1 ? w1 : 0.0f};
      const uint32_t base = (uint32_t)((b * a.H + cr.ry) * a.W + cr.ix) * row_bytes;
      const u32x2 g2 = {ok0 ? base : kNoCorner, ok1 ? base + row_bytes : kNoCorner};
      u32x2 o2 = g2;
      if constexpr (WIN) {
        // an inside corner of a window tile lies in the window (the vote)
        const uint32_t lw = (uint32_t)((cr.ry - wy0) * WW + (cr.ix - wx0)) * ROWB;
        o2 = u32x2{ok0 ? lw : ZERO_ROW, ok1 ? lw + ROWB : ZERO_ROW};
      }
      if (a.dbg_corner != nullptr && c_in) {
        const size_t e = (((size_t)b * KT + k) * a.HoWo + c_hw) * 4 + 2 * c_pair;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          a.dbg_corner[e + h] = g2[h] == kNoCorner ? -1 : (int32_t)(g2[h] / row_bytes);
          a.dbg_weight[e + h] = w2[h];
        }
      }
      // w2 holds bf16 values: their upper halves are exact (the elements are
      // read by value: a bit cast of a vector element would read element 0)
      const float wa = w2[0], wb = w2[1];
      reinterpret_cast<uint32_t*>(&Cw[k][c_px])[c_pair] =
          (__float_as_uint(wa) >> 16) | (__float_as_uint(wb) & 0xffff0000u);
      *reinterpret_cast<u32x2*>(reinterpret_cast<uint32_t*>(&Cx[k][c_px]) + 2 * c_pair) = o2;
    }
  };

  // ---- (b) blend: thread -> pixel pp = tid >> 2, 16-byte slice sl = tid & 3
  // of the chunk's 32 channels.
  const int sl = tid & 3;
  const int pp = tid >> 2;
  // Column tile: row r (pixel), 16-byte chunk k (channels 8k .. 8k+7) at
  // r * 64 + 16 * (k ^ ((r >> 2) & 3)): the 16 rows of an MFMA fragment read
  // and the 4 rows of a blend store each cover all 64 banks once.
  auto a_off = [](int r, int k) { return r * ROWB + 16 * (k ^ ((r >> 2) & 3)); };
  // channel h (0: low, 1: high half) of dword v0 of corner (a, 0) and of v1
  // of corner (a, 1), as one bf16 pair; its weighted sum with the corner
  // row's weight pair w added to acc
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  auto pair_dot = [](uint32_t v0, uint32_t v1, int h, uint32_t w, float acc) {
    // v_perm_b32 numbers the bytes of its second operand 0..3, of its first 4..7
    const uint32_t pr = __builtin_amdgcn_perm(v1, v0, h ? 0x07060302u : 0x05040100u);
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pr),
                                          __builtin_bit_cast(bf16x2, w), acc, false);
  };
  // the same with a zero accumulator, as one VOP3P instruction: the
  // builtin's zero becomes a register move plus the accumulating VOP2 form,
  // one VALU instruction more per corner row 0 dot
  auto pair_dot0 = [](uint32_t v0, uint32_t v1, int h, uint32_t w) {
    const uint32_t pr = __builtin_amdgcn_perm(v1, v0, h ? 0x07060302u : 0x05040100u);
    float r;
    asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(r) : "v"(pr), "v"(w));
    return r;
  };

  // ---- (c) MFMA: lane group g supplies channels 8g .. 8g+7 of the block.
  const int rl = lane & 15;
  const int g = lane >> 4;
  f32x4 acc[MT][NTW];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto a_frag = [&](const char* A, int mt) {
    return *reinterpret_cast<const u32x4*>(A + a_off(mt * 16 + rl, g));
  };
  // weight fragment nt of block (chunk c, tap t): a uniform base and this
  // lane's offset
  auto b_load = [&](int c, int t, int nt) {
    const u32x4* blk = wtile + (size_t)((t * a.nchunk + (c >> 1)) * 2 + (c & 1)) * 1024;
    return blk[wlane + nt * 64];
  };

  // The whole tile from the window (WIN) or, when some corner of the tile
  // lies beyond it, from memory.
  auto run = [&](auto from_win) {
    constexpr bool WIN = decltype(from_win)::value;
    build_tables(from_win);
    if constexpr (WIN) {
#pragma unroll
      for (int u = 0; u < FPT; ++u) fill_store(0, u, w0v[u]);
    }
    __syncthreads();  // tables and the first window visible

    // one corner of block s (chunk c) for this thread's slice, from its
    // table entry
    auto fetch = [&](uint32_t ent, int c) {
      if constexpr (WIN)
        return *reinterpret_cast<const u32x4*>(Win[c & 1] + ent + sl * 16);
      else
        return load16(xr, ent + (uint32_t)(c * CB + sl * 8) * 2);
    };

    u32x4 gv[4];       // corner vectors of the next block
    u32x4 bw[3][NTW];  // weight fragments, ring over the taps (3 divides KT)
    u32x4 af[AFD + 1];
    u32x4 fv[2];       // window loads in flight, by load index parity

    // ---- prologue: block 0 blended into As[0]; the corners of block 1, the
    // weights of blocks 0 and 1 and the first two window loads of chunk 1 in
    // flight
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      bw[0][nt] = b_load(0, 0, nt);
      bw[1][nt] = b_load(0, 1, nt);
    }
    {
      const u32x4 ent = Cx[0][pp];
      const u32x2 w = Cw[0][pp];
      u32x4 v[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) v[c] = fetch(ent[c], 0);
      float r[8];
#pragma unroll
      for (int cp = 0; cp < 2; ++cp)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          r[e] = pair_dot(v[2 * cp][e / 2], v[2 * cp + 1][e / 2], e & 1, w[cp],
                          cp == 0 ? 0.0f : r[e]);
      bf16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = static_cast<__bf16>(r[e]);
      *reinterpret_cast<u32x4*>(&As[0][a_off(pp, sl)]) = __builtin_bit_cast(u32x4, o);
    }
    {
      const u32x4 ent = Cx[1][pp];
#pragma unroll
      for (int c = 0; c < 4; ++c) gv[c] = fetch(ent[c], 0);
    }
    if (WIN && nch > 1) {
      fv[0] = fill_load(1, 0);
      fv[1] = fill_load(1, 1);
    }

    // ---- step (chunk c, tap t) = block s = KT c + t.  Slot j holds MFMA
    // (mt, nt) = (j / 2, j % 2) and beside it: blend unit (corner row j / 8,
    // channel j % 8) of block s+1; after a corner row's last unit the fetch of
    // its two corners for block s+2; after the last unit the bf16 rounding
    // and the column-tile write; column-tile fragments AFD tiles ahead; the
    // weight fragments of block s+2 in the first two slots (ring slot
    // (s + 2) % 3 = (s - 1) % 3, free since block s-1's MFMAs).
    // Window of chunk c+1: load u is issued at step s = KT (c + 1) + u - KT - 2
    // (two steps before it is written) and written at step (c, u), u < FPT,
    // before that step's barrier: after the last fetch from the buffer (chunk
    // c - 1, at step (c - 1, KT - 3)) and before the first fetch of chunk c+1
    // (at step (c, KT - 2)).
    for (int c = 0; c < nch; ++c) {
      static_for<KT>([&](auto T) {
        constexpr int t = decltype(T)::value;
        constexpr int t1 = (t + 1) % KT, t2 = (t + 2) % KT;  // taps of blocks s+1, s+2
        constexpr int fu = (t + 2) % KT;                      // window load issued here
        const int par = (c + t) & 1;  // s & 1 (KT is odd)
        const char* A = As[par];
        char* An = As[par ^ 1];
        const int c2 = t + 2 >= KT && c + 1 < nch ? c + 1 : c;  // chunk of s+2, clamped at the end

        if constexpr (WIN && t < FPT) {
          if (c + 1 < nch) fill_store((c + 1) & 1, t, fv[t & 1]);
        }
        __syncthreads();  // block s in As[par]; every wave done with block s-1
        if constexpr (WIN && fu < FPT) {
          const int cf = t + 2 >= KT ? c + 2 : c + 1;
          if (cf < nch) fv[fu & 1] = fill_load(cf, fu);
        }

#pragma unroll
        for (int u = 0; u < AFD; ++u) af[u] = a_frag(A, u);
        const u32x2 wt = Cw[t1][pp];
        const u32x4 en = Cx[t2][pp];
        float r[8];
        __builtin_amdgcn_sched_barrier(0);

        static_for<NSL>([&](auto J) {
          constexpr int j = decltype(J)::value;
          constexpr int mt = j / NTW, nt = j % NTW;
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, af[mt % (AFD + 1)]),
              __builtin_bit_cast(bf16x8, bw[t % 3][nt]), acc[mt][nt], 0, 0, 0);
          if constexpr (nt == 0 && mt + AFD < MT) af[(mt + AFD) % (AFD + 1)] = a_frag(A, mt + AFD);
          if constexpr (mt == 0) bw[t2 % 3][nt] = b_load(c2, t2, nt);
          // blend unit: corner row cp, channel e = 2 * (dword) + (half)
          constexpr int cp = j / 8, e = j % 8;
          if constexpr (cp == 0)
            r[e] = pair_dot0(gv[0][e / 2], gv[1][e / 2], e & 1, wt[0]);
          else
            r[e] = pair_dot(gv[2][e / 2], gv[3][e / 2], e & 1, wt[1], r[e]);
          if constexpr (e == 7) {
            gv[2 * cp] = fetch(en[2 * cp], c2);
            gv[2 * cp + 1] = fetch(en[2 * cp + 1], c2);
          }
          if constexpr (j == NSL - 1) {
            bf16x8 o;
#pragma unroll
            for (int q = 0; q < 8; ++q) o[q] = static_cast<__bf16>(r[q]);
            *reinterpret_cast<u32x4*>(&An[a_off(pp, sl)]) = __builtin_bit_cast(u32x4, o);
          }
          __builtin_amdgcn_sched_barrier(0);
        });
      });
    }
  };
  if (tile_far) run(std::integral_constant<bool, false>{});
  else run(std::integral_constant<bool, true>{});

  // ---- epilogue: + bias, fp32 store straight from the accumulators.
  // MFMA 16x16 result layout: lane l, register r -> row 4(l/16) + r,
  // column l % 16; 16-row tile mt = tile row mt (16 pixels).
  const __bf16* biasp = static_cast<const __bf16*>(a.bias);
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    const int o = otile * NO + wave * (NTW * 16) + nt * 16 + rl;
    if (o >= a.O) continue;
    const float bo = biasp ? static_cast<float>(biasp[o]) : 0.0f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int ho = ty0 + mt, wo = tx0 + 4 * g;
      if (ho >= a.Ho || wo >= a.Wo) continue;
      const f32x4 v = acc[mt][nt] + bo;
      const int hw = ho * a.Wo + wo;
      if constexpr (!NHWC) {
        float* dst = a.out + ((size_t)b * a.O + o) * a.HoWo + hw;
        if (a.vec_store && wo + 3 < a.Wo) {
          *reinterpret_cast<f32x4*>(dst) = v;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (wo + e < a.Wo) dst[e] = v[e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (wo + e < a.Wo) a.out[((size_t)b * a.HoWo + hw + e) * a.O + o] = v[e];
      }
    }
  }
}

bool bf16win_supported(const KernelConfig& kc) {
  return kc.bf16 && kc.kind == 4 && kc.CB == 64 && kc.NO == 256 && kc.M == kWinTH * kWinTW;
}

bool bf16win_fits(int kh, int kw, int C) {
  return kh == kWinK && kw == kWinK && C % 64 == 0;
}

int bf16win_tiles(int rows, int Wo, int& tiles_x) {
  tiles_x = (Wo + kWinTW - 1) / kWinTW;
  return ((rows + kWinTH - 1) / kWinTH) * tiles_x;
}

namespace {
template <class Src>
hipError_t launch_bf16win_src(const KernelConfig& kc, const Src& src, int64_t nblk,
                              hipStream_t s) {
  if (nblk <= 0) return hipSuccess;
  if (nblk > 0x7fffffff || !bf16win_supported(kc)) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)nblk), block(512);
  if (kc.nhwc) hipLaunchKernelGGL((fused_bf16win_kernel<true, Src>), grid, block, 0, s, src);
  else hipLaunchKernelGGL((fused_bf16win_kernel<false, Src>), grid, block, 0, s, src);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_fused_bf16win(const KernelConfig& kc, const FusedArgs& a, hipStream_t s) {
  if (!bf16win_fits(a.kh, a.kw, a.C) || a.K != kWinK * kWinK) return hipErrorInvalidValue;
  return launch_bf16win_src(kc, a, (int64_t)a.B * kc.tiles_per_img * kc.n_otiles, s);
}

hipError_t launch_fused_bf16win_multi(const KernelConfig& kc, const MultiArgs& m, hipStream_t s) {
  for (int i = 0; i < m.n; ++i)
    if (!bf16win_fits(m.a[i].kh, m.a[i].kw, m.a[i].C) || m.a[i].K != kWinK * kWinK)
      return hipErrorInvalidValue;
  return launch_bf16win_src(kc, m, m.start[m.n], s);
}

}  // namespace dcn
