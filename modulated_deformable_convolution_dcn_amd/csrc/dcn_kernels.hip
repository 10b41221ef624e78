// dcn_kernels.hip -- gfx950 kernels of the modulated deformable conv2d forward.
//
// The operator (page 1, "deform_conv.py": module docstring and
// deform_conv2d_gather; page 5, deformops README, "Deformable convolution"):
//   out[b,o,h,w] = bias[o] + sum_{k=(i,j)} sum_c weight[o,c,i,j] *
//                  mask[b,k,h,w] * bilinear(x[b,:,:,c], h-ph+i+dy, w-pw+j+dx)
// with corners outside the image counting as zero.
//
// Page 1 evaluates it as GATHER -> elementwise bilinear weights -> one matmul
// over a materialised [pixels, taps*channels] column matrix; page 5 notes the
// fused form in which that column matrix never exists.  Here one workgroup
// owns M output pixels x NO output channels and walks the (tap, channel
// block) axis.  Per step it:
//   (a) forms the sampling point, the four corner weights (bilinear weight x
//       validity x mask) and the four corner byte offsets for each of its M
//       pixels once per tap (shared through LDS);
//   (b) fetches each corner's 16-byte channel slice from the NHWC input with
//       buffer loads (a corner outside the image is a load past the buffer's
//       end, which returns zero without a memory access), blends the four
//       corners in registers and writes the blended row into an LDS column
//       tile [M x CB] -- the only place the column matrix ever exists;
//   (c) contracts that tile against the matching [CB x NO] block of the
//       packed weight with MFMA (fp32: v_mfma_f32_16x16x4_f32; bf16:
//       v_mfma_f32_16x16x32_bf16, fp32 accumulate), while the next step's
//       corner loads and weight block are already in flight;
// and finally adds the bias and writes NCHW or NHWC fp32 output.

#include <type_traits>

#include "dcn_device.h"
#include "dcn_launch.h"

namespace dcn {

template <class T, int M, int CB, int NO, int WM, int WN, bool NHWC>
__global__ __launch_bounds__(256) void fused_kernel(FusedArgs a) {
  constexpr int E = sizeof(T);
  constexpr int VEC = Ops<T>::VEC;       // elements per 16-byte fragment
  constexpr int LPR = CB / VEC;          // lanes that gather one pixel's CB channels
  constexpr int PPP = 256 / LPR;         // pixels per gather pass
  constexpr int NPASS = M / PPP;         // gather passes per k-block
  constexpr int AST = CB + VEC;          // LDS column-tile row stride (one pad fragment)
  constexpr int A_ELEMS = M * AST;
  constexpr int B_ELEMS = CB * NO;
  constexpr int B_PIECES = B_ELEMS * E / 16;
  constexpr int B_PER_T = (B_PIECES + 255) / 256;
  constexpr int R = CB / 4 / VEC;        // fragment reads per k-slot group per k-block
  constexpr int WROWS = M / WM, WCOLS = NO / WN;
  constexpr int MT = WROWS / 16, NT = WCOLS / 16;
  constexpr int NSLOT = 3;               // coefficient ring (taps in flight)
  static_assert(LPR >= 1 && 256 % LPR == 0 && NPASS >= 1 && M % PPP == 0, "gather shape");
  static_assert(R >= 1 && CB % (4 * VEC) == 0, "k-block shape");
  static_assert(WM * WN == 4 && MT >= 1 && NT >= 1, "wave tiling");
  static_assert(M % 64 == 0, "one lane per pixel in the coefficient stage");

  __shared__ __attribute__((aligned(16))) T As[2][A_ELEMS];
  __shared__ __attribute__((aligned(16))) T Bs[2][B_ELEMS];
  __shared__ f32x4 Cw[NSLOT][M];   // corner weights: bilinear x validity x mask
  __shared__ u32x4 Co[NSLOT][M];   // corner byte offsets in x (kNoCorner: outside)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  // ---- which tile: (image b, pixel tile, output-channel tile)
  const int logical = xcd_logical_block(blockIdx.x, gridDim.x);
  const int otile = logical % a.n_otiles;
  const int t2 = logical / a.n_otiles;
  const int tile = t2 % a.tiles_per_img;
  const int b = t2 / a.tiles_per_img;
  const int hw0 = tile * M;

  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, a.x_bytes);
  const T* wtiles = static_cast<const T*>(a.wpack) +
                    (size_t)otile * a.K * a.nchunk * B_ELEMS;
  const T* offp = static_cast<const T*>(a.offset);
  const T* maskp = static_cast<const T*>(a.mask);
  const uint32_t row_bytes = (uint32_t)a.C * E;
  const int NKB = a.K * a.nchunk;

  // ---- (a) sampling point -> corner weights and offsets, one tap, M pixels.
  // Split in two: the offset/mask loads are issued at the top of a step and
  // consumed after its MFMAs.  vmcnt counts in order, and a load under a
  // data-dependent branch makes the compiler drain the counter, so these are
  // branch-free buffer loads (a NULL mask is a zero-size buffer that reads as
  // 0, replaced by 1).  Thread (wave w, lane l) owns pixel l (+64 r) and
  // corner w, so the four waves share the work evenly.
  constexpr int CPL = M / 64;  // pixels per lane in the coefficient stage
  const bool has_mask = maskp != nullptr;
  const __amdgpu_buffer_rsrc_t offr = make_rsrc(offp, a.offset_bytes);
  const __amdgpu_buffer_rsrc_t mskr = make_rsrc(has_mask ? (const void*)maskp : (const void*)offp,
                                                has_mask ? a.mask_bytes : 0u);
  const int corner = wave;  // (a, b) = (corner >> 1, corner & 1)
  float c_dy[CPL], c_dx[CPL], c_mk[CPL];
  auto coef_load = [&](int kt) {
#pragma unroll
    for (int r = 0; r < CPL; ++r) {
      const uint32_t hw = (uint32_t)(hw0 + r * 64 + lane);
      const uint32_t ob = ((uint32_t)(b * 2 * a.K + 2 * kt) * (uint32_t)a.HoWo + hw) * E;
      const uint32_t mb = ((uint32_t)(b * a.K + kt) * (uint32_t)a.HoWo + hw) * E;
      c_dy[r] = load_scalar<T>(offr, ob);
      c_dx[r] = load_scalar<T>(offr, ob + (uint32_t)a.HoWo * E);
      c_mk[r] = load_scalar<T>(mskr, mb);
    }
  };
  auto coef_finish = [&](int kt) {
    const int slot = kt % NSLOT;
    const int i = kt / a.kw;
    const int j = kt - i * a.kw;
#pragma unroll
    for (int r = 0; r < CPL; ++r) {
      const int m = r * 64 + lane;
      const int hw = hw0 + m;
      const int ho = hw / a.Wo;
      const int wo = hw - ho * a.Wo;
      const int ca = corner >> 1, cb = corner & 1;
      const SamplePoint p =
          sample_point((float)(ho - a.ph + i), (float)(wo - a.pw + j), c_dy[r], c_dx[r]);
      const CornerRow cr = corner_row(p, ca, a.H, a.W);
      const float wy = ca ? p.ly : 1.0f - p.ly;
      const float wx = cb ? p.lx : 1.0f - p.lx;
      const float mk = has_mask ? c_mk[r] : 1.0f;
      const bool ok = (hw < a.HoWo) && (cb ? cr.ok1 : cr.ok0);
      const float cw = ok ? wy * wx * mk : 0.0f;
      const uint32_t co = ok ? (uint32_t)((b * a.H + cr.ry) * a.W + cr.ix + cb) * row_bytes
                             : kNoCorner;
      Cw[slot][m][corner] = cw;
      Co[slot][m][corner] = co;
      if (a.dbg_corner != nullptr && hw < a.HoWo) {
        const size_t e = (((size_t)b * a.K + kt) * a.HoWo + hw) * 4 + corner;
        a.dbg_corner[e] = co == kNoCorner ? -1 : (int32_t)(co / row_bytes);
        a.dbg_weight[e] = cw;
      }
    }
  };

  // ---- (b) corner loads into one of two register sets: the loads of block
  // kb+2 are in flight while block kb+1 (loaded a whole step earlier) is
  // blended and block kb is multiplied.
  const int li = tid % LPR;  // which 16-byte slice of the channel block
  const int pr = tid / LPR;  // which pixel of the pass
  u32x4 gv[2][NPASS][4];
  auto issue_gather = [&](int kb, auto set_tag) {
    constexpr int S = decltype(set_tag)::value;
    const int kt = kb / a.nchunk;
    const int cc = kb - kt * a.nchunk;
    const int ch = cc * CB + li * VEC;
    const bool chan_ok = ch < a.C;
    const uint32_t cbyte = (uint32_t)ch * E;
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
      const u32x4 off = Co[kt % NSLOT][ps * PPP + pr];
#pragma unroll
      for (int c = 0; c < 4; ++c)
        gv[S][ps][c] = load16(xr, chan_ok ? off[c] + cbyte : kNoCorner);
    }
  };
  auto finish_gather = [&](int kb, T* A, auto set_tag) {
    constexpr int S = decltype(set_tag)::value;
    const int kt = kb / a.nchunk;
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
      const f32x4 w = Cw[kt % NSLOT][ps * PPP + pr];
      const u32x4 r = Ops<T>::blend(w, gv[S][ps][0], gv[S][ps][1], gv[S][ps][2], gv[S][ps][3]);
      *reinterpret_cast<u32x4*>(&A[(ps * PPP + pr) * AST + li * VEC]) = r;
    }
  };

  // ---- weight block kb (contiguous in the packed layout) into registers
  u32x4 bq[B_PER_T];
  auto issue_b = [&](int kb) {
    const u32x4* src = reinterpret_cast<const u32x4*>(wtiles + (size_t)kb * B_ELEMS);
#pragma unroll
    for (int r = 0; r < B_PER_T; ++r) {
      const int idx = tid + r * 256;
      if (B_PIECES % 256 == 0 || idx < B_PIECES) bq[r] = src[idx];
    }
  };
  auto store_b = [&](T* Bt) {
#pragma unroll
    for (int r = 0; r < B_PER_T; ++r) {
      const int idx = tid + r * 256;
      if (B_PIECES % 256 == 0 || idx < B_PIECES) reinterpret_cast<u32x4*>(Bt)[idx] = bq[r];
    }
  };

  // ---- (c) MFMA over one k-block.  Channel order inside the block: k-slot
  // group g (lane / 16) owns channels [g*CB/4, (g+1)*CB/4); fragment read q
  // of a lane holds channels g*CB/4 + q*VEC + [0, VEC).  The packed weight
  // uses the same order, so any assignment is a permutation of the sum.
  // Fragments for read q+1 are fetched before the MFMAs of read q issue.
  const int rl = lane & 15;
  const int g = lane >> 4;
  const int wm = wave / WN, wn = wave % WN;
  f32x4 acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto mfma_block = [&](const T* A, const T* Bt) {
    u32x4 af[2][MT], bf[2][NT];
    auto fetch = [&](int q, int s) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        af[s][mt] = lds16(&A[(wm * WROWS + mt * 16 + rl) * AST + g * (CB / 4) + q * VEC]);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        bf[s][nt] = lds16(&Bt[((g * R + q) * NO + wn * WCOLS + nt * 16 + rl) * VEC]);
    };
    fetch(0, 0);
#pragma unroll
    for (int q = 0; q < R; ++q) {
      const int s = q & 1;
      if (q + 1 < R) fetch(q + 1, s ^ 1);
      if constexpr (sizeof(T) == 4) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
              acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                  __uint_as_float(af[s][mt][e]), __uint_as_float(bf[s][nt][e]), acc[mt][nt], 0,
                  0, 0);
      } else {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, af[s][mt]), __builtin_bit_cast(bf16x8, bf[s][nt]),
                acc[mt][nt], 0, 0, 0);
      }
    }
  };

  // ---- pipeline.  Step i (one barrier): load the offsets/mask of the tap
  // whose coefficients this step may produce, the weight block of i+1 and
  // the corners of i+2 -- in that order, so each consumer waits only for
  // what is older than the loads still in flight -- then MFMA block i, then
  // write coefficients (tap t is produced in step t*nchunk - 3), blend block
  // i+1 into the idle column buffer and store weight block i+1.  Every load
  // sequence is branch-free; past the end the last block is re-loaded into
  // the idle buffers instead of branching.
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  const int k1 = a.K > 1 ? 1 : 0;
  coef_load(0);
  coef_finish(0);
  coef_load(k1);
  coef_finish(k1);
  __syncthreads();
  issue_b(0);
  issue_gather(0, S0{});
  issue_gather(NKB > 1 ? 1 : 0, S1{});
  __syncthreads();  // every wave has read the offsets of blocks 0 and 1
  if (a.nchunk == 1 && a.K > 2) {
    coef_load(2);
    coef_finish(2);
  }
  finish_gather(0, As[0], S0{});
  store_b(Bs[0]);

  auto step = [&](int i, auto par) {
    constexpr int P = decltype(par)::value;  // i & 1: buffers and register set
    __syncthreads();  // block i is in LDS; every wave is done with block i-1
    const int tc = (i + 3) / a.nchunk;
    const bool coef_due = (i + 3) - tc * a.nchunk == 0 && tc < a.K;
    coef_load(tc < a.K ? tc : a.K - 1);
    issue_b(i + 1 < NKB ? i + 1 : NKB - 1);
    issue_gather(i + 2 < NKB ? i + 2 : NKB - 1, std::integral_constant<int, P>{});
    __builtin_amdgcn_sched_barrier(0);
    mfma_block(As[P], Bs[P]);
    __builtin_amdgcn_sched_barrier(0);
    if (coef_due) coef_finish(tc);
    finish_gather(i + 1 < NKB ? i + 1 : NKB - 1, As[P ^ 1], std::integral_constant<int, P ^ 1>{});
    store_b(Bs[P ^ 1]);
  };
  int i = 0;
  for (; i + 1 < NKB; i += 2) {
    step(i, S0{});
    step(i + 1, S1{});
  }
  if (i < NKB) step(i, S0{});

  // ---- epilogue: + bias, fp32 store.  MFMA 16x16 result layout: lane l,
  // register r holds row 4*(l/16) + r, column l % 16.
  const T* biasp = static_cast<const T*>(a.bias);
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int o = otile * NO + wn * WCOLS + nt * 16 + rl;
    if (o >= a.O) continue;
    const float bo = biasp ? to_f32<T>(biasp[o]) : 0.0f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int hw_r0 = hw0 + wm * WROWS + mt * 16 + g * 4;
      f32x4 v = acc[mt][nt];
      v += bo;
      if constexpr (NHWC) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (hw_r0 + r < a.HoWo) a.out[((size_t)b * a.HoWo + hw_r0 + r) * a.O + o] = v[r];
      } else {
        float* dst = a.out + ((size_t)b * a.O + o) * a.HoWo + hw_r0;
        if (a.vec_store && hw_r0 + 3 < a.HoWo) {
          *reinterpret_cast<f32x4*>(dst) = v;
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (hw_r0 + r < a.HoWo) dst[r] = v[r];
        }
      }
    }
  }
}

// ---------------------------------------------------------------- packing
// The packed weight is page 1's matrix (rows (i, j, c), columns o: it
// reorders weight[o, c, i, j] that way before its one matmul) cut into the
// kernels' [CB x NO] k-blocks, zero-padded, ordered
//   [o_tile][tap][c_chunk][block]
// where the block layout serves one kernel's fragment reads:
//   layout 0 (shared column tile): [CB/VEC][NO][VEC] -- each lane's VEC
//            consecutive channels of one output channel are contiguous;
//   layout 1 (k split over waves, CB = 64, VEC = 4): [wave][NO/16][g][16][4]
//            = channel 16*wave + 4g + e, output 16*nt + col -- one wave's MFMA
//            B fragments for a block are one contiguous run per nt;
//   layout 2 (32 x 32 per wave, CB = 64, VEC = 4): [half][NO/32][q][lane][4]
//            = channel 32*half + 16*(lane/32) + 4q + e, output 32n + lane%32
//            (32x32x2 MFMA B fragments) -- one 1 KB run per (n, q) for the
//            wave owning that channel half;
//   layout 3 (bf16 16x16x32 fragments, VEC = 8): [CB/32][NO/16][g][16][8]
//            = channel 32q + 8g + e, output 16*nt + col -- fragment (q, nt)
//            is one 1 KB run in lane order.
// The (channel c_in, output o_in) of element `in` of one packed block: the
// layouts above read backwards.  In every layout the lowest 16 / sizeof(T)
// packed elements of a 16-byte run are consecutive channels of one output.
__device__ __forceinline__ void packed_source(int in, int layout, int NO, int VEC, int& c_in,
                                              int& o_in) {
  const int NT = NO >> 4;
  switch (layout) {
    case 0:
      c_in = ((in / VEC) / NO) * VEC + in % VEC;
      o_in = (in / VEC) % NO;
      return;
    case 1: {
      const int t = in >> 8;
      c_in = (t / NT) * 16 + ((in >> 6) & 3) * 4 + (in & 3);
      o_in = (t % NT) * 16 + ((in >> 2) & 15);
      return;
    }
    case 2: {
      const int ln = (in >> 2) & 63, t = in >> 10, NN = NO >> 5;
      c_in = (t / NN) * 32 + (ln >> 5) * 16 + ((in >> 8) & 3) * 4 + (in & 3);
      o_in = (t % NN) * 32 + (ln & 31);
      return;
    }
    default: {
      const int t = in >> 9;
      c_in = (t / NT) * 32 + ((in >> 7) & 3) * 8 + (in & 7);
      o_in = (t % NT) * 16 + ((in >> 3) & 15);
      return;
    }
  }
}

// One 16-byte run of the packed weight per thread: a whole 16-byte write,
// its elements read from weight [O][C][kh][kw].  Consecutive threads take
// the same run position in the blocks of consecutive taps, so their reads of
// weight[o, c, tap] are consecutive words.  Padding channels and outputs are
// written as zeros.
template <class T>
__global__ __launch_bounds__(256) void pack_kernel(const T* __restrict__ w, T* __restrict__ wp,
                                                   int O, int C, int K, int CB, int NO, int VEC,
                                                   int nchunk, int layout, int64_t nruns) {
  constexpr int G = 16 / (int)sizeof(T);
  const int rpb = CB * NO / G;  // runs per block
  for (int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x; r < nruns;
       r += (int64_t)gridDim.x * 256) {
    // r = ((otile * nchunk + chunk) * rpb + run) * K + tap
    const int tap = (int)(r % K);
    const int64_t r2 = r / K;
    const int run = (int)(r2 % rpb);
    const int64_t oc = r2 / rpb;
    const int chunk = (int)(oc % nchunk), otile = (int)(oc / nchunk);
    const int64_t block = ((int64_t)otile * K + tap) * nchunk + chunk;  // [otile][tap][chunk]
    const int64_t idx = block * CB * NO + (int64_t)run * G;
    int c_in, o_in;
    packed_source(run * G, layout, NO, VEC, c_in, o_in);
    const int o = otile * NO + o_in, c0 = chunk * CB + c_in;
    T v[G];
#pragma unroll
    for (int e = 0; e < G; ++e) {
      const int c = c0 + e;
      v[e] = o < O && c < C ? w[((int64_t)o * C + c) * K + tap] : static_cast<T>(0.0f);
    }
    *reinterpret_cast<u32x4*>(wp + idx) = *reinterpret_cast<const u32x4*>(v);
  }
}

// ---------------------------------------------------------------- layout
// NCHW -> NHWC for callers that hold torchvision-layout input (page 5's
// drop-in takes NCHW).  One workgroup moves a 64-channel x 64-pixel tile
// through LDS.  Interior tiles (whole tile inside, pixel and channel counts
// multiples of the 16-byte vector) use 16-byte accesses on both sides:
// each thread reads VEC consecutive pixels of one channel and writes VEC
// consecutive channels of one pixel; edge tiles take the element-wise path.
// Element-exact: a pure copy.
template <class T>
__global__ __launch_bounds__(256) void nchw_to_nhwc_kernel(const T* __restrict__ src,
                                                           T* __restrict__ dst, int C, int HW,
                                                           int c_tiles, int p_tiles) {
  constexpr int VEC = 16 / sizeof(T);
  constexpr int PITCH = 64 + VEC;  // row pitch (elements): rows start 16 B apart in the banks
  __shared__ __attribute__((aligned(16))) T tile[64 * PITCH];
  const int t = blockIdx.x;
  const int pt = t % p_tiles;
  const int ct = (t / p_tiles) % c_tiles;
  const int b = t / (p_tiles * c_tiles);
  const int c0 = ct * 64, p0 = pt * 64;
  const T* s = src + (size_t)b * C * HW;
  T* d = dst + (size_t)b * HW * C;
  const int tid = threadIdx.x;
  const bool vec = c0 + 64 <= C && p0 + 64 <= HW && C % VEC == 0 && HW % VEC == 0;
  if (vec) {
    constexpr int LPR = 64 / VEC;      // lanes per 64-element row
    constexpr int RPP = 256 / LPR;     // rows per pass
    const int li = tid % LPR, r0 = tid / LPR;
#pragma unroll
    for (int r = r0; r < 64; r += RPP)
      *reinterpret_cast<u32x4*>(&tile[r * PITCH + li * VEC]) =
          *reinterpret_cast<const u32x4*>(s + (size_t)(c0 + r) * HW + p0 + li * VEC);
    __syncthreads();
#pragma unroll
    for (int r = r0; r < 64; r += RPP) {  // r: pixel, li: channel group
      T v[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) v[e] = tile[(li * VEC + e) * PITCH + r];
      *reinterpret_cast<u32x4*>(d + (size_t)(p0 + r) * C + c0 + li * VEC) =
          *reinterpret_cast<const u32x4*>(v);
    }
    return;
  }
  const int lane = tid & 63, row = tid >> 6;
  for (int r = row; r < 64; r += 4) {
    const int c = c0 + r, p = p0 + lane;
    if (c < C && p < HW) tile[r * PITCH + lane] = s[(size_t)c * HW + p];
  }
  __syncthreads();
  for (int r = row; r < 64; r += 4) {
    const int p = p0 + r, c = c0 + lane;
    if (c < C && p < HW) d[(size_t)p * C + c] = tile[lane * PITCH + r];
  }
}

hipError_t launch_nchw_to_nhwc(int bf16, const void* src, void* dst, int B, int C, int HW,
                               hipStream_t s) {
  const int c_tiles = (C + 63) / 64, p_tiles = (HW + 63) / 64;
  const int64_t nblk = (int64_t)B * c_tiles * p_tiles;
  if (nblk <= 0) return hipSuccess;
  if (nblk > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (bf16)
    hipLaunchKernelGGL(nchw_to_nhwc_kernel<__bf16>, dim3((unsigned)nblk), dim3(256), 0, s,
                       static_cast<const __bf16*>(src), static_cast<__bf16*>(dst), C, HW, c_tiles,
                       p_tiles);
  else
    hipLaunchKernelGGL(nchw_to_nhwc_kernel<float>, dim3((unsigned)nblk), dim3(256), 0, s,
                       static_cast<const float*>(src), static_cast<float*>(dst), C, HW, c_tiles,
                       p_tiles);
  return hipGetLastError();
}

// ---------------------------------------------------------------- corners
template <class T>
__global__ __launch_bounds__(256) void coords_kernel(const T* __restrict__ offset,
                                                     int32_t* __restrict__ y0x0,
                                                     uint8_t* __restrict__ valid4, int B, int K,
                                                     int kw, int Ho, int Wo, int ph, int pw,
                                                     int H, int W) {
  const int HoWo = Ho * Wo;
  const int64_t total = (int64_t)B * K * HoWo;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * 256) {
    const int hw = (int)(e % HoWo);
    const int k = (int)((e / HoWo) % K);
    const int b = (int)(e / ((int64_t)HoWo * K));
    const int ho = hw / Wo, wo = hw % Wo;
    const int i = k / kw, j = k % kw;
    const int64_t ob = ((int64_t)b * 2 * K + 2 * k) * HoWo + hw;
    const TapCorners t = tap_corners((float)(ho - ph + i), (float)(wo - pw + j),
                                     to_f32<T>(offset[ob]), to_f32<T>(offset[ob + HoWo]), H, W);
    y0x0[2 * e] = sat_i32(t.p.fy);
    y0x0[2 * e + 1] = sat_i32(t.p.fx);
    valid4[e] = (uint8_t)t.valid;
  }
}

// ---------------------------------------------------------------- dispatch
namespace {

template <class T, int CB, int NO, bool NHWC>
hipError_t launch_variant(const KernelConfig& kc, const FusedArgs& a, hipStream_t s) {
  constexpr int M = 64;
  constexpr int WM = NO == 256 ? 1 : (NO == 128 ? 2 : 4);
  constexpr int WN = 4 / WM;
  const int64_t nblk = (int64_t)a.B * kc.tiles_per_img * kc.n_otiles;
  if (nblk <= 0) return hipSuccess;
  if (nblk > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fused_kernel<T, M, CB, NO, WM, WN, NHWC>), dim3((unsigned)nblk),
                     dim3(256), 0, s, a);
  return hipGetLastError();
}

template <class T, int CB, bool NHWC>
hipError_t launch_no(const KernelConfig& kc, const FusedArgs& a, hipStream_t s) {
  switch (kc.NO) {
    case 16: return launch_variant<T, CB, 16, NHWC>(kc, a, s);
    case 64: return launch_variant<T, CB, 64, NHWC>(kc, a, s);
    case 128: return launch_variant<T, CB, 128, NHWC>(kc, a, s);
    default: return hipErrorInvalidValue;
  }
}

template <class T, bool NHWC>
hipError_t launch_cb(const KernelConfig& kc, const FusedArgs& a, hipStream_t s);

template <>
hipError_t launch_cb<float, false>(const KernelConfig& kc, const FusedArgs& a, hipStream_t s) {
  if (kc.NO == 256) {
    if (kc.CB == 16) return launch_variant<float, 16, 256, false>(kc, a, s);
    if (kc.CB == 32) return launch_variant<float, 32, 256, false>(kc, a, s);
    return hipErrorInvalidValue;
  }
  if (kc.CB == 16) return launch_no<float, 16, false>(kc, a, s);
  if (kc.CB == 64) return launch_no<float, 64, false>(kc, a, s);
  return hipErrorInvalidValue;
}
template <>
hipError_t launch_cb<float, true>(const KernelConfig& kc, const FusedArgs& a, hipStream_t s) {
  if (kc.NO == 256) {
    if (kc.CB == 16) return launch_variant<float, 16, 256, true>(kc, a, s);
    if (kc.CB == 32) return launch_variant<float, 32, 256, true>(kc, a, s);
    return hipErrorInvalidValue;
  }
  if (kc.CB == 16) return launch_no<float, 16, true>(kc, a, s);
  if (kc.CB == 64) return launch_no<float, 64, true>(kc, a, s);
  return hipErrorInvalidValue;
}
template <>
hipError_t launch_cb<__bf16, false>(const KernelConfig& kc, const FusedArgs& a, hipStream_t s) {
  if (kc.NO == 256) {
    if (kc.CB == 32) return launch_variant<__bf16, 32, 256, false>(kc, a, s);
    if (kc.CB == 64) return launch_variant<__bf16, 64, 256, false>(kc, a, s);
    return hipErrorInvalidValue;
  }
  if (kc.CB == 32) return launch_no<__bf16, 32, false>(kc, a, s);
  if (kc.CB == 64) return launch_no<__bf16, 64, false>(kc, a, s);
  return hipErrorInvalidValue;
}
template <>
hipError_t launch_cb<__bf16, true>(const KernelConfig& kc, const FusedArgs& a, hipStream_t s) {
  if (kc.NO == 256) {
    if (kc.CB == 32) return launch_variant<__bf16, 32, 256, true>(kc, a, s);
    if (kc.CB == 64) return launch_variant<__bf16, 64, 256, true>(kc, a, s);
    return hipErrorInvalidValue;
  }
  if (kc.CB == 32) return launch_no<__bf16, 32, true>(kc, a, s);
  if (kc.CB == 64) return launch_no<__bf16, 64, true>(kc, a, s);
  return hipErrorInvalidValue;
}

unsigned grid_for(int64_t total) {
  int64_t g = (total + 255) / 256;
  if (g < 1) g = 1;
  if (g > 65535) g = 65535;
  return (unsigned)g;
}

}  // namespace

bool config_supported(const KernelConfig& kc) {
  if (kc.kind == 1) return wsk_supported(kc);
  if (kc.kind == 2) return quad_supported(kc);
  if (kc.kind == 3) return bf16w_supported(kc);
  if (kc.kind == 4) return bf16win_supported(kc);
  if (kc.M != 64) return false;
  if (kc.NO != 16 && kc.NO != 64 && kc.NO != 128 && kc.NO != 256) return false;
  if (kc.bf16) return kc.CB == 32 || kc.CB == 64;
  if (kc.NO == 256) return kc.CB == 16 || kc.CB == 32;
  return kc.CB == 16 || kc.CB == 64;
}

int64_t packed_weight_elems(const KernelConfig& kc, int K) {
  return (int64_t)kc.n_otiles * K * kc.nchunk * kc.CB * kc.NO;
}

hipError_t launch_pack(const KernelConfig& kc, const void* weight, void* wpack, int O, int C,
                       int kh, int kw, hipStream_t s) {
  const int64_t total = packed_weight_elems(kc, kh * kw);
  const int K = kh * kw;
  const int layout = kc.bf16 ? (kc.kind >= 3 ? 3 : 0) : kc.kind;
  const int G = kc.bf16 ? 8 : 4;  // elements per 16-byte run (CB is a multiple of it)
  if (kc.CB % G != 0) return hipErrorInvalidValue;
  const int64_t nruns = total / G;
  const unsigned grid = grid_for(nruns);
  if (kc.bf16)
    hipLaunchKernelGGL(pack_kernel<__bf16>, dim3(grid), dim3(256), 0, s,
                       static_cast<const __bf16*>(weight), static_cast<__bf16*>(wpack), O, C, K,
                       kc.CB, kc.NO, 8, kc.nchunk, layout, nruns);
  else
    hipLaunchKernelGGL(pack_kernel<float>, dim3(grid), dim3(256), 0, s,
                       static_cast<const float*>(weight), static_cast<float*>(wpack), O, C, K,
                       kc.CB, kc.NO, 4, kc.nchunk, layout, nruns);
  return hipGetLastError();
}

hipError_t launch_fused(const KernelConfig& kc, const FusedArgs& a, hipStream_t s) {
  // only that kernel splits taps or runs tap groups
  if (kc.kind != 2 && (a.nsplit != 1 || a.wsplit != 1)) return hipErrorInvalidValue;
  if (kc.kind == 1) return launch_fused_wsk(kc, a, s);
  if (kc.kind == 2) return launch_fused_quad(kc, a, s);
  if (kc.kind == 3) return launch_fused_bf16w(kc, a, s);
  if (kc.kind == 4) return launch_fused_bf16win(kc, a, s);
  if (kc.bf16) {
    return kc.nhwc ? launch_cb<__bf16, true>(kc, a, s) : launch_cb<__bf16, false>(kc, a, s);
  }
  return kc.nhwc ? launch_cb<float, true>(kc, a, s) : launch_cb<float, false>(kc, a, s);
}

hipError_t launch_fused_multi(const KernelConfig& kc, const MultiArgs& m, hipStream_t s) {
  if (m.n < 1 || m.n > kMaxBranches) return hipErrorInvalidValue;
  for (int i = 0; i < m.n; ++i)  // one grid slot per tile; tap groups only in that kernel
    if (m.a[i].nsplit != 1 || (kc.kind != 2 && m.a[i].wsplit != 1)) return hipErrorInvalidValue;
  if (kc.kind == 1) return launch_fused_wsk_multi(kc, m, s);
  if (kc.kind == 2) return launch_fused_quad_multi(kc, m, s);
  if (kc.kind == 3) return launch_fused_bf16w_multi(kc, m, s);
  if (kc.kind == 4) return launch_fused_bf16win_multi(kc, m, s);
  return hipErrorInvalidConfiguration;
}

hipError_t launch_coords(int bf16, const void* offset, int32_t* y0x0, uint8_t* valid4, int B,
                         int K, int kw, int Ho, int Wo, int ph, int pw, int H, int W,
                         hipStream_t s) {
  const int64_t total = (int64_t)B * K * Ho * Wo;
  if (total <= 0) return hipSuccess;
  if (bf16) {
    hipLaunchKernelGGL(coords_kernel<__bf16>, dim3(grid_for(total)), dim3(256), 0, s,
                       static_cast<const __bf16*>(offset), y0x0, valid4, B, K, kw, Ho, Wo, ph,
                       pw, H, W);
  } else {
    hipLaunchKernelGGL(coords_kernel<float>, dim3(grid_for(total)), dim3(256), 0, s,
                       static_cast<const float*>(offset), y0x0, valid4, B, K, kw, Ho, Wo, ph,
                       pw, H, W);
  }
  return hipGetLastError();
}

}  // namespace dcn
