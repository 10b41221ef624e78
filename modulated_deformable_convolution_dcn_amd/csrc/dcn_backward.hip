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
//              the modulated column tile and the g tile go to LDS transposed
//              and MFMA accumulates dW[c, o] over the run, then one atomic
//              add per weight element;
//   bwd_bias   a per-channel sum of g.

#include "dcn_device.h"
#include "dcn_launch.h"

namespace dcn {

namespace {

constexpr int TILE = 64;   // output pixels per tile
constexpr int GPAD = 4;    // LDS row padding (floats)

__device__ __forceinline__ void atomic_add(float* p, float v) { unsafeAtomicAdd(p, v); }

// Per (pixel, tap): the sampling point and the validity-masked corner
// weights, their derivatives and the corner pixel indices (row-major in the
// image) -- the same tap_point as the forward.
struct TapTerms {
  float w[4], dwy[4], dwx[4];
  int pix[4];
  int y0, x0;  // corner (0, 0), clamped to [-1, H] x [-1, W]
  bool ok[4];
};

__device__ __forceinline__ TapTerms tap_terms(const BwdArgs& a, int b, int ho, int wo, int k) {
  const int i = k / a.kw, j = k - (k / a.kw) * a.kw;
  const size_t ob = ((size_t)(b * 2 * a.K + 2 * k) * a.HoWo) + (size_t)ho * a.Wo + wo;
  const float dy = a.offset[ob], dx = a.offset[ob + a.HoWo];
  const TapPoint t = tap_point(dy, dx, ho - a.ph + i, wo - a.pw + j, a.H, a.W);
  const float hy = 1.0f - t.ly, hx = 1.0f - t.lx;
  const float wv[4] = {hy * hx, hy * t.lx, t.ly * hx, t.ly * t.lx};
  const float vy[4] = {-hx, -t.lx, hx, t.lx};
  const float vx[4] = {-hy, hy, -t.ly, t.ly};
  const int y0 = (int)fminf(fmaxf(t.y0, -1.0f), (float)a.H);
  const int x0 = (int)fminf(fmaxf(t.x0, -1.0f), (float)a.W);
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

__device__ __forceinline__ float gout_at(const BwdArgs& a, int b, int o, int hw) {
  return a.nhwc_g ? a.gout[((size_t)b * a.HoWo + hw) * a.O + o]
                  : a.gout[((size_t)b * a.O + o) * a.HoWo + hw];
}

}  // namespace

// ---------------------------------------------------------------- data grads
// LDS budget of the input-gradient window, per padded output count.
constexpr int bwd_window_floats(int OP) {
  return OP <= 16 ? 32768 : OP <= 64 ? 29696 : OP <= 128 ? 25600 : 16896;
}
constexpr int WSTR = 68;  // floats per window position: 64 channels + 4 (bank spread)

// One workgroup = an 8 x 8 block of output pixels of one image.  Its
// sampling points cluster around the block, so the input gradient of the
// window [wy0, wy0 + WH) x [wx0, wx0 + WW) (the block's footprint grown by R
// on every side) is accumulated in LDS with LDS atomics and flushed to
// memory once per 64-channel chunk; corners outside the window (far
// offsets) go straight to memory.  R < 0: no window.
template <int OP>  // padded output channels: 16, 64, 128 or 256
__global__ __launch_bounds__(256) void bwd_data_kernel(BwdArgs a, int R, int tiles_x,
                                                       int tiles_per_img) {
  constexpr int GST = OP + GPAD;     // g tile row stride
  constexpr int SST = 64 + GPAD;     // gs tile row stride
  __shared__ __attribute__((aligned(16))) float Gs[TILE * GST];
  __shared__ __attribute__((aligned(16))) float gsT[TILE * SST];
  __shared__ __attribute__((aligned(16))) float win[bwd_window_floats(OP)];
  // per-tap table of the block's 64 sampling points (written by wave 0):
  // {y0, x0, validity bits, pixel inside the output} and {ly, lx, mask}
  __shared__ int4 Ti[TILE];
  __shared__ f32x4 Tf[TILE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int logical = xcd_logical_block(blockIdx.x, gridDim.x);
  const int tile = logical % tiles_per_img, b = logical / tiles_per_img;
  const int ty = tile / tiles_x, tx = tile - (tile / tiles_x) * tiles_x;
  const bool use_win = R >= 0;
  const int WH = 8 + a.kh + 2 * R, WW = 8 + a.kw + 2 * R;
  const int wy0 = 8 * ty - a.ph - R, wx0 = 8 * tx - a.pw - R;
  // pixel px of the block -> output (8ty + px / 8, 8tx + px % 8)
  auto px_hw = [&](int px, int& hw) {
    const int ho = 8 * ty + (px >> 3), wo = 8 * tx + (px & 7);
    hw = ho * a.Wo + wo;
    return ho < a.Ho && wo < a.Wo;
  };

  // g tile [64 pixels][OP outputs], zero outside
  for (int e = tid; e < TILE * OP; e += 256) {
    const int o = e / TILE, px = e % TILE;
    int hw;
    const bool in = px_hw(px, hw);
    Gs[px * GST + o] = (o < a.O && in) ? gout_at(a, b, o, hw) : 0.0f;
  }

  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, a.x_bytes);
  const int rl = lane & 15, g = lane >> 4;
  const int sl = tid & 15;  // 4-channel slice of the 64-channel chunk
  const int nwin = use_win ? WH * WW : 0;
  // wave 0: the offsets / mask of the next tap, loaded one tap ahead
  int t_hw = 0;
  const bool t_in = tid < TILE && px_hw(tid, t_hw);
  float n_dy = 0.f, n_dx = 0.f, n_m = 1.f;
  auto t_load = [&](int k) {
    if (!t_in) return;
    const size_t ob = (size_t)(b * 2 * a.K + 2 * k) * a.HoWo + t_hw;
    n_dy = a.offset[ob];
    n_dx = a.offset[ob + a.HoWo];
    n_m = a.mask ? a.mask[(size_t)(b * a.K + k) * a.HoWo + t_hw] : 1.0f;
  };
  if (tid < TILE) t_load(0);
  for (int chunk = 0; chunk < a.nchunk; ++chunk) {
    for (int e = tid; e < nwin * WSTR; e += 256) win[e] = 0.0f;
    const int ch = chunk * 64 + 4 * sl;
    const bool chan_ok = ch < a.C;
    for (int k = 0; k < a.K; ++k) {
      const int kb = k * a.nchunk + chunk;
      __syncthreads();  // g tile / window zeroed; previous gs tile and table consumed
      if (tid < TILE) {  // (0) the table of tap k, then the loads of the next tap
        const int ho = t_hw / a.Wo, wo = t_hw - (t_hw / a.Wo) * a.Wo;
        const int i = k / a.kw, j = k - (k / a.kw) * a.kw;
        const TapPoint tp = tap_point(n_dy, n_dx, ho - a.ph + i, wo - a.pw + j, a.H, a.W);
        Ti[tid] = make_int4((int)fminf(fmaxf(tp.y0, -1.0f), (float)a.H),
                            (int)fminf(fmaxf(tp.x0, -1.0f), (float)a.W), (int)tp.valid,
                            t_in ? 1 : 0);
        Tf[tid] = f32x4{tp.ly, tp.lx, n_m, 0.0f};
        t_load(k + 1 < a.K ? k + 1 : 0);
      }
      // (1) gs[px, c] = sum_o g[px, o] W[o, c, k]: wave w -> pixel rows 16w..
      f32x4 acc[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
      const float* wt = a.wt + (size_t)kb * OP * 64;
#pragma unroll 4
      for (int q = 0; q < OP / 16; ++q) {
        const f32x4 af =
            *reinterpret_cast<const f32x4*>(&Gs[(16 * wave + rl) * GST + 16 * q + 4 * g]);
        f32x4 bf[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          bf[nt] = *reinterpret_cast<const f32x4*>(&wt[((4 * q + g) * 64 + 16 * nt + rl) * 4]);
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int nt = 0; nt < 4; ++nt)
            acc[nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[e], bf[nt][e], acc[nt], 0, 0, 0);
      }
      // MFMA 16x16 layout: lane l, register r -> row 4(l/16) + r, column l % 16
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          gsT[(16 * wave + 4 * g + r) * SST + 16 * nt + rl] = acc[nt][r];
      __syncthreads();

      // (2) per (pixel, 4-channel slice): corners, input-gradient adds,
      // mask / offset sums
#pragma unroll 1
      for (int p = 0; p < 4; ++p) {
        const int px = 16 * p + (tid >> 4);
        int hw;
        const bool in = px_hw(px, hw);
        float sm = 0.f, sdy = 0.f, sdx = 0.f, m = 0.f;
        if (in) {
          const int4 ti = Ti[px];
          const f32x4 tf = Tf[px];
          TapTerms t;
          {
            const float ly = tf[0], lx = tf[1], hy = 1.0f - ly, hx = 1.0f - lx;
            const float wv[4] = {hy * hx, hy * lx, ly * hx, ly * lx};
            const float vy[4] = {-hx, -lx, hx, lx};
            const float vx[4] = {-hy, hy, -ly, ly};
            t.y0 = ti.x;
            t.x0 = ti.y;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              t.ok[q] = (ti.z >> q) & 1;
              t.w[q] = t.ok[q] ? wv[q] : 0.0f;
              t.dwy[q] = t.ok[q] ? vy[q] : 0.0f;
              t.dwx[q] = t.ok[q] ? vx[q] : 0.0f;
              t.pix[q] = (b * a.H + ti.x + (q >> 1)) * a.W + ti.y + (q & 1);
            }
          }
          m = tf[2];
          const f32x4 gs = *reinterpret_cast<const f32x4*>(&gsT[px * SST + 4 * sl]);
          if (chan_ok) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              if (!t.ok[q]) continue;
              const uint32_t off = ((uint32_t)t.pix[q] * (uint32_t)a.C + (uint32_t)ch) * 4u;
              const f32x4 v = __builtin_bit_cast(f32x4, load16(xr, off));
              const float cw = m * t.w[q];
              const int wy = t.y0 + (q >> 1) - wy0, wx = t.x0 + (q & 1) - wx0;
              if (use_win && wy >= 0 && wy < WH && wx >= 0 && wx < WW) {
                float* dst = &win[(wy * WW + wx) * WSTR + 4 * sl];
#pragma unroll
                for (int e = 0; e < 4; ++e) atomicAdd(dst + e, gs[e] * cw);
              } else {
                float* dst = a.gx + (size_t)t.pix[q] * a.C + ch;
#pragma unroll
                for (int e = 0; e < 4; ++e) atomic_add(dst + e, gs[e] * cw);
              }
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                sm = __builtin_fmaf(gs[e] * t.w[q], v[e], sm);
                sdy = __builtin_fmaf(gs[e] * t.dwy[q], v[e], sdy);
                sdx = __builtin_fmaf(gs[e] * t.dwx[q], v[e], sdx);
              }
            }
          }
        }
        // sum over the 16 lanes of the pixel (lanes 16*(l/16) .. +15)
#pragma unroll
        for (int sh = 8; sh >= 1; sh >>= 1) {
          sm += __shfl_xor(sm, sh, 16);
          sdy += __shfl_xor(sdy, sh, 16);
          sdx += __shfl_xor(sdx, sh, 16);
        }
        if (sl == 0 && in) {
          if (a.gmask) atomic_add(a.gmask + (size_t)(b * a.K + k) * a.HoWo + hw, sm);
          if (a.goff) {
            atomic_add(a.goff + (size_t)(b * 2 * a.K + 2 * k) * a.HoWo + hw, m * sdy);
            atomic_add(a.goff + (size_t)(b * 2 * a.K + 2 * k + 1) * a.HoWo + hw, m * sdx);
          }
        }
      }
    }
    // (3) flush the window's input gradient of this chunk
    __syncthreads();
    for (int e = tid; e < nwin * 64; e += 256) {
      const int pos = e >> 6, c = e & 63;
      const int y = wy0 + pos / WW, xx = wx0 + pos % WW;
      const float v = win[pos * WSTR + c];
      if (v != 0.0f && y >= 0 && y < a.H && xx >= 0 && xx < a.W && chunk * 64 + c < a.C)
        atomic_add(a.gx + ((size_t)(b * a.H + y) * a.W + xx) * a.C + chunk * 64 + c, v);
    }
    __syncthreads();  // flush done before the next chunk zeroes the window
  }
}

// ---------------------------------------------------------------- weight grad
template <int NT>  // 16-column output tiles per wave = OP / 16
__global__ __launch_bounds__(256) void bwd_weight_kernel(BwdArgs a, int tiles_per_run,
                                                         int runs_per_img) {
  constexpr int OP = 16 * NT;
  constexpr int ST_ = TILE + GPAD;
  __shared__ __attribute__((aligned(16))) float ST[64 * ST_];   // [channel][pixel]
  __shared__ __attribute__((aligned(16))) float GT[OP * ST_];   // [output][pixel]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int logical = xcd_logical_block(blockIdx.x, gridDim.x);
  const int run = logical % runs_per_img;
  const int t2 = logical / runs_per_img;
  const int b = t2 % a.B;
  const int kb = t2 / a.B;
  const int k = kb / a.nchunk, chunk = kb - k * a.nchunk;
  const int rl = lane & 15, g = lane >> 4;
  const int sl = tid & 15;
  const int ch = chunk * 64 + 4 * sl;
  const bool chan_ok = ch < a.C;
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, a.x_bytes);

  f32x4 acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int t_end = min((run + 1) * tiles_per_run, a.tiles_per_img);
  for (int tile = run * tiles_per_run; tile < t_end; ++tile) {
    const int hw0 = tile * TILE;
    __syncthreads();  // previous tile's operands consumed
    // modulated column tile, transposed: ST[c][px]
#pragma unroll 1
    for (int p = 0; p < 4; ++p) {
      const int px = 16 * p + (tid >> 4);
      const int hw = hw0 + px;
      f32x4 s = {0.f, 0.f, 0.f, 0.f};
      if (hw < a.HoWo && chan_ok) {
        const int ho = hw / a.Wo, wo = hw - (hw / a.Wo) * a.Wo;
        const TapTerms t = tap_terms(a, b, ho, wo, k);
        const float m = a.mask ? a.mask[((size_t)(b * a.K + k)) * a.HoWo + hw] : 1.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t off = t.ok[q] ? ((uint32_t)t.pix[q] * (uint32_t)a.C + (uint32_t)ch) * 4u
                                       : kNoCorner;
          const f32x4 v = __builtin_bit_cast(f32x4, load16(xr, off));
#pragma unroll
          for (int e = 0; e < 4; ++e) s[e] = __builtin_fmaf(t.w[q], v[e], s[e]);
        }
        s = s * m;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) ST[(4 * sl + e) * ST_ + px] = s[e];
    }
    // g tile, transposed: GT[o][px]
    for (int e = tid; e < OP * TILE; e += 256) {
      const int o = e / TILE, px = e % TILE;
      const int hw = hw0 + px;
      GT[o * ST_ + px] = (o < a.O && hw < a.HoWo) ? gout_at(a, b, o, hw) : 0.0f;
    }
    __syncthreads();
    // dW[c, o] += sum_px ST[c][px] GT[o][px]: wave w -> channel rows 16w..
#pragma unroll
    for (int j = 0; j < TILE / 16; ++j) {
      const f32x4 af = *reinterpret_cast<const f32x4*>(&ST[(16 * wave + rl) * ST_ + 16 * j + 4 * g]);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const f32x4 bf = *reinterpret_cast<const f32x4*>(&GT[(16 * nt + rl) * ST_ + 16 * j + 4 * g]);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[e], bf[e], acc[nt], 0, 0, 0);
      }
    }
  }
  const int i = k / a.kw, jj = k - (k / a.kw) * a.kw;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int o = 16 * nt + rl;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int c = chunk * 64 + 16 * wave + 4 * g + r;
      if (c < a.C && o < a.O)
        atomic_add(a.gw + (((size_t)o * a.C + c) * a.kh + i) * a.kw + jj, acc[nt][r]);
    }
  }
}

// ---------------------------------------------------------------- bias grad
__global__ __launch_bounds__(256) void bwd_bias_kernel(BwdArgs a) {
  __shared__ float red[256];
  const int o = blockIdx.x % a.O, b = blockIdx.x / a.O;
  float s = 0.f;
  for (int hw = threadIdx.x; hw < a.HoWo; hw += 256) s += gout_at(a, b, o, hw);
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) atomic_add(a.gb + o, red[0]);
}

// ---------------------------------------------------------------- helpers
__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ p, int64_t n) {
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256)
    p[e] = 0.0f;
}

// weight [O][C][kh][kw] -> per (tap, 64-channel chunk) block [OP/4][64][4]:
// element (o, c) at ((o / 4) * 64 + c % 64) * 4 + o % 4, so one 16-byte read
// gives a lane 4 consecutive outputs of one channel (4 MFMA k-steps).
__global__ __launch_bounds__(256) void bwd_pack_kernel(const float* __restrict__ w,
                                                       float* __restrict__ wt, int O, int C,
                                                       int K, int OP, int nchunk) {
  const int64_t total = (int64_t)O * C * K;
  for (int64_t s = (int64_t)blockIdx.x * 256 + threadIdx.x; s < total;
       s += (int64_t)gridDim.x * 256) {
    const int tap = (int)(s % K);
    const int64_t oc = s / K;
    const int c = (int)(oc % C), o = (int)(oc / C);
    const int64_t blk = (int64_t)tap * nchunk + c / 64;
    wt[blk * OP * 64 + ((o / 4) * 64 + c % 64) * 4 + o % 4] = w[s];
  }
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

int bwd_out_pad(int O) { return O <= 16 ? 16 : O <= 64 ? 64 : O <= 128 ? 128 : 256; }

int64_t bwd_workspace_floats(int O, int C, int K) {
  return (int64_t)K * ((C + 63) / 64) * bwd_out_pad(O) * 64;
}

hipError_t launch_backward(const BwdArgs& a0, const float* weight, float* ws, hipStream_t s) {
  BwdArgs a = a0;
  const int OP = bwd_out_pad(a.O);
  hipError_t e;
  // zero the accumulated outputs and the padded weight blocks
  const int64_t nx = (int64_t)a.B * a.H * a.W * a.C;
  if ((e = zero(a.gx, nx, s)) != hipSuccess) return e;
  if ((e = zero(a.goff, (int64_t)a.B * 2 * a.K * a.HoWo, s)) != hipSuccess) return e;
  if ((e = zero(a.gmask, (int64_t)a.B * a.K * a.HoWo, s)) != hipSuccess) return e;
  if ((e = zero(a.gw, (int64_t)a.O * a.C * a.K, s)) != hipSuccess) return e;
  if ((e = zero(a.gb, a.O, s)) != hipSuccess) return e;
  const int64_t nws = bwd_workspace_floats(a.O, a.C, a.K);
  if ((e = zero(ws, nws, s)) != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_pack_kernel, dim3(grid_of((int64_t)a.O * a.C * a.K)), dim3(256), 0, s,
                     weight, ws, a.O, a.C, a.K, OP, a.nchunk);
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
    const dim3 grid((unsigned)nblk), block(256);
    switch (OP) {
      case 16: hipLaunchKernelGGL(bwd_data_kernel<16>, grid, block, 0, s, a, R, tiles_x, tiles); break;
      case 64: hipLaunchKernelGGL(bwd_data_kernel<64>, grid, block, 0, s, a, R, tiles_x, tiles); break;
      case 128: hipLaunchKernelGGL(bwd_data_kernel<128>, grid, block, 0, s, a, R, tiles_x, tiles); break;
      default: hipLaunchKernelGGL(bwd_data_kernel<256>, grid, block, 0, s, a, R, tiles_x, tiles); break;
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (a.gw) {
    // runs of pixel tiles: about 2048 workgroups in all
    const int64_t per_run_units = (int64_t)a.K * a.nchunk * a.B;
    int64_t runs = (2048 + per_run_units - 1) / per_run_units;
    if (runs > a.tiles_per_img) runs = a.tiles_per_img;
    if (runs < 1) runs = 1;
    const int tiles_per_run = (int)((a.tiles_per_img + runs - 1) / runs);
    const int runs_per_img = (a.tiles_per_img + tiles_per_run - 1) / tiles_per_run;
    const int64_t g = per_run_units * runs_per_img;
    if (g > 0x7fffffff) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)g), block(256);
    switch (OP) {
      case 16: hipLaunchKernelGGL(bwd_weight_kernel<1>, grid, block, 0, s, a, tiles_per_run, runs_per_img); break;
      case 64: hipLaunchKernelGGL(bwd_weight_kernel<4>, grid, block, 0, s, a, tiles_per_run, runs_per_img); break;
      case 128: hipLaunchKernelGGL(bwd_weight_kernel<8>, grid, block, 0, s, a, tiles_per_run, runs_per_img); break;
      default: hipLaunchKernelGGL(bwd_weight_kernel<16>, grid, block, 0, s, a, tiles_per_run, runs_per_img); break;
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (a.gb) {
    hipLaunchKernelGGL(bwd_bias_kernel, dim3((unsigned)(a.O * a.B)), dim3(256), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace dcn
