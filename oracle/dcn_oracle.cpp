// dcn_oracle.cpp -- CPU oracle for the modulated deformable conv2d forward.
//
// TEST INFRASTRUCTURE ONLY (see dcn_oracle.h).  A plain loop nest written
// from the operator's definition on page 1 ("deform_conv.py", module
// docstring and deform_conv2d_gather): no SIMD intrinsics, no BLAS, no
// blocking.  Build: g++ -O2 -std=c++17 -ffp-contract=off -shared -fPIC.
//
// Each step below names the part of that page it follows.

#include "dcn_oracle.h"

#include <cmath>
#include <cstdlib>
#include <thread>
#include <vector>

namespace {

struct Dims {
  int64_t B, C, H, W, O, kh, kw, ph, pw, K, Ho, Wo;
};

bool make_dims(const dcn_oracle_shape* s, Dims* d) {
  d->B = s->batch; d->C = s->in_ch; d->H = s->height; d->W = s->width;
  d->O = s->out_ch; d->kh = s->kernel_h; d->kw = s->kernel_w;
  d->ph = s->pad_h; d->pw = s->pad_w;
  if (d->B < 0 || d->C <= 0 || d->H <= 0 || d->W <= 0 || d->O <= 0 || d->kh <= 0 ||
      d->kw <= 0 || d->ph < 0 || d->pw < 0)
    return false;
  d->K = d->kh * d->kw;
  // Output size for stride 1, dilation 1 (page 1: wo = w + 2*pw - kw + 1;
  // the row count follows the same rule).
  d->Ho = d->H + 2 * d->ph - d->kh + 1;
  d->Wo = d->W + 2 * d->pw - d->kw + 1;
  return d->Ho > 0 && d->Wo > 0;
}

// The sampling point of tap (i, j) at output (ho, wo), page 1: the base grid
// (ho - pad + i) is an exact integer in the input dtype, then ONE fp32 add of
// the learned offset; floor and fraction are fp32 too.  `volatile` keeps the
// compiler from forming anything but the single rounded add.
struct Coord {
  float y0, x0, ly, lx;
};

Coord tap_coord(const Dims& d, int64_t ho, int64_t wo, int64_t i, int64_t j, float dy,
                float dx) {
  volatile float gy = static_cast<float>(ho - d.ph + i);
  volatile float gx = static_cast<float>(wo - d.pw + j);
  volatile float py = gy + dy;
  volatile float px = gx + dx;
  Coord c;
  c.y0 = std::floor(static_cast<float>(py));
  c.x0 = std::floor(static_cast<float>(px));
  volatile float ly = py - c.y0;
  volatile float lx = px - c.x0;
  c.ly = ly;
  c.lx = lx;
  return c;
}

// Corner (a, b) of the 2x2 neighbourhood is inside the image exactly when
// 0 <= y0+a <= H-1 and 0 <= x0+b <= W-1 (page 1, the `valid` comparison);
// compared in float so that no integer conversion of a far-away point is
// needed.
bool corner_valid(const Dims& d, float y0, float x0, int a, int b) {
  volatile float yy = y0 + static_cast<float>(a);
  volatile float xx = x0 + static_cast<float>(b);
  return yy >= 0.0f && yy <= static_cast<float>(d.H - 1) && xx >= 0.0f &&
         xx <= static_cast<float>(d.W - 1);
}

void forward_pixel(const Dims& d, const float* x, const float* offset, const float* mask,
                   const float* weight, const float* bias, int64_t p, double* out_row,
                   double* norm_row, std::vector<double>& s) {
  const int64_t hw = d.Ho * d.Wo;
  const int64_t b = p / hw;
  const int64_t ho = (p % hw) / d.Wo;
  const int64_t wo = p % d.Wo;

  // s[k][c]: the modulated bilinear sample of channel c at tap k -- one row
  // of page 1's column matrix `cols`, whose column index is (tap, channel).
  for (int64_t k = 0; k < d.K; ++k) {
    // Tap order k = i*kw + j (page 1: ki = arange(kh).repeat_interleave(kw),
    // kj = arange(kw).repeat(kh)).
    const int64_t i = k / d.kw;
    const int64_t j = k % d.kw;
    // offset viewed as [B, K, 2, Ho, Wo]: row offset first, then column
    // offset (page 1: off[:, :, 0] feeds py, off[:, :, 1] feeds px).
    const float dy = offset[((b * 2 * d.K + 2 * k) * d.Ho + ho) * d.Wo + wo];
    const float dx = offset[((b * 2 * d.K + 2 * k + 1) * d.Ho + ho) * d.Wo + wo];
    const double m = mask ? static_cast<double>(mask[((b * d.K + k) * d.Ho + ho) * d.Wo + wo])
                          : 1.0;
    const Coord cd = tap_coord(d, ho, wo, i, j, dy, dx);
    const double ly = cd.ly, lx = cd.lx;
    // The four bilinear weights of corners (0,0), (0,1), (1,0), (1,1)
    // (page 1, the (dy, dx, wgt) tuple list).
    const double wgt[2][2] = {{(1.0 - ly) * (1.0 - lx), (1.0 - ly) * lx},
                              {ly * (1.0 - lx), ly * lx}};
    double* sk = &s[k * d.C];
    for (int64_t c = 0; c < d.C; ++c) sk[c] = 0.0;
    for (int a = 0; a < 2; ++a) {
      for (int bb = 0; bb < 2; ++bb) {
        if (!corner_valid(d, cd.y0, cd.x0, a, bb)) continue;  // outside counts as 0
        const int64_t yy = static_cast<int64_t>(cd.y0) + a;
        const int64_t xx = static_cast<int64_t>(cd.x0) + bb;
        const float* v = &x[((b * d.H + yy) * d.W + xx) * d.C];
        for (int64_t c = 0; c < d.C; ++c) sk[c] += wgt[a][bb] * static_cast<double>(v[c]);
      }
    }
    // Modulation: the blended sample times mask_k (page 1 multiplies each
    // corner term by msk; doing it once after the sum is the same value).
    for (int64_t c = 0; c < d.C; ++c) sk[c] *= m;
  }

  // Contraction over (tap, channel) with weight[o, c, i, j] (page 1:
  // wmat = weight.permute(2, 3, 1, 0) -> rows (i, j, c); cols @ wmat), then
  // the bias (page 1: out + bias.view(1, o, 1, 1)).
  for (int64_t o = 0; o < d.O; ++o) {
    double acc = 0.0, nrm = 0.0;
    for (int64_t k = 0; k < d.K; ++k) {
      const int64_t i = k / d.kw;
      const int64_t j = k % d.kw;
      const double* sk = &s[k * d.C];
      for (int64_t c = 0; c < d.C; ++c) {
        const double w = weight[((o * d.C + c) * d.kh + i) * d.kw + j];
        acc += w * sk[c];
        nrm += std::fabs(w) * std::fabs(sk[c]);
      }
    }
    out_row[o] = acc + (bias ? static_cast<double>(bias[o]) : 0.0);
    if (norm_row) norm_row[o] = nrm;
  }
}

// Float -> int32 that saturates instead of overflowing (only the far-away
// corners of huge offsets ever reach the limits; they are invalid anyway).
int32_t to_i32_sat(float v) {
  if (v >= 2147483648.0f) return 2147483647;
  if (v < -2147483648.0f) return -2147483647 - 1;
  return static_cast<int32_t>(v);
}

int resolve_threads(int nthreads, int64_t work) {
  int n = nthreads > 0 ? nthreads : static_cast<int>(std::thread::hardware_concurrency());
  if (n < 1) n = 1;
  if (work < n) n = static_cast<int>(work > 0 ? work : 1);
  return n;
}

}  // namespace

extern "C" int dcn_oracle_forward(const dcn_oracle_shape* s, const float* x,
                                  const float* offset, const float* mask, const float* weight,
                                  const float* bias, const int64_t* pixels, int64_t npixels,
                                  double* out, double* norm, int nthreads) {
  if (!s || !offset || !weight || !out) return 1;
  Dims d;
  if (!make_dims(s, &d)) return 2;
  const int64_t total = d.B * d.Ho * d.Wo;
  if (npixels < 0) return 2;
  if (!pixels && npixels != total) return 2;
  if (npixels > 0 && !x) return 1;
  if (pixels) {
    for (int64_t n = 0; n < npixels; ++n)
      if (pixels[n] < 0 || pixels[n] >= total) return 2;
  }
  const int nt = resolve_threads(nthreads, npixels);
  std::vector<std::thread> pool;
  // Static interleaved split over the pixel list; each pixel is computed by
  // one thread start to finish, so the thread count changes no result.
  for (int t = 0; t < nt; ++t) {
    pool.emplace_back([&, t]() {
      std::vector<double> sbuf(static_cast<size_t>(d.K * d.C));
      for (int64_t n = t; n < npixels; n += nt) {
        const int64_t p = pixels ? pixels[n] : n;
        forward_pixel(d, x, offset, mask, weight, bias, p, out + n * d.O,
                      norm ? norm + n * d.O : nullptr, sbuf);
      }
    });
  }
  for (auto& th : pool) th.join();
  return 0;
}

extern "C" int dcn_oracle_coords(const dcn_oracle_shape* s, const float* offset,
                                 int32_t* y0x0, uint8_t* valid4, int nthreads) {
  if (!s || !offset || !y0x0 || !valid4) return 1;
  Dims d;
  if (!make_dims(s, &d)) return 2;
  const int64_t rows = d.B * d.K * d.Ho;  // one work item per (b, k, ho) row
  const int nt = resolve_threads(nthreads, rows);
  std::vector<std::thread> pool;
  for (int t = 0; t < nt; ++t) {
    pool.emplace_back([&, t]() {
      for (int64_t r = t; r < rows; r += nt) {
        const int64_t b = r / (d.K * d.Ho);
        const int64_t k = (r / d.Ho) % d.K;
        const int64_t ho = r % d.Ho;
        const int64_t i = k / d.kw, j = k % d.kw;
        for (int64_t wo = 0; wo < d.Wo; ++wo) {
          const float dy = offset[((b * 2 * d.K + 2 * k) * d.Ho + ho) * d.Wo + wo];
          const float dx = offset[((b * 2 * d.K + 2 * k + 1) * d.Ho + ho) * d.Wo + wo];
          const Coord cd = tap_coord(d, ho, wo, i, j, dy, dx);
          const int64_t e = ((b * d.K + k) * d.Ho + ho) * d.Wo + wo;
          y0x0[2 * e] = to_i32_sat(cd.y0);
          y0x0[2 * e + 1] = to_i32_sat(cd.x0);
          uint8_t v = 0;
          for (int a = 0; a < 2; ++a)
            for (int bb = 0; bb < 2; ++bb)
              if (corner_valid(d, cd.y0, cd.x0, a, bb)) v |= static_cast<uint8_t>(1u << (2 * a + bb));
          valid4[e] = v;
        }
      }
    });
  }
  for (auto& th : pool) th.join();
  return 0;
}

// ---------------------------------------------------------------- backward
// The forward, differentiated term by term.  For output pixel (b, ho, wo),
// tap k with sampling point p in floor cell (y0, x0), fractions (ly, lx):
//   su[c]  = sum_valid w_ab x_ab[c]           (unmodulated sample)
//   s[c]   = m su[c]                          (the column-matrix entry)
//   out[o] = bias[o] + sum_{k,c} W[o,c,k] s[c]
// so with g[o] = dL/dout[o] and gs[c] = sum_o g[o] W[o,c,k]:
//   dL/dW[o,c,k]   += g[o] s[c]               dL/dbias[o] += g[o]
//   dL/dx_ab[c]    += gs[c] m w_ab            (valid corners)
//   dL/dm          += sum_c gs[c] su[c]
//   dL/ddy         += m sum_c gs[c] sum_valid (d w_ab / d ly) x_ab[c]
//   dL/ddx         += m sum_c gs[c] sum_valid (d w_ab / d lx) x_ab[c]
// with d w / d ly = {-(1-lx), -lx, (1-lx), lx} and d w / d lx =
// {-(1-ly), (1-ly), -ly, ly} for corners (0,0), (0,1), (1,0), (1,1).
namespace {

struct BwdAcc {
  std::vector<double> gx, ngx, gw, ngw, gb, ngb;
};

void backward_pixel(const Dims& d, const float* x, const float* offset, const float* mask,
                    const float* weight, const float* grad_out, int64_t p, BwdAcc& acc,
                    double* goff, double* gmask, double* ngoff, double* ngmask,
                    std::vector<double>& gs, std::vector<double>& gsa) {
  const int64_t hw = d.Ho * d.Wo;
  const int64_t b = p / hw;
  const int64_t ho = (p % hw) / d.Wo;
  const int64_t wo = p % d.Wo;
  auto g_at = [&](int64_t o) {
    return static_cast<double>(grad_out[((b * d.O + o) * d.Ho + ho) * d.Wo + wo]);
  };
  for (int64_t o = 0; o < d.O; ++o) {
    acc.gb[o] += g_at(o);
    acc.ngb[o] += std::fabs(g_at(o));
  }
  for (int64_t k = 0; k < d.K; ++k) {
    const int64_t i = k / d.kw, j = k % d.kw;
    const int64_t oy = ((b * 2 * d.K + 2 * k) * d.Ho + ho) * d.Wo + wo;
    const int64_t ox = ((b * 2 * d.K + 2 * k + 1) * d.Ho + ho) * d.Wo + wo;
    const int64_t om = ((b * d.K + k) * d.Ho + ho) * d.Wo + wo;
    const double m = mask ? static_cast<double>(mask[om]) : 1.0;
    const Coord cd = tap_coord(d, ho, wo, i, j, offset[oy], offset[ox]);
    const double ly = cd.ly, lx = cd.lx;
    const double wgt[4] = {(1.0 - ly) * (1.0 - lx), (1.0 - ly) * lx, ly * (1.0 - lx), ly * lx};
    const double dwy[4] = {-(1.0 - lx), -lx, 1.0 - lx, lx};
    const double dwx[4] = {-(1.0 - ly), 1.0 - ly, -ly, ly};
    const float* v[4] = {nullptr, nullptr, nullptr, nullptr};
    int64_t at[4] = {0, 0, 0, 0};
    for (int a = 0; a < 2; ++a)
      for (int bb = 0; bb < 2; ++bb) {
        if (!corner_valid(d, cd.y0, cd.x0, a, bb)) continue;
        const int64_t yy = static_cast<int64_t>(cd.y0) + a;
        const int64_t xx = static_cast<int64_t>(cd.x0) + bb;
        at[2 * a + bb] = ((b * d.H + yy) * d.W + xx) * d.C;
        v[2 * a + bb] = &x[at[2 * a + bb]];
      }
    // gs[c] = sum_o g[o] W[o, c, k] and its absolute-term bound
    for (int64_t c = 0; c < d.C; ++c) {
      double t = 0.0, ta = 0.0;
      for (int64_t o = 0; o < d.O; ++o) {
        const double w = weight[((o * d.C + c) * d.kh + i) * d.kw + j];
        t += g_at(o) * w;
        ta += std::fabs(g_at(o)) * std::fabs(w);
      }
      gs[c] = t;
      gsa[c] = ta;
    }
    double sm = 0.0, nsm = 0.0, sdy = 0.0, nsdy = 0.0, sdx = 0.0, nsdx = 0.0;
    for (int64_t c = 0; c < d.C; ++c) {
      double su = 0.0, sua = 0.0, ty = 0.0, tya = 0.0, tx = 0.0, txa = 0.0;
      for (int q = 0; q < 4; ++q) {
        if (!v[q]) continue;
        const double xv = v[q][c];
        su += wgt[q] * xv;
        sua += wgt[q] * std::fabs(xv);
        ty += dwy[q] * xv;
        tya += std::fabs(dwy[q] * xv);
        tx += dwx[q] * xv;
        txa += std::fabs(dwx[q] * xv);
        acc.gx[at[q] + c] += gs[c] * m * wgt[q];
        acc.ngx[at[q] + c] += gsa[c] * std::fabs(m) * wgt[q];
      }
      sm += gs[c] * su;
      nsm += gsa[c] * sua;
      sdy += gs[c] * ty;
      nsdy += gsa[c] * tya;
      sdx += gs[c] * tx;
      nsdx += gsa[c] * txa;
      for (int64_t o = 0; o < d.O; ++o) {
        const int64_t wi = ((o * d.C + c) * d.kh + i) * d.kw + j;
        acc.gw[wi] += g_at(o) * m * su;
        acc.ngw[wi] += std::fabs(g_at(o)) * std::fabs(m) * sua;
      }
    }
    if (gmask) gmask[om] = sm;
    if (ngmask) ngmask[om] = nsm;
    if (goff) {
      goff[oy] = m * sdy;
      goff[ox] = m * sdx;
    }
    if (ngoff) {
      ngoff[oy] = std::fabs(m) * nsdy;
      ngoff[ox] = std::fabs(m) * nsdx;
    }
  }
}

}  // namespace

extern "C" int dcn_oracle_backward(const dcn_oracle_shape* s, const float* x,
                                   const float* offset, const float* mask, const float* weight,
                                   const float* grad_out, double* gx, double* goff,
                                   double* gmask, double* gw, double* gb, double* ngx,
                                   double* ngoff, double* ngmask, double* ngw, double* ngb,
                                   int nthreads) {
  if (!s || !x || !offset || !weight || !grad_out) return 1;
  Dims d;
  if (!make_dims(s, &d)) return 2;
  const int64_t npix = d.B * d.Ho * d.Wo;
  const int64_t nx = d.B * d.H * d.W * d.C, nw = d.O * d.C * d.K;
  const int nt = resolve_threads(nthreads, npix);
  std::vector<BwdAcc> accs(static_cast<size_t>(nt));
  std::vector<std::thread> pool;
  for (int t = 0; t < nt; ++t) {
    pool.emplace_back([&, t]() {
      BwdAcc& a = accs[t];
      a.gx.assign(nx, 0.0);
      a.ngx.assign(nx, 0.0);
      a.gw.assign(nw, 0.0);
      a.ngw.assign(nw, 0.0);
      a.gb.assign(d.O, 0.0);
      a.ngb.assign(d.O, 0.0);
      std::vector<double> gsv(static_cast<size_t>(d.C)), gsa(static_cast<size_t>(d.C));
      // contiguous pixel ranges: the per-thread sums run in pixel order
      const int64_t lo = npix * t / nt, hi = npix * (t + 1) / nt;
      for (int64_t p = lo; p < hi; ++p)
        backward_pixel(d, x, offset, mask, weight, grad_out, p, a, goff, gmask, ngoff, ngmask,
                       gsv, gsa);
    });
  }
  for (auto& th : pool) th.join();
  auto reduce = [&](double* dst, std::vector<double> BwdAcc::*field, int64_t n) {
    if (!dst) return;
    for (int64_t e = 0; e < n; ++e) dst[e] = 0.0;
    for (int t = 0; t < nt; ++t) {
      const std::vector<double>& v = accs[t].*field;
      for (int64_t e = 0; e < n; ++e) dst[e] += v[e];
    }
  };
  reduce(gx, &BwdAcc::gx, nx);
  reduce(ngx, &BwdAcc::ngx, nx);
  reduce(gw, &BwdAcc::gw, nw);
  reduce(ngw, &BwdAcc::ngw, nw);
  reduce(gb, &BwdAcc::gb, d.O);
  reduce(ngb, &BwdAcc::ngb, d.O);
  return 0;
}

// ---------------------------------------------------------------- MSDA
// Page 5, "Multi-scale deformable attention": sample each level's value map
// bilinearly at the normalised location and sum with the attention weights.
// The pixel coordinate of a normalised location follows the half-pixel
// convention (pixel centres at (i + 0.5) / size), each step rounded to fp32.
extern "C" int dcn_oracle_msda(int64_t B, int64_t S, int64_t G, int64_t D, int64_t Q,
                               int64_t L, int64_t K, const int64_t* shapes, const float* value,
                               const float* locations, const float* weights, int softmax,
                               double* out, double* norm, int nthreads) {
  if (!shapes || !value || !locations || !weights || !out) return 1;
  if (B < 0 || S <= 0 || G <= 0 || D <= 0 || Q < 0 || L <= 0 || K <= 0) return 2;
  std::vector<int64_t> start(static_cast<size_t>(L));
  int64_t total = 0;
  for (int64_t l = 0; l < L; ++l) {
    if (shapes[2 * l] <= 0 || shapes[2 * l + 1] <= 0) return 2;
    start[l] = total;
    total += shapes[2 * l] * shapes[2 * l + 1];
  }
  if (total != S) return 2;
  const int64_t pairs = B * Q * G;
  const int nt = resolve_threads(nthreads, pairs);
  std::vector<std::thread> pool;
  for (int t = 0; t < nt; ++t) {
    pool.emplace_back([&, t]() {
      std::vector<double> a(static_cast<size_t>(L * K));
      for (int64_t n = t; n < pairs; n += nt) {
        const int64_t g = n % G, bq = n / G, b = bq / Q;
        const float* wrow = &weights[n * L * K];  // (b, q, g) row of (B, Q, G, L*K)
        if (softmax) {
          double mx = -INFINITY, sum = 0.0;
          for (int64_t e = 0; e < L * K; ++e) mx = std::fmax(mx, (double)wrow[e]);
          for (int64_t e = 0; e < L * K; ++e) sum += std::exp((double)wrow[e] - mx);
          for (int64_t e = 0; e < L * K; ++e) a[e] = std::exp((double)wrow[e] - mx) / sum;
        } else {
          for (int64_t e = 0; e < L * K; ++e) a[e] = wrow[e];
        }
        double* orow = &out[n * D];
        double* nrow = norm ? &norm[n * D] : nullptr;
        for (int64_t c = 0; c < D; ++c) {
          orow[c] = 0.0;
          if (nrow) nrow[c] = 0.0;
        }
        for (int64_t l = 0; l < L; ++l) {
          const int64_t H = shapes[2 * l], W = shapes[2 * l + 1];
          for (int64_t k = 0; k < K; ++k) {
            const float* loc = &locations[((n * L + l) * K + k) * 2];
            volatile float sx = loc[0] * static_cast<float>(W);
            volatile float sy = loc[1] * static_cast<float>(H);
            volatile float px = sx - 0.5f;
            volatile float py = sy - 0.5f;
            const float x0 = std::floor(static_cast<float>(px));
            const float y0 = std::floor(static_cast<float>(py));
            volatile float fx = px - x0;
            volatile float fy = py - y0;
            const double lx = static_cast<float>(fx), ly = static_cast<float>(fy);
            const double wgt[2][2] = {{(1.0 - ly) * (1.0 - lx), (1.0 - ly) * lx},
                                      {ly * (1.0 - lx), ly * lx}};
            const double ak = a[l * K + k];
            for (int ca = 0; ca < 2; ++ca)
              for (int cb = 0; cb < 2; ++cb) {
                volatile float yy = y0 + static_cast<float>(ca);
                volatile float xx = x0 + static_cast<float>(cb);
                if (!(yy >= 0.0f && yy <= static_cast<float>(H - 1) && xx >= 0.0f &&
                      xx <= static_cast<float>(W - 1)))
                  continue;  // outside the level counts as zero
                const int64_t pix = start[l] + static_cast<int64_t>(yy) * W +
                                    static_cast<int64_t>(xx);
                const float* v = &value[((b * S + pix) * G + g) * D];
                for (int64_t c = 0; c < D; ++c) {
                  orow[c] += ak * wgt[ca][cb] * static_cast<double>(v[c]);
                  if (nrow) nrow[c] += std::fabs(ak) * wgt[ca][cb] * std::fabs((double)v[c]);
                }
              }
          }
        }
      }
    });
  }
  for (auto& th : pool) th.join();
  return 0;
}

// ---------------------------------------------------------------- single-scale
// Page 5, "Single-scale deformable sampling" (DCNv3 of InternImage): the same
// sampling points as the deformable convolution, but no spatial weight: each
// channel group g aggregates its own K bilinear samples with one weight per
// (group, tap, pixel).  Per (b, ho, wo, g) and channel c of the group:
//   out = sum_k a_{g,k} * bilinear(x[b, :, :, g*D + c], ho - ph + i_k + dy, wo - pw + j_k + dx)
// with the point, floor and fractions exactly as in the convolution (one fp32
// add of the offset to the exact grid) and fp64 from the weights on.
extern "C" int dcn_oracle_dsample(const dcn_oracle_ds_shape* s, const float* x,
                                  const float* offset, const float* weights, int softmax,
                                  double* out, double* norm, int nthreads) {
  if (!s || !x || !offset || !weights || !out) return 1;
  if (s->batch < 0 || s->groups <= 0 || s->group_ch <= 0 || s->height <= 0 || s->width <= 0 ||
      s->kernel_h <= 0 || s->kernel_w <= 0 || s->pad_h < 0 || s->pad_w < 0)
    return 2;
  // the convolution's geometry (no output channels here; O is unused)
  dcn_oracle_shape cs = {s->batch, s->groups * s->group_ch, s->height, s->width, 1,
                         s->kernel_h, s->kernel_w, s->pad_h, s->pad_w};
  Dims d;
  if (!make_dims(&cs, &d)) return 2;
  const int64_t G = s->groups, D = s->group_ch;
  const int64_t pairs = d.B * d.Ho * d.Wo * G;  // one work item per (pixel, group)
  const int nt = resolve_threads(nthreads, pairs);
  std::vector<std::thread> pool;
  for (int t = 0; t < nt; ++t) {
    pool.emplace_back([&, t]() {
      std::vector<double> a(static_cast<size_t>(d.K));
      for (int64_t n = t; n < pairs; n += nt) {
        const int64_t g = n % G;
        const int64_t p = n / G;  // (b*Ho + ho)*Wo + wo
        const int64_t b = p / (d.Ho * d.Wo);
        const int64_t ho = (p / d.Wo) % d.Ho;
        const int64_t wo = p % d.Wo;
        // aggregation weights of the K taps: weights[b, g*K + k, ho, wo],
        // used as given or as a softmax over the K taps (fp64)
        for (int64_t k = 0; k < d.K; ++k)
          a[k] = weights[((b * G * d.K + g * d.K + k) * d.Ho + ho) * d.Wo + wo];
        if (softmax) {
          double mx = -INFINITY, sum = 0.0;
          for (int64_t k = 0; k < d.K; ++k) mx = std::fmax(mx, a[k]);
          for (int64_t k = 0; k < d.K; ++k) sum += std::exp(a[k] - mx);
          for (int64_t k = 0; k < d.K; ++k) a[k] = std::exp(a[k] - mx) / sum;
        }
        double* orow = &out[p * G * D + g * D];
        double* nrow = norm ? &norm[p * G * D + g * D] : nullptr;
        for (int64_t c = 0; c < D; ++c) {
          orow[c] = 0.0;
          if (nrow) nrow[c] = 0.0;
        }
        for (int64_t k = 0; k < d.K; ++k) {
          const int64_t i = k / d.kw, j = k % d.kw;
          // offset channel (g*K + k)*2 = dy, +1 = dx: the convolution's
          // [B, 2K, Ho, Wo] layout with one block of 2K channels per group
          const int64_t oc = (b * G * 2 * d.K + (g * d.K + k) * 2) * d.Ho * d.Wo + ho * d.Wo + wo;
          const float dy = offset[oc];
          const float dx = offset[oc + d.Ho * d.Wo];
          const Coord cd = tap_coord(d, ho, wo, i, j, dy, dx);
          const double ly = cd.ly, lx = cd.lx;
          const double wgt[2][2] = {{(1.0 - ly) * (1.0 - lx), (1.0 - ly) * lx},
                                    {ly * (1.0 - lx), ly * lx}};
          for (int64_t c = 0; c < D; ++c) {
            double sv = 0.0, sa = 0.0;
            for (int ca = 0; ca < 2; ++ca)
              for (int cb = 0; cb < 2; ++cb) {
                if (!corner_valid(d, cd.y0, cd.x0, ca, cb)) continue;  // outside: 0
                const int64_t yy = static_cast<int64_t>(cd.y0) + ca;
                const int64_t xx = static_cast<int64_t>(cd.x0) + cb;
                const double v = x[((b * d.H + yy) * d.W + xx) * G * D + g * D + c];
                sv += wgt[ca][cb] * v;
                sa += wgt[ca][cb] * std::fabs(v);
              }
            orow[c] += a[k] * sv;
            if (nrow) nrow[c] += std::fabs(a[k]) * sa;
          }
        }
      }
    });
  }
  for (auto& th : pool) th.join();
  return 0;
}
