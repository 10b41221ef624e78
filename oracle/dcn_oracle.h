/*
 * dcn_oracle.h -- CPU oracle for the modulated deformable 2-D convolution
 * forward (DCNv2; stride 1, dilation 1, one offset group, groups = 1).
 *
 * TEST INFRASTRUCTURE ONLY.  This library is the slow, obviously correct
 * definition that the GPU path is checked against.  Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load it.  It
 * shares no code, header, table or helper with the GPU library.
 *
 * What it computes is the operator as page 1 ("deform_conv.py", litert-
 * community/Idol; module docstring and the body of deform_conv2d_gather)
 * states it: for output pixel (h, w) and tap k = (i, j), k = i*kw + j,
 * sample the input bilinearly at (h - pad_h + i + dy_k, w - pad_w + j + dx_k),
 * corners outside the image count as zero, multiply by mask_k, contract over
 * (tap, channel) with weight[o, c, i, j], add bias[o].
 *
 * Precision: the sampling coordinate and its floor/fraction are formed in
 * fp32 (page 1 builds them in the input dtype: an exact integer grid plus
 * one add of the offset); everything after that (bilinear weights, blend,
 * contraction, bias) is fp64.
 *
 * Layouts (all dense, row-major, no padding):
 *   x      [B, H, W, C]       token-major NHWC (page 1, "token-major input")
 *   offset [B, 2K, Ho, Wo]    channel 2k = dy (row), 2k+1 = dx (column)
 *   mask   [B, K, Ho, Wo]     NULL means all ones (v1 deformable conv)
 *   weight [O, C, kh, kw]
 *   bias   [O]                NULL means zero
 * with Ho = H + 2*pad_h - kh + 1, Wo = W + 2*pad_w - kw + 1.
 */
#ifndef DCN_ORACLE_H
#define DCN_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int64_t batch, in_ch, height, width;
  int64_t out_ch, kernel_h, kernel_w;
  int64_t pad_h, pad_w;
} dcn_oracle_shape;

/* Return codes: 0 ok, 1 null pointer, 2 bad shape. */

/*
 * Forward on a list of output pixels.
 *   pixels  linear pixel ids p = (b*Ho + ho)*Wo + wo, or NULL for all B*Ho*Wo
 *           pixels in order (then npixels must equal B*Ho*Wo).
 *   out     [npixels, O] fp64: bias[o] + sum_k sum_c weight[o,c,i_k,j_k]*s[k][c]
 *   norm    [npixels, O] fp64 (may be NULL): sum_k sum_c |weight| * |s[k][c]|,
 *           the error normaliser (it excludes the bias).
 *   nthreads <= 0 means std::thread::hardware_concurrency().
 * Every element's arithmetic is independent of the thread count.
 */
int dcn_oracle_forward(const dcn_oracle_shape* s, const float* x, const float* offset,
                       const float* mask, const float* weight, const float* bias,
                       const int64_t* pixels, int64_t npixels, double* out, double* norm,
                       int nthreads);

/*
 * Sampling corners alone, for every (b, k, ho, wo):
 *   y0x0   [B, K, Ho, Wo, 2] int32: floor of the fp32 sampling row / column
 *          (defined when |floor| < 2^31)
 *   valid4 [B, K, Ho, Wo] uint8: bit (2a + b) set when corner (y0+a, x0+b)
 *          lies inside the image.
 */
int dcn_oracle_coords(const dcn_oracle_shape* s, const float* offset, int32_t* y0x0,
                      uint8_t* valid4, int nthreads);

/*
 * Backward: the gradients of a scalar loss L given g = dL/dout, obtained by
 * differentiating the forward above term by term (the pages state the
 * forward only; this is its exact derivative).  The sampling value is
 * piecewise bilinear in the offsets; the offset gradient is its derivative
 * inside the floor cell of the sampling point (d ly / d dy = d lx / d dx = 1,
 * with floor and validity held fixed), corners outside the image contribute
 * nothing.
 *   grad_out [B, O, Ho, Wo] fp32 (the forward's NCHW layout)
 * Outputs (fp64; any may be NULL; each non-NULL one is fully written):
 *   gx    [B, H, W, C]      dL/dx
 *   goff  [B, 2K, Ho, Wo]   dL/doffset (channel 2k: dy, 2k+1: dx)
 *   gmask [B, K, Ho, Wo]    dL/dmask (also when mask is NULL, at mask = 1)
 *   gw    [O, C, kh, kw]    dL/dweight
 *   gb    [O]               dL/dbias
 * and normalisers of the same shapes (any may be NULL): the sum of the
 * absolute values of the terms of each gradient element, with the inner
 * contraction sum_o g[o] * weight[o, c, k] expanded into absolute terms too.
 * Gradients are sums over output pixels: each thread accumulates its own
 * copy and the copies are added in thread order, so a given nthreads always
 * gives the same bits (memory: one copy of gx and gw per thread).
 */
int dcn_oracle_backward(const dcn_oracle_shape* s, const float* x, const float* offset,
                        const float* mask, const float* weight, const float* grad_out,
                        double* gx, double* goff, double* gmask, double* gw, double* gb,
                        double* ngx, double* ngoff, double* ngmask, double* ngw, double* ngb,
                        int nthreads);

/*
 * Multi-scale deformable attention sampling (page 5, deformops README,
 * "Multi-scale deformable attention": value (B, sum H*W, G, D), per-level
 * shapes and start offsets, locations (B, Q, G, L, K, 2) normalised to
 * [0, 1], weights (B, Q, G, L*K) used as given or normalised by a softmax
 * over levels and points).  For each (b, q, g):
 *   out[b, q, g, :] = sum_{l, k} a[l, k] * bilinear(value level l, head g, at p)
 * with p = (x * W_l - 0.5, y * H_l - 0.5) in pixels (location component 0 is
 * x, the column; 1 is y, the row), each product and difference rounded to
 * fp32 (no fused multiply-add); corners outside the level count as zero.
 *   shapes  [L][2] (H_l, W_l); starts[l] = sum_{m < l} H_m W_m
 *   out     [B, Q, G, D] fp64; norm (may be NULL) the absolute-term sum
 *           sum a * w_corner * |value| with |a|.
 * softmax != 0: a = softmax over the L*K logits of (b, q, g) (fp64).
 */
int dcn_oracle_msda(int64_t B, int64_t S, int64_t G, int64_t D, int64_t Q, int64_t L, int64_t K,
                    const int64_t* shapes, const float* value, const float* locations,
                    const float* weights, int softmax, double* out, double* norm, int nthreads);

/*
 * Single-scale deformable sampling (page 5, deformops README, "Single-scale
 * deformable sampling": the DCNv3 operator of InternImage, sampling and
 * aggregation without the spatial weight of deformable convolution).  The
 * channels are G groups of D; each group has its own offsets and one
 * aggregation weight per (tap, pixel).  For output (b, ho, wo) and channel
 * g*D + c:
 *   out = sum_k a[b, g, k, ho, wo] *
 *         bilinear(x[b, :, :, g*D + c], ho - pad_h + i_k + dy, wo - pad_w + j_k + dx)
 * with the sampling point, floor, fractions and corner validity exactly as
 * in dcn_oracle_forward (stride 1, dilation 1, tap k = i*kw + j).
 *   x       [B, H, W, G*D]     NHWC
 *   offset  [B, G*2K, Ho, Wo]  channel (g*K + k)*2 = dy, (g*K + k)*2 + 1 = dx
 *   weights [B, G*K, Ho, Wo]   a of (g, k) at channel g*K + k; logits when
 *                              softmax != 0 (a = softmax over the K taps of
 *                              one (b, g, ho, wo), in fp64)
 *   out     [B, Ho, Wo, G*D] fp64 (NHWC); norm (may be NULL) the same shape:
 *           sum_k |a| * sum_corners w * |x|.
 */
typedef struct {
  int64_t batch, groups, group_ch, height, width;
  int64_t kernel_h, kernel_w, pad_h, pad_w;
} dcn_oracle_ds_shape;

int dcn_oracle_dsample(const dcn_oracle_ds_shape* s, const float* x, const float* offset,
                       const float* weights, int softmax, double* out, double* norm,
                       int nthreads);

#ifdef __cplusplus
}
#endif
#endif
