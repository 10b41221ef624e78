/*
 * dcn.h -- C ABI of the MI355X (gfx950) modulated deformable conv2d forward.
 *
 * The operation (page 1, "deform_conv.py", litert-community/Idol: module
 * docstring and deform_conv2d_gather; page 5, deformops README, section
 * "Deformable convolution"): for every output pixel (h, w) and kernel tap
 * k = (i, j), k = i*kw + j, sample the input bilinearly at
 *     (h - pad_h + i + dy_k,  w - pad_w + j + dx_k),
 * with each of the four neighbouring corners that lies outside the image
 * counting as zero; multiply the sample by mask_k; contract over
 * (tap, channel) with weight[o, c, i, j]; add bias[o].  Stride 1,
 * dilation 1, one offset group, groups = 1.  A NULL mask is the unmodulated
 * (v1) operator, i.e. mask = 1 (page 5 "v2 with a mask and v1 without").
 *
 * Layouts (dense, row-major, no padding or strides):
 *   x      [B, H, W, C]       NHWC, "token-major": row (b, y, x) holds the C
 *                             channels of one pixel (page 1 builds exactly
 *                             this token table before gathering)
 *   offset [B, 2K, Ho, Wo]    channel 2k = dy (row), 2k+1 = dx (column) of
 *                             tap k (page 1 views it as [B, K, 2, Ho, Wo])
 *   mask   [B, K, Ho, Wo]     or NULL
 *   weight [O, C, kh, kw]     the usual conv weight
 *   bias   [O]                or NULL (zero)
 *   out    [B, O, Ho, Wo] (DCN_OUT_NCHW) or [B, Ho, Wo, O] (DCN_OUT_NHWC)
 * with Ho = H + 2*pad_h - kh + 1 and Wo = W + 2*pad_w - kw + 1.
 * x, offset, mask, weight and bias all have the plan's in_dtype; out is fp32.
 * Accumulation is fp32 for every dtype (page 5: float32 accumulation, no
 * TF32-style reduced-precision contraction).
 *
 * Memory: every pointer passed to a dcn_* call that takes a stream is a
 * DEVICE pointer (hipMalloc / torch CUDA tensor) on the current device, and
 * must be 16-byte aligned.  The caller owns all device memory, including the
 * workspace; the library never allocates or frees device memory and never
 * synchronises.  A plan owns only host memory and is immutable after
 * dcn_create, so one plan may be used from several threads at once.
 *
 * Streams: `stream` is a hipStream_t (NULL = the legacy default stream).
 * Calls are asynchronous on that stream; device-side faults surface at the
 * caller's next synchronisation, as for any HIP launch.
 *
 * Errors: every call returns a dcn_status; no C++ exception crosses the ABI.
 * Descriptor problems are reported by dcn_create; pointer problems by the
 * call that receives the pointer.  dcn_last_error() gives a message for the
 * most recent failure on the calling thread.
 */
#ifndef DCN_H
#define DCN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct dcn_plan_s* dcn_plan;

typedef enum {
  DCN_OK = 0,
  DCN_E_NULL = 1,        /* a required pointer is NULL                     */
  DCN_E_SHAPE = 2,       /* sizes out of range, Ho or Wo <= 0, overflow     */
  DCN_E_DTYPE = 3,       /* unknown dtype / layout value                    */
  DCN_E_UNSUPPORTED = 4, /* valid operator, but outside this build's limits */
  DCN_E_ALIGN = 5,       /* a device pointer is not 16-byte aligned         */
  DCN_E_HIP = 6,         /* a HIP runtime call or kernel launch failed      */
  DCN_E_INTERNAL = 7,    /* unexpected host-side failure                    */
  DCN_E_WORKSPACE = 8    /* workspace NULL or smaller than required         */
} dcn_status;

typedef enum { DCN_F32 = 0, DCN_BF16 = 1 } dcn_dtype;
typedef enum { DCN_OUT_NCHW = 0, DCN_OUT_NHWC = 1 } dcn_layout;

/*
 * Problem descriptor.  Limits of this build (DCN_E_UNSUPPORTED otherwise):
 *   in_ch  a multiple of 4 (fp32) or 8 (bf16): each pixel's channel vector is
 *          fetched with 16-byte loads
 *   the bytes of x, and B*O*Ho*Wo*4, below 2^31
 *   out_dtype DCN_F32
 * Any kernel_h, kernel_w >= 1 and pad >= 0 with Ho, Wo >= 1 is accepted.
 */
typedef struct {
  int32_t batch;      /* B                                   */
  int32_t in_ch;      /* C                                   */
  int32_t height;     /* H                                   */
  int32_t width;      /* W                                   */
  int32_t out_ch;     /* O                                   */
  int32_t kernel_h;   /* kh                                  */
  int32_t kernel_w;   /* kw                                  */
  int32_t pad_h;      /* ph (zero padding of the grid, rows)  */
  int32_t pad_w;      /* pw                                  */
  int32_t in_dtype;   /* dcn_dtype of x/offset/mask/weight/bias */
  int32_t out_dtype;  /* dcn_dtype of out: DCN_F32            */
  int32_t out_layout; /* dcn_layout                           */
} dcn_desc;

/* Validate `desc` and build a plan (host memory only).  *plan is set to NULL
 * on failure.  Does not touch the GPU. */
dcn_status dcn_create(const dcn_desc* desc, dcn_plan* plan);

/* Free a plan.  NULL is accepted and ignored. */
dcn_status dcn_destroy(dcn_plan plan);

/* Output size of a plan: Ho, Wo (either pointer may be NULL). */
dcn_status dcn_output_size(dcn_plan plan, int32_t* ho, int32_t* wo);

/* Bytes of device workspace a forward call runs fastest with: the weight
 * repacked as [tap][channel block][out channel] tiles (page 1 reorders the
 * weight to rows (i, j, c), columns o before its one matmul), zero-padded to
 * the kernel's tile sizes, then -- for plans whose grid would leave most of
 * the GPU idle even with two tap groups per workgroup (see dcn_tap_schedule)
 * -- scratch for a split of the tap sum: the taps are divided into up to 4
 * runs computed side by side into fp32 partial outputs that a second kernel
 * adds (in run order, deterministic) together with the bias. */
dcn_status dcn_workspace_bytes(dcn_plan plan, size_t* bytes);

/* How the plan's forward divides the sum over the K taps (fp32 plans with
 * 17..64 output channels and few output tiles; every other plan reports 1,
 * K, 1):
 *   *runs          workgroups per output tile, each summing a contiguous run
 *                  of taps into a partial output (1: no split; used only when
 *                  the workspace holds dcn_workspace_bytes bytes)
 *   *taps_per_run  taps per run (the last run may have fewer)
 *   *groups        tap groups inside each workgroup: 2 = 8 waves, each half
 *                  summing half of the workgroup's taps, the halves added in
 *                  on-chip memory (no workspace needed)
 * Any pointer may be NULL.  The choice is the whole map's; row-band calls use
 * it too, so bands stay bit-identical to the whole-map call. */
dcn_status dcn_tap_schedule(dcn_plan plan, int32_t* runs, int32_t* taps_per_run,
                            int32_t* groups);

/* Bytes of the packed weight at the start of the workspace (<= the
 * dcn_workspace_bytes size).  dcn_pack_weight writes only these bytes; a
 * forward call given a workspace of fewer than dcn_workspace_bytes bytes
 * (but at least these) runs without the tap split. */
dcn_status dcn_packed_weight_bytes(dcn_plan plan, size_t* bytes);

/* Repack `weight` [O, C, kh, kw] into `workspace` (device, >= the size
 * dcn_packed_weight_bytes reports).  One kernel launch on `stream`.  Callers
 * whose weight does not change may call this once and then reuse the
 * packed workspace with dcn_forward_packed. */
dcn_status dcn_pack_weight(dcn_plan plan, const void* weight, void* workspace,
                           size_t workspace_bytes, void* stream);

/* The forward from an already packed weight: one fused kernel launch on
 * `stream` (sampling point, bilinear gather and modulation into an on-chip
 * column tile, MFMA contraction, bias epilogue); with the tap split (see
 * dcn_workspace_bytes) the fused kernel writes partial sums into the
 * workspace's scratch and a reduce kernel writes `out`.  `workspace` holds
 * the packed weight (dcn_pack_weight) in its first dcn_packed_weight_bytes
 * bytes, which are only read; `workspace_bytes` (>= dcn_packed_weight_bytes,
 * else DCN_E_WORKSPACE) is its size, and bytes beyond the packed weight are
 * overwritten when the call splits its taps: calls that may overlap in time
 * (different streams) then need workspaces of their own.  `mask` and `bias`
 * may be NULL.  `out` must not overlap any input or the workspace. */
dcn_status dcn_forward_packed(dcn_plan plan, const void* x, const void* offset,
                              const void* mask, void* workspace, size_t workspace_bytes,
                              const void* bias, void* out, void* stream);

/* The whole forward: dcn_pack_weight then dcn_forward_packed, both on
 * `stream`, with one workspace (>= dcn_packed_weight_bytes bytes;
 * dcn_workspace_bytes enables the tap split). */
dcn_status dcn_forward(dcn_plan plan, const void* x, const void* offset, const void* mask,
                       const void* weight, const void* bias, void* out, void* workspace,
                       size_t workspace_bytes, void* stream);

/* A band of output rows (page 1, deform_conv2d_gather's row0 argument: the
 * offsets and mask of a call may cover a horizontal strip of the output
 * only, while x is always the whole input map).  Computes output rows
 * [row0, row0 + rows) of the plan's operator from an already packed weight:
 *   offset [B, 2K, rows, Wo], mask [B, K, rows, Wo] or NULL  -- the band's
 *          rows only (row r of the band is output row row0 + r)
 *   out    [B, O, rows, Wo] (NCHW) or [B, rows, Wo, O] (NHWC), fp32
 *   x, workspace, bias exactly as for dcn_forward_packed.
 * Sampling points use the absolute output row, so the bands of a partition
 * of [0, Ho) reproduce dcn_forward_packed's output row for row.
 * DCN_E_SHAPE unless 0 <= row0, 0 <= rows and row0 + rows <= Ho; rows == 0
 * is a no-op.  One fused kernel launch on `stream` (plus the reduce when
 * the band's grid splits its taps). */
dcn_status dcn_forward_rows(dcn_plan plan, int32_t row0, int32_t rows, const void* x,
                            const void* offset, const void* mask, void* workspace,
                            size_t workspace_bytes, const void* bias, void* out,
                            void* stream);

/* Several deformable convolutions on ONE input map in one call (page 2: the
 * BiRefNet decoder's deformable ASPP blocks run four branches on the same
 * map).  Branch i is plans[i]'s operator with its own offsets[i], masks[i]
 * (or NULL), packed_weights[i] (from dcn_pack_weight with plans[i],
 * workspace_bytes[i] bytes), biases[i] (or NULL) and outs[i]; x is shared.
 * `masks` and `biases` may themselves be NULL (no branch has one).  All
 * plans must read the same input (batch, in_ch, height, width, in_dtype:
 * else DCN_E_SHAPE); kernel size, padding, out_ch and out_layout may
 * differ.  Branches that run the same kernel variant share ONE launch (the
 * workgroups of all of them in one grid); 1 <= n <= 8 (n == 0 is a no-op,
 * more is DCN_E_UNSUPPORTED).  Per-branch pointer rules and errors as for
 * dcn_forward_packed, but the branches never split their taps (the common
 * grid is already wide) and the workspaces are only read; nothing is
 * launched unless every branch validates. */
dcn_status dcn_forward_multi(int32_t n, const dcn_plan* plans, const void* x,
                             const void* const* offsets, const void* const* masks,
                             const void* const* packed_weights, const size_t* workspace_bytes,
                             const void* const* biases, void* const* outs, void* stream);

/* Backward of the forward (plans with out_ch <= 256; DCN_E_UNSUPPORTED
 * otherwise): given grad_out = dL/dout in the plan's output layout (fp32,
 * like out), writes fp32
 *   grad_x      [B, H, W, C]       dL/dx (NHWC, like x)
 *   grad_offset [B, 2K, Ho, Wo]    dL/doffset (channel 2k: dy, 2k+1: dx)
 *   grad_mask   [B, K, Ho, Wo]     dL/dmask (with a NULL mask: at mask = 1)
 *   grad_weight [O, C, kh, kw]     dL/dweight
 *   grad_bias   [O]                dL/dbias
 * Any gradient pointer may be NULL (not computed); every non-NULL one is
 * fully overwritten.  The gradients are the exact derivative of the forward
 * (the pages define the forward only): the sample is bilinear inside the
 * floor cell of the sampling point, so the offset gradient is the derivative
 * inside that cell with the floor and corner validity held fixed, and
 * corners outside the image contribute nothing.  The input, offset and mask
 * gradients are sums over many output pixels and taps accumulated with fp32
 * atomic adds (page 5 names atomic adds into fp32 accumulators as the way
 * these gradients are gathered), so they are not bitwise repeatable.
 * Operands x, offset, mask and weight have the plan's in_dtype.  For bf16
 * plans they are first widened exactly into fp32 copies in the workspace, and
 * the backward then accumulates and writes fp32 (page 5, "Backend
 * selection": half-precision training with a float32 accumulator).
 * workspace: >= dcn_backward_workspace_bytes (the weight re-packed for the
 * input-gradient contraction, plus the fp32 copies for bf16 plans), device,
 * 16-byte aligned.  x, grad_x: 16-byte aligned; offset, mask, weight
 * element-aligned; the rest 4-byte aligned.  Asynchronous on `stream`. */
dcn_status dcn_backward_workspace_bytes(dcn_plan plan, size_t* bytes);
dcn_status dcn_backward(dcn_plan plan, const void* x, const void* offset, const void* mask,
                        const void* weight, const void* grad_out, void* grad_x,
                        void* grad_offset, void* grad_mask, void* grad_weight, void* grad_bias,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Multi-scale deformable attention sampling (page 5, deformops README,
 * "Multi-scale deformable attention"; the second operator on the same
 * gather machinery).  Shapes: B batch, G heads, D channels per head, Q
 * queries, L levels of sizes H_l x W_l, K points per level, S = sum H_l W_l.
 *   value     [B, S, G, D]       the L feature maps, flattened row-major and
 *                                concatenated (level l starts at
 *                                sum_{m<l} H_m W_m)
 *   locations [B, Q, G, L, K, 2] normalised (x, y): component 0 is the
 *                                column, 1 the row, (0, 0) the top-left edge
 *   weights   [B, Q, G, L*K]     attention weights, or logits when
 *                                desc.softmax != 0 (then normalised over the
 *                                L*K points of each (b, q, g) in the kernel)
 *   out       [B, Q, G, D]       = [B, Q, G*D]
 *   out[b,q,g,:] = sum_{l,k} a * bilinear(level l, head g, at
 *                  (x * W_l - 0.5, y * H_l - 0.5) pixels)
 * with each product / difference of the pixel coordinate rounded to fp32
 * and corners outside the level counting as zero.  value, locations and
 * weights share the plan's dtype (DCN_F32 or DCN_BF16; page 5: half
 * precision throughout); bf16 values are widened exactly, blending and
 * accumulation are fp32 and out is fp32.  L <= 8, K <= 8, D a multiple of 4
 * (fp32) or 8 (bf16), at most 1024.  level_hw is a HOST array [L][2] of
 * (H_l, W_l) copied into the plan.  The value buffer must hold exactly S
 * positions (dcn_msda_value_positions).
 */
typedef struct dcn_msda_plan_s* dcn_msda_plan;
typedef struct {
  int32_t batch, num_queries, num_heads, head_dim, num_levels, num_points;
  int32_t dtype;    /* DCN_F32 or DCN_BF16: value, locations and weights */
  int32_t softmax;  /* 0: weights as given; 1: softmax of logits */
} dcn_msda_desc;
dcn_status dcn_msda_create(const dcn_msda_desc* desc, const int32_t* level_hw,
                           dcn_msda_plan* plan);
dcn_status dcn_msda_destroy(dcn_msda_plan plan);
dcn_status dcn_msda_value_positions(dcn_msda_plan plan, int32_t* positions);
/* One kernel launch on `stream`; value and out 16-byte aligned, locations
 * and weights element-aligned; no input may overlap out. */
dcn_status dcn_msda_forward(dcn_msda_plan plan, const void* value, const void* locations,
                            const void* weights, void* out, void* stream);

/*
 * Single-scale deformable sampling (page 5, deformops README, "Single-scale
 * deformable sampling": the DCNv3 operator of InternImage, which samples and
 * aggregates without the spatial weight of deformable convolution).  The
 * C = G*D channels are G groups of D; each group has its own offsets and one
 * aggregation weight a per (tap, pixel).  For output (b, ho, wo) and channel
 * g*D + c:
 *   out = sum_k a[b, g*K + k, ho, wo] *
 *         bilinear(x[b, :, :, g*D + c], ho - pad_h + i + dy, wo - pad_w + j + dx)
 * with tap k = i*kw + j, the sampling point, floor and corner validity of
 * the deformable convolution above (corners outside count as zero), and a
 * used as given (softmax = 0) or normalised by a softmax over the K taps of
 * each (b, g, ho, wo) (softmax = 1).  Stride 1, dilation 1.
 *   x       [B, H, W, G*D]      NHWC, dtype
 *   offset  [B, G*2K, Ho, Wo]   channel (g*K + k)*2 = dy, +1 = dx, dtype
 *   weights [B, G*K, Ho, Wo]    a (or logits), dtype
 *   out     [B, Ho, Wo, G*D] (DCN_OUT_NHWC) or [B, G*D, Ho, Wo] (DCN_OUT_NCHW), fp32
 * Limits (DCN_E_UNSUPPORTED otherwise): group_ch a multiple of 4 (fp32) or 8
 * (bf16); x and offset below 2^31 bytes.  Accumulation is fp32.
 */
typedef struct dcn_dsample_plan_s* dcn_dsample_plan;
typedef struct {
  int32_t batch, groups, group_ch, height, width;
  int32_t kernel_h, kernel_w, pad_h, pad_w;
  int32_t dtype;       /* dcn_dtype of x, offset, weights */
  int32_t softmax;     /* 0: weights as given; 1: softmax over the K taps */
  int32_t out_layout;  /* dcn_layout */
} dcn_dsample_desc;
dcn_status dcn_dsample_create(const dcn_dsample_desc* desc, dcn_dsample_plan* plan);
dcn_status dcn_dsample_destroy(dcn_dsample_plan plan);
dcn_status dcn_dsample_output_size(dcn_dsample_plan plan, int32_t* ho, int32_t* wo);
/* One kernel launch on `stream`; x and out 16-byte aligned, offset and
 * weights element-aligned; out must not overlap an input. */
dcn_status dcn_dsample_forward(dcn_dsample_plan plan, const void* x, const void* offset,
                               const void* weights, void* out, void* stream);

/* Layout conversion for callers holding NCHW input (page 5's torchvision
 * drop-in takes torchvision's argument order and NCHW layout): writes
 * dst[b, y, x, c] = src[b, c, y, x] for a [batch, channels, height, width]
 * tensor of `dtype` (DCN_F32 or DCN_BF16).  src and dst are device buffers of
 * batch*channels*height*width elements, 16-byte aligned, not overlapping.
 * One LDS-tiled transpose kernel on `stream`; a zero-sized tensor is a
 * no-op; DCN_E_SHAPE for negative sizes or more than 2^31 - 1 elements. */
dcn_status dcn_nchw_to_nhwc(const void* src, void* dst, int32_t batch, int32_t channels,
                            int32_t height, int32_t width, int32_t dtype, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops or harnesses that forbid hipMalloc): the whole
 * forward of dcn_forward without a caller workspace.  The packed weight (and,
 * when it fits, the tap split's partial sums) live in a static device array of
 * DCN_NOALLOC_SCRATCH_BYTES bytes that the library holds on every GPU it runs
 * on until the process ends; the call itself allocates nothing.  Arguments,
 * layouts and errors as for dcn_forward; DCN_E_UNSUPPORTED when the plan's
 * packed weight is larger than the array.  Every call on one GPU uses that
 * GPU's one array, so calls that may overlap in time on one GPU (different
 * streams, or different host threads) race and must be serialised by the
 * caller; calls on one stream are ordered and safe.  The first call on a
 * device resolves the array's address there (a host-side runtime query). */
#define DCN_NOALLOC_SCRATCH_BYTES (32u << 20)
dcn_status dcn_forward_noalloc(dcn_plan plan, const void* x, const void* offset,
                               const void* mask, const void* weight, const void* bias,
                               void* out, void* stream);

/* Test hook, not on the timed path: the sampling-corner stage alone (the
 * floor of the sampling point and the validity of its four corners, page 1
 * "deform_conv.py", deform_conv2d_gather: torch.floor and the `valid`
 * comparison), from the device functions every kernel builds its corner
 * table with.  For every (b, k, ho, wo) it writes y0x0[2e], y0x0[2e+1] =
 * floor of the fp32 sampling row / column (saturated to int32) and
 * valid4[e] = bit (2a + b) set when corner (y0 + a, x0 + b) is inside the
 * image, where e = ((b*K + k)*Ho + ho)*Wo + wo.  Both are device buffers of
 * B*K*Ho*Wo (x2 for y0x0) elements. */
dcn_status dcn_debug_coords(dcn_plan plan, const void* offset, int32_t* y0x0, uint8_t* valid4,
                            void* stream);

/* Test hook: exactly dcn_forward_packed (same kernel, same launch, `out`
 * written as usual), and in addition the fused kernel exports the corner
 * table it builds and gathers from -- for every (b, k, pixel p = ho*Wo + wo)
 * and corner c = 2a + b of the sampling point's floor (y0, x0):
 *   corner_index[e] = (b*H + y0 + a)*W + x0 + b, the input pixel the corner
 *                     loads, or -1 for a corner outside the image (not loaded)
 *   corner_weight[e] = bilinear weight x mask of that corner as the blend
 *                     uses it (0 outside; rounded to bf16 in the wide bf16
 *                     kernel), with e = ((b*K + k)*Ho*Wo + p)*4 + c.
 * Both are device buffers of B*K*Ho*Wo*4 elements, 4-byte aligned. */
dcn_status dcn_debug_corner_table(dcn_plan plan, const void* x, const void* offset,
                                  const void* mask, void* workspace, size_t workspace_bytes,
                                  const void* bias, void* out, int32_t* corner_index,
                                  float* corner_weight, void* stream);

/* Static string naming a status. */
const char* dcn_status_string(dcn_status status);

/* Message describing the most recent failing call on this thread ("" if none). */
const char* dcn_last_error(void);

/* ABI version: major * 10000 + minor * 100 + patch. */
int32_t dcn_version(void);

#ifdef __cplusplus
}
#endif
#endif /* DCN_H */
