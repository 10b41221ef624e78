// dcn_launch.h -- internal interface between the C ABI (dcn_api.cpp) and the
// kernels (dcn_kernels.hip).  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace dcn {

// Tile configuration chosen once per plan.
struct KernelConfig {
  int kind;       // 0: shared column tile (dcn_kernels.hip), 1: k split over waves
                  // (dcn_wsk.hip), 2: 32 pixels x 32 channels per wave (dcn_quad.hip),
                  // 3: bf16, 128 pixels x 256 outputs per workgroup (dcn_bf16.hip),
                  // 4: bf16, 8 x 16 pixels x 256 outputs, corners from an LDS
                  //    window (dcn_bf16win.hip)
  int bf16;       // 0: fp32 operands, 1: bf16 operands
  int M;          // output pixels per workgroup
  int CB;         // channels per k-block (one tap, one channel chunk)
  int NO;         // output channels per workgroup (padded)
  int nhwc;       // output layout: 0 NCHW, 1 NHWC
  int nchunk;     // ceil(C / CB)
  int n_otiles;   // ceil(O / NO)
  int tiles_per_img;  // ceil(Ho*Wo / M); kind 4: 2-D tiles, ceil(Ho / 8) * ceil(Wo / 16)
};

// Arguments of the fused forward kernel (passed by value).
struct FusedArgs {
  const void* x;       // [B,H,W,C] in_dtype
  const void* offset;  // [B,2K,Ho,Wo] in_dtype
  const void* mask;    // [B,K,Ho,Wo] in_dtype or nullptr
  const void* wpack;   // packed weight (see dcn_pack_weight)
  const void* bias;    // [O] in_dtype or nullptr
  float* out;          // [B,O,Ho,Wo] or [B,Ho,Wo,O] fp32
  int B, C, H, W, O, kh, kw, K, ph, pw, Ho, Wo, HoWo;
  int nchunk, n_otiles, tiles_per_img;
  int tiles_x;         // kind 4: 16-column tiles per tile row
  uint32_t x_bytes;    // bytes of x (< 2^31)
  uint32_t offset_bytes;  // bytes of offset (< 2^31)
  uint32_t mask_bytes;    // bytes of mask (< 2^31; 0 when mask is NULL)
  int vec_store;       // NCHW: Ho*Wo % 4 == 0, so 4 consecutive pixels store as one 16-B write
  // Split of the tap sum (32x32-per-wave kernel only; the others need nsplit 1):
  // split s sums taps [s * kper, min(K, (s + 1) * kper)) into out + s * split_stride,
  // without bias; a reduce adds the splits and the bias afterwards.
  int nsplit;          // 1: the whole sum plus bias, straight into out
  int kper;            // taps per split (K when nsplit is 1)
  uint32_t split_stride;  // floats between consecutive splits' partial outputs
  // Tap groups inside each workgroup (32x32-per-wave kernel only, else 1):
  // 2 = 8-wave workgroups whose two 4-wave groups each sum half of the
  // split's taps, added in LDS; every split then has at least 2 taps.
  int wsplit;
  // Test hook (dcn_debug_corner_table; nullptr on every other call): the
  // kernel also writes each (b, tap, pixel)'s corner-table entry as it builds
  // it -- corner token index (b*H + y)*W + x (-1 for an outside corner) and
  // corner weight -- into [B, K, Ho*Wo, 4] arrays, corner (a, b) at 2a + b.
  int32_t* dbg_corner;
  float* dbg_weight;
};

// Arguments of the fp32 backward kernels (dcn_backward.hip).
struct BwdArgs {
  const float* x;       // [B,H,W,C]
  const float* offset;  // [B,2K,Ho,Wo]
  const float* mask;    // [B,K,Ho,Wo] or nullptr (ones)
  const float* gout;    // dL/dout, [B,O,Ho,Wo] or [B,Ho,Wo,O] (nhwc_g)
  const float* wt;      // weight re-packed for the data gradient (workspace)
  float* gx;            // [B,H,W,C]    or nullptr: not wanted
  float* goff;          // [B,2K,Ho,Wo] or nullptr
  float* gmask;         // [B,K,Ho,Wo]  or nullptr
  float* gw;            // [O,C,kh,kw]  or nullptr
  float* gb;            // [O]          or nullptr
  int B, C, H, W, O, kh, kw, K, ph, pw, Ho, Wo, HoWo;
  int nchunk;           // ceil(C / 64)
  int tiles_per_img;    // ceil(Ho*Wo / 64)
  int nhwc_g;
  uint32_t x_bytes;
};

// Floats of workspace the backward needs; the launch zero-fills the
// gradients it writes, re-packs the weight and runs the three kernels.
int64_t bwd_workspace_floats(int O, int C, int K);
// bf16 -> fp32 copy of n elements (exact), one kernel on `stream`.
hipError_t launch_widen_bf16(const void* src, float* dst, int64_t n, hipStream_t stream);
hipError_t launch_backward(const BwdArgs& a, const float* weight, float* workspace,
                           hipStream_t stream);

// Multi-scale deformable attention sampling (dcn_msda.hip), fp32.
constexpr int kMsdaMaxLevels = 8;
constexpr int kMsdaMaxPoints = 8;
struct MsdaArgs {
  const void* value;       // [B, S, G, D]               operand dtype
  const void* locations;   // [B, Q, G, L, K, 2] normalised (x, y), operand dtype
  const void* weights;     // [B, Q, G, L*K]             operand dtype
  float* out;              // [B, Q, G, D]
  int64_t npairs;          // B * Q * G
  int B, S, G, D, Q, L, K, softmax;
  int H[kMsdaMaxLevels], W[kMsdaMaxLevels], start[kMsdaMaxLevels];
  uint32_t value_bytes;
};
hipError_t launch_msda(const MsdaArgs& a, int bf16, hipStream_t stream);

// Single-scale deformable sampling (dcn_dsample.hip): x [B,H,W,G*D] NHWC,
// offset [B,G*2K,Ho,Wo] (channel (g*K + k)*2 = dy), weights [B,G*K,Ho,Wo]
// (logits when softmax), out [B,Ho,Wo,G*D] or [B,G*D,Ho,Wo] fp32.
struct DsArgs {
  const void* x;
  const void* offset;
  const void* weights;
  float* out;
  int B, G, D, H, W, kh, kw, K, ph, pw, Ho, Wo, HoWo;
  int softmax;
  int tiles_per_img;   // ceil(Ho*Wo / 64)
  int n_ctiles;        // channel tiles of dsample_vectors_per_tile() vectors
  uint32_t x_bytes, offset_bytes, weights_bytes;
};
// 16-byte vectors per workgroup channel tile (4, 8 or 16) for C channels.
int dsample_vectors_per_tile(int C, int bf16);
hipError_t launch_dsample(const DsArgs& a, int bf16, int nhwc, hipStream_t stream);

// Several branches (same input map, own offsets/mask/weight/bias/output and
// kernel size) in one launch: branch i owns the logical workgroups
// [start[i], start[i+1]).
constexpr int kMaxBranches = 8;
struct MultiArgs {
  int n;
  int start[kMaxBranches + 1];
  FusedArgs a[kMaxBranches];
};

// Kernel variants compiled into the library; false if none matches.
bool config_supported(const KernelConfig& kc);

// Elements (of the operand dtype) of the packed weight for `kc`, C/O/K sizes.
int64_t packed_weight_elems(const KernelConfig& kc, int K);

hipError_t launch_pack(const KernelConfig& kc, const void* weight, void* wpack, int O, int C,
                       int kh, int kw, hipStream_t stream);

hipError_t launch_fused(const KernelConfig& kc, const FusedArgs& a, hipStream_t stream);

// One launch over all branches of `m` (kinds 1..3; every branch's config must
// match `kc` up to tiles_per_img / n_otiles, which `m.start` accounts for).
// hipErrorInvalidConfiguration for the general kernel (kind 0).
hipError_t launch_fused_multi(const KernelConfig& kc, const MultiArgs& m, hipStream_t stream);

// The k-split-over-waves kernel (fp32, 64- or 128-wide output tiles).
bool wsk_supported(const KernelConfig& kc);
hipError_t launch_fused_wsk(const KernelConfig& kc, const FusedArgs& a, hipStream_t stream);
hipError_t launch_fused_wsk_multi(const KernelConfig& kc, const MultiArgs& m, hipStream_t stream);

// The 32-pixel x 32-channel-per-wave kernel (fp32, 64-wide output tiles).
bool quad_supported(const KernelConfig& kc);
hipError_t launch_fused_quad(const KernelConfig& kc, const FusedArgs& a, hipStream_t stream);
// out[i] = bias[o(i)] + sum over s < nsplit of part[s * stride + i], i < B*O*Ho*Wo,
// summed in split order (deterministic); o(i) from the output layout.
hipError_t launch_split_reduce(const float* part, int nsplit, uint32_t stride, const float* bias,
                               float* out, int B, int O, int HoWo, int nhwc, hipStream_t s);
hipError_t launch_fused_quad_multi(const KernelConfig& kc, const MultiArgs& m, hipStream_t stream);

// The wide bf16 kernel (128 pixels x 256 output channels per workgroup).
bool bf16w_supported(const KernelConfig& kc);
hipError_t launch_fused_bf16w(const KernelConfig& kc, const FusedArgs& a, hipStream_t stream);
hipError_t launch_fused_bf16w_multi(const KernelConfig& kc, const MultiArgs& m, hipStream_t stream);

// The wide bf16 kernel with an LDS input window (kh, kw <= 3, C % 64 == 0).
bool bf16win_supported(const KernelConfig& kc);
bool bf16win_fits(int kh, int kw, int C);
// 2-D tiles of the window kernel for `rows` x Wo output pixels; sets tiles_x.
int bf16win_tiles(int rows, int Wo, int& tiles_x);
hipError_t launch_fused_bf16win(const KernelConfig& kc, const FusedArgs& a, hipStream_t stream);
hipError_t launch_fused_bf16win_multi(const KernelConfig& kc, const MultiArgs& m,
                                      hipStream_t stream);

// dst[b, p, c] = src[b, c, p] for p over height*width pixels.
hipError_t launch_nchw_to_nhwc(int bf16, const void* src, void* dst, int B, int C, int HW,
                               hipStream_t stream);

hipError_t launch_coords(int bf16, const void* offset, int32_t* y0x0, uint8_t* valid4, int B,
                         int K, int kw, int Ho, int Wo, int ph, int pw, int H, int W,
                         hipStream_t stream);

}  // namespace dcn
