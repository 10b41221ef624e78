// dcn_api.cpp -- C ABI of the gfx950 DCNv2 forward (declared in include/dcn.h).
//
// Host side only: descriptor validation, tile-configuration choice, pointer
// checks and kernel launches on the caller's stream.  Nothing here allocates
// device memory or synchronises.  Shapes are refused rather than guessed
// (page 2, "patch_deform.py", refuses a rewrite it cannot prove in range;
// page 5 names its errors instead of falling back silently).

#include "dcn.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <memory>
#include <mutex>
#include <new>

#include "dcn_launch.h"

struct dcn_msda_plan_s {
  dcn_msda_desc d;
  int S;
  int H[dcn::kMsdaMaxLevels], W[dcn::kMsdaMaxLevels], start[dcn::kMsdaMaxLevels];
};

struct dcn_dsample_plan_s {
  dcn_dsample_desc d;
  int K, Ho, Wo;
  int tiles_per_img, n_ctiles;
  uint32_t x_bytes, offset_bytes, weights_bytes;
};

struct dcn_plan_s {
  dcn_desc d;
  int K, Ho, Wo;
  dcn::KernelConfig kc;
  size_t wpack_bytes;    // packed weight at the start of the workspace (256-B multiple)
  size_t ws_bytes;       // + scratch for the split tap sum (0 bytes when the plan never splits)
  int nsplit, kper;      // tap split of the whole-map grid (1, K: none); bands use the same
  int wsplit;            // tap groups per workgroup of the whole-map grid (1 or 2); bands too
  uint32_t x_bytes;
};

namespace {

thread_local char g_last_error[512] = "";

dcn_status fail(dcn_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
dcn_status fail(dcn_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

dcn_status ok() {
  g_last_error[0] = '\0';
  return DCN_OK;
}

constexpr int64_t kLimit31 = int64_t(1) << 31;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Tile configuration for a validated descriptor.
dcn::KernelConfig choose_config(const dcn_desc& d, int Ho, int Wo) {
  dcn::KernelConfig kc{};
  kc.bf16 = d.in_dtype == DCN_BF16;
  const int O = d.out_ch, C = d.in_ch;
  if (!kc.bf16 && O > 16 && O <= 64 && C >= 32) {
    // fp32, up to 64 output channels: each wave owns 32 pixels x 32
    // channels of every k-block, no workgroup barrier (dcn_quad.hip)
    kc.kind = 2;
    kc.CB = 64;
    kc.NO = 64;
    kc.M = 64;
  } else if (kc.bf16 && O > 128 && dcn::bf16win_fits(d.kernel_h, d.kernel_w, C)) {
    // bf16, wide outputs, small kernels: 8 x 16 pixels x 256 output channels
    // per workgroup, corners blended from an LDS input window (dcn_bf16win.hip)
    kc.kind = 4;
    kc.CB = 64;
    kc.NO = 256;
    kc.M = 128;
  } else if (kc.bf16 && O > 128 && C >= 32) {
    // bf16, wide outputs: 128 pixels x 256 output channels per workgroup,
    // one workgroup per CU (dcn_bf16.hip)
    kc.kind = 3;
    kc.CB = C <= 64 ? 64 : C <= 128 ? 128 : 256;
    kc.NO = 256;
    kc.M = 128;
  } else if (!kc.bf16 && O > 16 && O <= 128 && C >= 32) {
    // fp32 with a small output tile: k split over the four waves, no
    // workgroup barrier in the main loop (dcn_wsk.hip)
    kc.kind = 1;
    kc.CB = 64;
    kc.NO = O <= 64 ? 64 : 128;
    kc.M = kc.NO == 64 ? 64 : 32;
  } else {
    kc.kind = 0;
    kc.M = 64;
    kc.NO = O <= 16 ? 16 : O <= 64 ? 64 : O <= 128 ? 128 : 256;
    if (kc.bf16) {
      kc.CB = C <= 32 ? 32 : 64;
    } else {
      kc.CB = C <= 16 ? 16 : (kc.NO == 256 ? 32 : 64);
    }
  }
  kc.nhwc = d.out_layout == DCN_OUT_NHWC;
  kc.nchunk = (int)ceil_div(C, kc.CB);
  kc.n_otiles = (int)ceil_div(O, kc.NO);
  int tiles_x = 0;
  kc.tiles_per_img = kc.kind == 4 ? dcn::bf16win_tiles(Ho, Wo, tiles_x)
                                  : (int)ceil_div((int64_t)Ho * Wo, kc.M);
  return kc;
}

// The 32x32-per-wave kernel holds two 4-wave workgroups per CU (one wave per
// SIMD each); 256 CUs give 512 resident workgroups.  A grid that fills at most
// half of them first runs 8-wave workgroups whose two tap groups each sum half
// of the taps (added in LDS, no partial outputs in memory), so the chip holds
// two waves per SIMD; if even those fill at most half of the 256 resident
// 8-wave workgroups, the tap sum is also split over up to 4 workgroups per
// tile (each split a contiguous run of taps, at least one per tap group) and
// a reduce adds the splits and the bias.
constexpr int64_t kResidentQuadWG = 512;

void choose_split(const dcn::KernelConfig& kc, int K, int64_t nwg, int& nsplit, int& kper,
                  int& wsplit) {
  nsplit = 1;
  kper = K;
  wsplit = 1;
  if (kc.kind != 2 || nwg <= 0 || 2 * nwg > kResidentQuadWG) return;
  if (K >= 2) wsplit = 2;
  const int64_t resident = kResidentQuadWG / wsplit;
  int64_t cap = resident / nwg;
  if (cap > 4) cap = 4;
  if (cap > K / wsplit) cap = K / wsplit;
  for (int ns = (int)cap; ns >= 2; --ns) {
    const int kp = (int)ceil_div(K, ns);
    const int n = (int)ceil_div(K, kp);
    if (K - (n - 1) * kp >= wsplit) {  // the last run keeps a tap per group
      kper = kp;
      nsplit = n;
      return;
    }
  }
}

// Floats between consecutive splits' partial outputs: the output's element
// count rounded up to 64 (keeps every partial 256-byte aligned).
int64_t split_stride(int64_t B, int64_t O, int64_t HoWo) { return (B * O * HoWo + 63) / 64 * 64; }

dcn_status hip_fail(hipError_t e, const char* what) {
  return fail(DCN_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

extern "C" {

int32_t dcn_version(void) { return 10100; }

const char* dcn_status_string(dcn_status s) {
  switch (s) {
    case DCN_OK: return "DCN_OK";
    case DCN_E_NULL: return "DCN_E_NULL: a required pointer is NULL";
    case DCN_E_SHAPE: return "DCN_E_SHAPE: invalid sizes";
    case DCN_E_DTYPE: return "DCN_E_DTYPE: unknown dtype or layout";
    case DCN_E_UNSUPPORTED: return "DCN_E_UNSUPPORTED: outside this build's limits";
    case DCN_E_ALIGN: return "DCN_E_ALIGN: misaligned device pointer";
    case DCN_E_HIP: return "DCN_E_HIP: HIP runtime error";
    case DCN_E_INTERNAL: return "DCN_E_INTERNAL: internal error";
    case DCN_E_WORKSPACE: return "DCN_E_WORKSPACE: workspace missing or too small";
  }
  return "unknown dcn_status";
}

const char* dcn_last_error(void) { return g_last_error; }

dcn_status dcn_create(const dcn_desc* desc, dcn_plan* plan) {
  try {
    if (!plan) return fail(DCN_E_NULL, "dcn_create: plan output pointer is NULL");
    *plan = nullptr;
    if (!desc) return fail(DCN_E_NULL, "dcn_create: desc is NULL");
    const dcn_desc& d = *desc;
    if (d.in_dtype != DCN_F32 && d.in_dtype != DCN_BF16)
      return fail(DCN_E_DTYPE, "in_dtype %d is not DCN_F32 or DCN_BF16", d.in_dtype);
    if (d.out_dtype != DCN_F32 && d.out_dtype != DCN_BF16)
      return fail(DCN_E_DTYPE, "out_dtype %d is not a dcn_dtype", d.out_dtype);
    if (d.out_layout != DCN_OUT_NCHW && d.out_layout != DCN_OUT_NHWC)
      return fail(DCN_E_DTYPE, "out_layout %d is not a dcn_layout", d.out_layout);
    if (d.batch < 0 || d.in_ch < 1 || d.height < 1 || d.width < 1 || d.out_ch < 1 ||
        d.kernel_h < 1 || d.kernel_w < 1 || d.pad_h < 0 || d.pad_w < 0)
      return fail(DCN_E_SHAPE,
                  "sizes must satisfy B>=0, C,H,W,O,kh,kw>=1, pad>=0 (got B=%d C=%d H=%d W=%d "
                  "O=%d kh=%d kw=%d ph=%d pw=%d)",
                  d.batch, d.in_ch, d.height, d.width, d.out_ch, d.kernel_h, d.kernel_w,
                  d.pad_h, d.pad_w);
    const int64_t Ho = (int64_t)d.height + 2 * (int64_t)d.pad_h - d.kernel_h + 1;
    const int64_t Wo = (int64_t)d.width + 2 * (int64_t)d.pad_w - d.kernel_w + 1;
    if (Ho < 1 || Wo < 1)
      return fail(DCN_E_SHAPE, "output size %lld x %lld is empty (kernel larger than padded input)",
                  (long long)Ho, (long long)Wo);
    if (d.out_dtype != DCN_F32)
      return fail(DCN_E_UNSUPPORTED, "only fp32 output is built (out_dtype=%d)", d.out_dtype);
    const int64_t E = d.in_dtype == DCN_BF16 ? 2 : 4;
    const int vec = (int)(16 / E);
    if (d.in_ch % vec != 0)
      return fail(DCN_E_UNSUPPORTED,
                  "in_ch=%d must be a multiple of %d: channel vectors are fetched with 16-byte "
                  "loads",
                  d.in_ch, vec);
    const int64_t K = (int64_t)d.kernel_h * d.kernel_w;
    const int64_t HoWo = Ho * Wo;
    const int64_t x_bytes = (int64_t)d.batch * d.height * d.width * d.in_ch * E;
    if (x_bytes >= kLimit31 || (int64_t)d.height * d.width * d.in_ch * E >= kLimit31)
      return fail(DCN_E_UNSUPPORTED, "input is %lld bytes; this build addresses < 2^31",
                  (long long)x_bytes);
    if (K >= kLimit31 / 2 || HoWo >= kLimit31 ||
        (int64_t)d.batch * 2 * K * HoWo * E >= kLimit31 ||
        (int64_t)d.batch * d.out_ch * HoWo >= kLimit31)
      return fail(DCN_E_UNSUPPORTED, "offset/output element counts must stay below 2^31");

    dcn::KernelConfig kc = choose_config(d, (int)Ho, (int)Wo);
    if (!dcn::config_supported(kc))
      return fail(DCN_E_INTERNAL, "no kernel variant for CB=%d NO=%d", kc.CB, kc.NO);
    const int64_t wp = dcn::packed_weight_elems(kc, (int)K);
    if (wp * E >= kLimit31)
      return fail(DCN_E_UNSUPPORTED, "packed weight of %lld bytes is too large",
                  (long long)(wp * E));
    if ((int64_t)d.batch * kc.tiles_per_img * kc.n_otiles >= kLimit31)
      return fail(DCN_E_UNSUPPORTED, "too many tiles");

    dcn_plan p = new (std::nothrow) dcn_plan_s;
    if (!p) return fail(DCN_E_INTERNAL, "out of host memory");
    p->d = d;
    p->K = (int)K;
    p->Ho = (int)Ho;
    p->Wo = (int)Wo;
    p->kc = kc;
    p->wpack_bytes = (size_t)((wp * E + 255) / 256 * 256);
    choose_split(kc, (int)K, (int64_t)d.batch * kc.tiles_per_img * kc.n_otiles, p->nsplit,
                 p->kper, p->wsplit);
    const int64_t scratch =
        p->nsplit > 1 ? p->nsplit * split_stride(d.batch, d.out_ch, HoWo) * 4 : 0;
    p->ws_bytes = p->wpack_bytes + (size_t)scratch;
    p->x_bytes = (uint32_t)x_bytes;
    *plan = p;
    return ok();
  } catch (...) {
    return fail(DCN_E_INTERNAL, "dcn_create: unexpected exception");
  }
}

dcn_status dcn_destroy(dcn_plan plan) {
  delete plan;
  return ok();
}

dcn_status dcn_output_size(dcn_plan plan, int32_t* ho, int32_t* wo) {
  if (!plan) return fail(DCN_E_NULL, "dcn_output_size: plan is NULL");
  if (ho) *ho = plan->Ho;
  if (wo) *wo = plan->Wo;
  return ok();
}

dcn_status dcn_workspace_bytes(dcn_plan plan, size_t* bytes) {
  if (!plan || !bytes) return fail(DCN_E_NULL, "dcn_workspace_bytes: NULL argument");
  *bytes = plan->ws_bytes;
  return ok();
}

dcn_status dcn_packed_weight_bytes(dcn_plan plan, size_t* bytes) {
  if (!plan || !bytes) return fail(DCN_E_NULL, "dcn_packed_weight_bytes: NULL argument");
  *bytes = plan->wpack_bytes;
  return ok();
}

dcn_status dcn_pack_weight(dcn_plan plan, const void* weight, void* workspace,
                           size_t workspace_bytes, void* stream) {
  try {
    if (!plan) return fail(DCN_E_NULL, "dcn_pack_weight: plan is NULL");
    if (!weight) return fail(DCN_E_NULL, "dcn_pack_weight: weight is NULL");
    if (!workspace || workspace_bytes < plan->wpack_bytes)
      return fail(DCN_E_WORKSPACE, "packed weight needs %zu bytes, got %zu at %p",
                  plan->wpack_bytes, workspace_bytes, workspace);
    const size_t E = plan->kc.bf16 ? 2 : 4;
    if (!aligned(weight, E)) return fail(DCN_E_ALIGN, "weight is not %zu-byte aligned", E);
    if (!aligned(workspace, 16)) return fail(DCN_E_ALIGN, "workspace is not 16-byte aligned");
    const dcn_desc& d = plan->d;
    hipError_t e = dcn::launch_pack(plan->kc, weight, workspace, d.out_ch, d.in_ch, d.kernel_h,
                                    d.kernel_w, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "weight pack launch");
    return ok();
  } catch (...) {
    return fail(DCN_E_INTERNAL, "dcn_pack_weight: unexpected exception");
  }
}

namespace {

// Validated kernel arguments for output rows [row0, row0 + rows) from a
// packed weight.  The band is the plan's operator with the sampling grid
// shifted down by row0: the kernels form grid row = ho - pad_h + i, so a band
// launches with pad_h - row0 and rows output rows (the offsets, mask and
// output cover the band only).  *empty is set when there is nothing to read
// or write (empty batch or band).
dcn_status make_args(const char* who, dcn_plan plan, int32_t row0, int32_t rows, const void* x,
                     const void* offset, const void* mask, const void* packed_weight,
                     size_t workspace_bytes, const void* bias, void* out, dcn::FusedArgs& a,
                     dcn::KernelConfig& kc, bool& empty) {
  empty = false;
  if (!plan) return fail(DCN_E_NULL, "%s: plan is NULL", who);
  const dcn_desc& d = plan->d;
  if (row0 < 0 || rows < 0 || (int64_t)row0 + rows > plan->Ho)
    return fail(DCN_E_SHAPE, "%s: rows [%d, %d + %d) outside the output's %d rows", who, row0,
                row0, rows, plan->Ho);
  if (d.batch == 0 || rows == 0) {
    empty = true;
    return ok();
  }
  if (!x || !offset || !out) return fail(DCN_E_NULL, "%s: x, offset and out are required", who);
  if (!packed_weight || workspace_bytes < plan->wpack_bytes)
    return fail(DCN_E_WORKSPACE, "%s: packed weight needs %zu bytes, got %zu at %p", who,
                plan->wpack_bytes, workspace_bytes, packed_weight);
  const size_t E = plan->kc.bf16 ? 2 : 4;
  if (!aligned(x, 16) || !aligned(out, 16) || !aligned(packed_weight, 16))
    return fail(DCN_E_ALIGN, "%s: x, out and the packed weight must be 16-byte aligned", who);
  if (!aligned(offset, E) || (mask && !aligned(mask, E)) || (bias && !aligned(bias, E)))
    return fail(DCN_E_ALIGN, "%s: offset, mask and bias must be %zu-byte aligned", who, E);
  a = dcn::FusedArgs{};
  a.x = x;
  a.offset = offset;
  a.mask = mask;
  a.wpack = packed_weight;
  a.bias = bias;
  a.out = static_cast<float*>(out);
  a.B = d.batch;
  a.C = d.in_ch;
  a.H = d.height;
  a.W = d.width;
  a.O = d.out_ch;
  a.kh = d.kernel_h;
  a.kw = d.kernel_w;
  a.K = plan->K;
  a.ph = d.pad_h - row0;
  a.pw = d.pad_w;
  a.Ho = rows;
  a.Wo = plan->Wo;
  a.HoWo = rows * plan->Wo;
  kc = plan->kc;
  int tiles_x = 0;
  kc.tiles_per_img = kc.kind == 4 ? dcn::bf16win_tiles(rows, plan->Wo, tiles_x)
                                  : (int)ceil_div(a.HoWo, kc.M);
  a.tiles_x = tiles_x;
  a.nchunk = kc.nchunk;
  a.n_otiles = kc.n_otiles;
  a.tiles_per_img = kc.tiles_per_img;
  a.x_bytes = plan->x_bytes;
  a.offset_bytes = (uint32_t)((size_t)d.batch * 2 * plan->K * a.HoWo * E);
  a.mask_bytes = mask ? (uint32_t)((size_t)d.batch * plan->K * a.HoWo * E) : 0u;
  // NCHW: 4 consecutive pixels store as one 16-byte write when they start
  // 16-byte aligned (kind 4's 2-D tiles start rows at multiples of Wo)
  a.vec_store = kc.kind == 4 ? (plan->Wo % 4) == 0 : (a.HoWo % 4) == 0;
  a.nsplit = 1;
  a.kper = plan->K;
  a.split_stride = 0;
  a.wsplit = 1;
  return ok();
}

dcn_status forward_band(const char* who, dcn_plan plan, int32_t row0, int32_t rows,
                        const void* x, const void* offset, const void* mask, void* workspace,
                        size_t workspace_bytes, const void* bias, void* out, void* stream,
                        int32_t* dbg_corner = nullptr, float* dbg_weight = nullptr) {
  try {
    dcn::FusedArgs a;
    dcn::KernelConfig kc;
    bool empty;
    dcn_status st = make_args(who, plan, row0, rows, x, offset, mask, workspace,
                              workspace_bytes, bias, out, a, kc, empty);
    if (st != DCN_OK || empty) return st;
    a.dbg_corner = dbg_corner;
    a.dbg_weight = dbg_weight;
    a.wsplit = plan->wsplit;  // like the split: the whole map's choice, also for a band
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    // split tap sum when the plan's whole-map grid is small and the workspace
    // carries the scratch; a band splits like the whole map, so the bands of a
    // partition reproduce the whole-map output bit for bit
    const int nsplit = plan->nsplit, kper = plan->kper;
    const int64_t stride = split_stride(a.B, a.O, a.HoWo);
    const size_t scratch = workspace_bytes - plan->wpack_bytes;
    if (nsplit > 1 && (size_t)(nsplit * stride * 4) <= scratch && stride < kLimit31) {
      float* part = reinterpret_cast<float*>(static_cast<char*>(workspace) + plan->wpack_bytes);
      float* out_f = a.out;
      const float* bias_f = static_cast<const float*>(a.bias);
      a.out = part;
      a.bias = nullptr;
      a.nsplit = nsplit;
      a.kper = kper;
      a.split_stride = (uint32_t)stride;
      hipError_t e = dcn::launch_fused(kc, a, hs);
      if (e != hipSuccess) return hip_fail(e, "fused forward launch (tap split)");
      e = dcn::launch_split_reduce(part, nsplit, (uint32_t)stride, bias_f, out_f, a.B, a.O,
                                   a.HoWo, kc.nhwc, hs);
      if (e != hipSuccess) return hip_fail(e, "split reduce launch");
      return ok();
    }
    hipError_t e = dcn::launch_fused(kc, a, hs);
    if (e != hipSuccess) return hip_fail(e, "fused forward launch");
    return ok();
  } catch (...) {
    return fail(DCN_E_INTERNAL, "%s: unexpected exception", who);
  }
}

bool same_kernel(const dcn::KernelConfig& p, const dcn::KernelConfig& q) {
  return p.kind == q.kind && p.bf16 == q.bf16 && p.M == q.M && p.CB == q.CB && p.NO == q.NO &&
         p.nhwc == q.nhwc;
}

}  // namespace

dcn_status dcn_tap_schedule(dcn_plan plan, int32_t* runs, int32_t* taps_per_run,
                            int32_t* groups) {
  if (!plan) return fail(DCN_E_NULL, "dcn_tap_schedule: plan is NULL");
  if (runs) *runs = plan->nsplit;
  if (taps_per_run) *taps_per_run = plan->kper;
  if (groups) *groups = plan->wsplit;
  return ok();
}

dcn_status dcn_forward_packed(dcn_plan plan, const void* x, const void* offset, const void* mask,
                              void* workspace, size_t workspace_bytes, const void* bias,
                              void* out, void* stream) {
  return forward_band("dcn_forward_packed", plan, 0, plan ? plan->Ho : 0, x, offset, mask,
                      workspace, workspace_bytes, bias, out, stream);
}

dcn_status dcn_forward_rows(dcn_plan plan, int32_t row0, int32_t rows, const void* x,
                            const void* offset, const void* mask, void* workspace,
                            size_t workspace_bytes, const void* bias, void* out,
                            void* stream) {
  return forward_band("dcn_forward_rows", plan, row0, rows, x, offset, mask, workspace,
                      workspace_bytes, bias, out, stream);
}

dcn_status dcn_forward_multi(int32_t n, const dcn_plan* plans, const void* x,
                             const void* const* offsets, const void* const* masks,
                             const void* const* packed_weights, const size_t* workspace_bytes,
                             const void* const* biases, void* const* outs, void* stream) {
  try {
    if (n == 0) return ok();
    if (n < 0) return fail(DCN_E_SHAPE, "dcn_forward_multi: %d branches", n);
    if (n > dcn::kMaxBranches)
      return fail(DCN_E_UNSUPPORTED, "dcn_forward_multi: %d branches (1..%d supported)", n,
                  dcn::kMaxBranches);
    if (!plans || !offsets || !packed_weights || !workspace_bytes || !outs)
      return fail(DCN_E_NULL, "dcn_forward_multi: plans, offsets, packed_weights, "
                              "workspace_bytes and outs are required arrays");
    for (int i = 0; i < n; ++i) {
      if (!plans[i]) return fail(DCN_E_NULL, "dcn_forward_multi: plan %d is NULL", i);
      const dcn_desc& p = plans[i]->d;
      const dcn_desc& q = plans[0]->d;
      if (p.batch != q.batch || p.in_ch != q.in_ch || p.height != q.height ||
          p.width != q.width || p.in_dtype != q.in_dtype)
        return fail(DCN_E_SHAPE, "dcn_forward_multi: branch %d reads a different input than "
                                 "branch 0 (batch, channels, size and dtype must match)", i);
    }
    dcn::FusedArgs args[dcn::kMaxBranches];
    dcn::KernelConfig cfg[dcn::kMaxBranches];
    bool live[dcn::kMaxBranches];
    for (int i = 0; i < n; ++i) {
      bool empty;
      dcn_status st = make_args("dcn_forward_multi", plans[i], 0, plans[i]->Ho, x, offsets[i],
                                masks ? masks[i] : nullptr, packed_weights[i],
                                workspace_bytes[i], biases ? biases[i] : nullptr, outs[i],
                                args[i], cfg[i], empty);
      if (st != DCN_OK) return st;
      // tap groups as in the branch's own calls (never a split into runs), so
      // each branch reproduces its own forward_packed call bit for bit
      args[i].wsplit = plans[i]->wsplit;
      live[i] = !empty;
    }
    // one launch per group of branches that run the same kernel variant (and
    // tap-group count); the general kernel takes its branches one launch each
    bool done[dcn::kMaxBranches] = {};
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    for (int i = 0; i < n; ++i) {
      if (!live[i] || done[i]) continue;
      if (cfg[i].kind == 0) {
        hipError_t e = dcn::launch_fused(cfg[i], args[i], hs);
        if (e != hipSuccess) return hip_fail(e, "fused forward launch");
        done[i] = true;
        continue;
      }
      dcn::MultiArgs m{};
      int64_t total = 0;
      for (int j = i; j < n; ++j) {
        if (!live[j] || done[j] || !same_kernel(cfg[i], cfg[j]) ||
            args[j].wsplit != args[i].wsplit)
          continue;
        m.start[m.n] = (int)total;
        m.a[m.n] = args[j];
        ++m.n;
        total += (int64_t)args[j].B * cfg[j].tiles_per_img * cfg[j].n_otiles;
        done[j] = true;
      }
      if (total >= kLimit31)
        return fail(DCN_E_UNSUPPORTED, "dcn_forward_multi: %lld workgroups", (long long)total);
      m.start[m.n] = (int)total;
      hipError_t e = dcn::launch_fused_multi(cfg[i], m, hs);
      if (e != hipSuccess) return hip_fail(e, "multi-branch forward launch");
    }
    return ok();
  } catch (...) {
    return fail(DCN_E_INTERNAL, "dcn_forward_multi: unexpected exception");
  }
}

namespace {
// Backward workspace: the re-packed weight, then for bf16 plans fp32 copies
// of x, offset, mask and weight (each region 256-byte aligned).
struct BwdLayout {
  size_t wt, x, off, mask, w, total;
};
size_t round256(size_t n) { return (n + 255) / 256 * 256; }
BwdLayout bwd_layout(dcn_plan plan) {
  const dcn_desc& d = plan->d;
  BwdLayout L{};
  L.wt = 0;
  size_t at = round256((size_t)dcn::bwd_workspace_floats(d.out_ch, d.in_ch, plan->K) * 4);
  if (d.in_dtype == DCN_BF16) {
    const size_t HoWo = (size_t)plan->Ho * plan->Wo;
    L.x = at;
    at += round256((size_t)d.batch * d.height * d.width * d.in_ch * 4);
    L.off = at;
    at += round256((size_t)d.batch * 2 * plan->K * HoWo * 4);
    L.mask = at;
    at += round256((size_t)d.batch * plan->K * HoWo * 4);
    L.w = at;
    at += round256((size_t)d.out_ch * d.in_ch * plan->K * 4);
  }
  L.total = at;
  return L;
}
}  // namespace

dcn_status dcn_backward_workspace_bytes(dcn_plan plan, size_t* bytes) {
  if (!plan || !bytes) return fail(DCN_E_NULL, "dcn_backward_workspace_bytes: NULL argument");
  *bytes = bwd_layout(plan).total;
  return ok();
}

dcn_status dcn_backward(dcn_plan plan, const void* x, const void* offset, const void* mask,
                        const void* weight, const void* grad_out, void* grad_x,
                        void* grad_offset, void* grad_mask, void* grad_weight, void* grad_bias,
                        void* workspace, size_t workspace_bytes, void* stream) {
  try {
    if (!plan) return fail(DCN_E_NULL, "dcn_backward: plan is NULL");
    const dcn_desc& d = plan->d;
    const bool bf16 = d.in_dtype == DCN_BF16;
    if (bf16 && 2 * (int64_t)plan->x_bytes >= kLimit31)
      return fail(DCN_E_UNSUPPORTED, "dcn_backward: the fp32 copy of a bf16 x must stay below "
                                     "2^31 bytes");
    if (d.out_ch > 256)
      return fail(DCN_E_UNSUPPORTED, "dcn_backward: out_ch %d > 256", d.out_ch);
    size_t need = 0;
    dcn_backward_workspace_bytes(plan, &need);
    if (d.batch == 0) return ok();
    if (!x || !offset || !weight || !grad_out)
      return fail(DCN_E_NULL, "dcn_backward: x, offset, weight and grad_out are required");
    if (!workspace || workspace_bytes < need)
      return fail(DCN_E_WORKSPACE, "dcn_backward: workspace needs %zu bytes, got %zu at %p",
                  need, workspace_bytes, workspace);
    if (!aligned(x, 16) || !aligned(workspace, 16) || (grad_x && !aligned(grad_x, 16)))
      return fail(DCN_E_ALIGN, "dcn_backward: x, grad_x and the workspace must be 16-byte "
                               "aligned");
    const size_t E = bf16 ? 2 : 4;
    const void* ops[] = {offset, mask, weight};
    for (const void* q : ops)
      if (q && !aligned(q, E)) return fail(DCN_E_ALIGN, "dcn_backward: misaligned operand");
    const void* rest[] = {grad_out, grad_offset, grad_mask, grad_weight, grad_bias};
    for (const void* q : rest)
      if (q && !aligned(q, 4)) return fail(DCN_E_ALIGN, "dcn_backward: misaligned pointer");
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    if (bf16) {
      // bf16 operands: widen x, offset, mask and weight exactly into fp32
      // copies in the workspace; the backward then runs in fp32 throughout
      // (fp32 accumulators, fp32 gradients)
      const BwdLayout L = bwd_layout(plan);
      char* ws = static_cast<char*>(workspace);
      const int64_t HoWo = (int64_t)plan->Ho * plan->Wo;
      struct {
        const void* src;
        size_t at;
        int64_t n;
      } cv[] = {{x, L.x, (int64_t)d.batch * d.height * d.width * d.in_ch},
                {offset, L.off, (int64_t)d.batch * 2 * plan->K * HoWo},
                {mask, L.mask, mask ? (int64_t)d.batch * plan->K * HoWo : 0},
                {weight, L.w, (int64_t)d.out_ch * d.in_ch * plan->K}};
      for (auto& c : cv) {
        hipError_t e = dcn::launch_widen_bf16(c.src, reinterpret_cast<float*>(ws + c.at), c.n, hs);
        if (e != hipSuccess) return hip_fail(e, "bf16 widen launch");
      }
      x = ws + L.x;
      offset = ws + L.off;
      mask = mask ? ws + L.mask : nullptr;
      weight = ws + L.w;
    }
    dcn::BwdArgs a{};
    a.x = static_cast<const float*>(x);
    a.offset = static_cast<const float*>(offset);
    a.mask = static_cast<const float*>(mask);
    a.gout = static_cast<const float*>(grad_out);
    a.gx = static_cast<float*>(grad_x);
    a.goff = static_cast<float*>(grad_offset);
    a.gmask = static_cast<float*>(grad_mask);
    a.gw = static_cast<float*>(grad_weight);
    a.gb = static_cast<float*>(grad_bias);
    a.B = d.batch;
    a.C = d.in_ch;
    a.H = d.height;
    a.W = d.width;
    a.O = d.out_ch;
    a.kh = d.kernel_h;
    a.kw = d.kernel_w;
    a.K = plan->K;
    a.ph = d.pad_h;
    a.pw = d.pad_w;
    a.Ho = plan->Ho;
    a.Wo = plan->Wo;
    a.HoWo = plan->Ho * plan->Wo;
    a.nchunk = (int)ceil_div(d.in_ch, 64);
    a.tiles_per_img = (int)ceil_div(a.HoWo, 64);
    a.nhwc_g = d.out_layout == DCN_OUT_NHWC;
    a.x_bytes = bf16 ? 2 * plan->x_bytes : plan->x_bytes;
    hipError_t e = dcn::launch_backward(a, static_cast<const float*>(weight),
                                        static_cast<float*>(workspace), hs);
    if (e != hipSuccess) return hip_fail(e, "backward launch");
    return ok();
  } catch (...) {
    return fail(DCN_E_INTERNAL, "dcn_backward: unexpected exception");
  }
}

dcn_status dcn_msda_create(const dcn_msda_desc* desc, const int32_t* level_hw,
                           dcn_msda_plan* plan) {
  try {
    if (plan) *plan = nullptr;
    if (!desc || !level_hw || !plan) return fail(DCN_E_NULL, "dcn_msda_create: NULL argument");
    const dcn_msda_desc& d = *desc;
    if (d.batch < 0 || d.num_queries < 0 || d.num_heads <= 0 || d.head_dim <= 0 ||
        d.num_levels <= 0 || d.num_points <= 0)
      return fail(DCN_E_SHAPE, "dcn_msda_create: sizes must be positive (batch, queries >= 0)");
    if (d.dtype != DCN_F32 && d.dtype != DCN_BF16)
      return fail(DCN_E_DTYPE, "dcn_msda_create: dtype %d", d.dtype);
    const int vec = d.dtype == DCN_BF16 ? 8 : 4;
    if (d.num_levels > dcn::kMsdaMaxLevels || d.num_points > dcn::kMsdaMaxPoints)
      return fail(DCN_E_UNSUPPORTED, "dcn_msda_create: at most %d levels and %d points",
                  dcn::kMsdaMaxLevels, dcn::kMsdaMaxPoints);
    if (d.head_dim % vec != 0 || d.head_dim > 1024)
      return fail(DCN_E_UNSUPPORTED, "dcn_msda_create: head_dim %d must be a multiple of %d, "
                                     "at most 1024", d.head_dim, vec);
    std::unique_ptr<dcn_msda_plan_s> p(new dcn_msda_plan_s{});
    p->d = d;
    int64_t S = 0;
    for (int l = 0; l < d.num_levels; ++l) {
      const int32_t H = level_hw[2 * l], W = level_hw[2 * l + 1];
      if (H <= 0 || W <= 0) return fail(DCN_E_SHAPE, "dcn_msda_create: level %d is %dx%d", l, H, W);
      p->H[l] = H;
      p->W[l] = W;
      p->start[l] = (int)S;
      S += (int64_t)H * W;
      if (S >= kLimit31) return fail(DCN_E_UNSUPPORTED, "dcn_msda_create: too many positions");
    }
    p->S = (int)S;
    const int64_t vbytes =
        (int64_t)d.batch * S * d.num_heads * d.head_dim * (d.dtype == DCN_BF16 ? 2 : 4);
    const int64_t pairs = (int64_t)d.batch * d.num_queries * d.num_heads;
    if (vbytes >= kLimit31 || pairs * d.head_dim >= kLimit31 ||
        pairs * d.num_levels * d.num_points * 2 >= kLimit31)
      return fail(DCN_E_UNSUPPORTED, "dcn_msda_create: tensors must stay below 2^31 elements "
                                     "(value below 2^31 bytes)");
    *plan = p.release();
    return ok();
  } catch (...) {
    return fail(DCN_E_INTERNAL, "dcn_msda_create: unexpected exception");
  }
}

dcn_status dcn_msda_destroy(dcn_msda_plan plan) {
  delete plan;
  return ok();
}

dcn_status dcn_msda_value_positions(dcn_msda_plan plan, int32_t* positions) {
  if (!plan || !positions) return fail(DCN_E_NULL, "dcn_msda_value_positions: NULL argument");
  *positions = plan->S;
  return ok();
}

dcn_status dcn_msda_forward(dcn_msda_plan plan, const void* value, const void* locations,
                            const void* weights, void* out, void* stream) {
  try {
    if (!plan) return fail(DCN_E_NULL, "dcn_msda_forward: plan is NULL");
    const dcn_msda_desc& d = plan->d;
    const int64_t pairs = (int64_t)d.batch * d.num_queries * d.num_heads;
    if (pairs == 0) return ok();
    if (!value || !locations || !weights || !out)
      return fail(DCN_E_NULL, "dcn_msda_forward: value, locations, weights and out are required");
    const size_t E = d.dtype == DCN_BF16 ? 2 : 4;
    if (!aligned(value, 16) || !aligned(out, 16) || !aligned(locations, E) ||
        !aligned(weights, E))
      return fail(DCN_E_ALIGN, "dcn_msda_forward: value and out must be 16-byte aligned, "
                               "locations and weights %zu-byte", E);
    dcn::MsdaArgs a{};
    a.value = value;
    a.locations = locations;
    a.weights = weights;
    a.out = static_cast<float*>(out);
    a.npairs = pairs;
    a.B = d.batch;
    a.S = plan->S;
    a.G = d.num_heads;
    a.D = d.head_dim;
    a.Q = d.num_queries;
    a.L = d.num_levels;
    a.K = d.num_points;
    a.softmax = d.softmax ? 1 : 0;
    for (int l = 0; l < d.num_levels; ++l) {
      a.H[l] = plan->H[l];
      a.W[l] = plan->W[l];
      a.start[l] = plan->start[l];
    }
    a.value_bytes = (uint32_t)((int64_t)d.batch * plan->S * d.num_heads * d.head_dim * E);
    hipError_t e = dcn::launch_msda(a, d.dtype == DCN_BF16, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "msda launch");
    return ok();
  } catch (...) {
    return fail(DCN_E_INTERNAL, "dcn_msda_forward: unexpected exception");
  }
}

dcn_status dcn_dsample_create(const dcn_dsample_desc* desc, dcn_dsample_plan* plan) {
  try {
    if (plan) *plan = nullptr;
    if (!desc || !plan) return fail(DCN_E_NULL, "dcn_dsample_create: NULL argument");
    const dcn_dsample_desc& d = *desc;
    if (d.dtype != DCN_F32 && d.dtype != DCN_BF16)
      return fail(DCN_E_DTYPE, "dcn_dsample_create: dtype %d", d.dtype);
    if (d.out_layout != DCN_OUT_NCHW && d.out_layout != DCN_OUT_NHWC)
      return fail(DCN_E_DTYPE, "dcn_dsample_create: out_layout %d", d.out_layout);
    if (d.batch < 0 || d.groups < 1 || d.group_ch < 1 || d.height < 1 || d.width < 1 ||
        d.kernel_h < 1 || d.kernel_w < 1 || d.pad_h < 0 || d.pad_w < 0)
      return fail(DCN_E_SHAPE, "dcn_dsample_create: sizes must satisfy B>=0, G,D,H,W,kh,kw>=1, "
                               "pad>=0");
    const int64_t Ho = (int64_t)d.height + 2 * (int64_t)d.pad_h - d.kernel_h + 1;
    const int64_t Wo = (int64_t)d.width + 2 * (int64_t)d.pad_w - d.kernel_w + 1;
    if (Ho < 1 || Wo < 1) return fail(DCN_E_SHAPE, "dcn_dsample_create: empty output");
    const int64_t E = d.dtype == DCN_BF16 ? 2 : 4;
    if (d.group_ch % (16 / E) != 0)
      return fail(DCN_E_UNSUPPORTED, "dcn_dsample_create: group_ch %d must be a multiple of %d "
                                     "(16-byte channel vectors)", d.group_ch, (int)(16 / E));
    const int64_t C = (int64_t)d.groups * d.group_ch, K = (int64_t)d.kernel_h * d.kernel_w;
    const int64_t HoWo = Ho * Wo;
    const int64_t xb = (int64_t)d.batch * d.height * d.width * C * E;
    const int64_t ob = (int64_t)d.batch * d.groups * 2 * K * HoWo * E;
    if (xb >= kLimit31 || ob >= kLimit31 || (int64_t)d.batch * C * HoWo >= kLimit31 ||
        K >= kLimit31 / 2 || HoWo >= kLimit31)
      return fail(DCN_E_UNSUPPORTED, "dcn_dsample_create: tensors must stay below 2^31 bytes / "
                                     "elements");
    std::unique_ptr<dcn_dsample_plan_s> p(new dcn_dsample_plan_s{});
    p->d = d;
    p->K = (int)K;
    p->Ho = (int)Ho;
    p->Wo = (int)Wo;
    p->tiles_per_img = (int)ceil_div(HoWo, 64);
    const int ct = dcn::dsample_vectors_per_tile((int)C, d.dtype == DCN_BF16) * (int)(16 / E);
    p->n_ctiles = (int)ceil_div(C, ct);
    if ((int64_t)d.batch * p->tiles_per_img * p->n_ctiles >= kLimit31)
      return fail(DCN_E_UNSUPPORTED, "dcn_dsample_create: too many tiles");
    p->x_bytes = (uint32_t)xb;
    p->offset_bytes = (uint32_t)ob;
    p->weights_bytes = (uint32_t)(ob / 2);
    *plan = p.release();
    return ok();
  } catch (...) {
    return fail(DCN_E_INTERNAL, "dcn_dsample_create: unexpected exception");
  }
}

dcn_status dcn_dsample_destroy(dcn_dsample_plan plan) {
  delete plan;
  return ok();
}

dcn_status dcn_dsample_output_size(dcn_dsample_plan plan, int32_t* ho, int32_t* wo) {
  if (!plan) return fail(DCN_E_NULL, "dcn_dsample_output_size: plan is NULL");
  if (ho) *ho = plan->Ho;
  if (wo) *wo = plan->Wo;
  return ok();
}

dcn_status dcn_dsample_forward(dcn_dsample_plan plan, const void* x, const void* offset,
                               const void* weights, void* out, void* stream) {
  try {
    if (!plan) return fail(DCN_E_NULL, "dcn_dsample_forward: plan is NULL");
    const dcn_dsample_desc& d = plan->d;
    if (d.batch == 0) return ok();
    if (!x || !offset || !weights || !out)
      return fail(DCN_E_NULL, "dcn_dsample_forward: x, offset, weights and out are required");
    const size_t E = d.dtype == DCN_BF16 ? 2 : 4;
    if (!aligned(x, 16) || !aligned(out, 16) || !aligned(offset, E) || !aligned(weights, E))
      return fail(DCN_E_ALIGN, "dcn_dsample_forward: x and out must be 16-byte aligned, offset "
                               "and weights %zu-byte", E);
    dcn::DsArgs a{};
    a.x = x;
    a.offset = offset;
    a.weights = weights;
    a.out = static_cast<float*>(out);
    a.B = d.batch;
    a.G = d.groups;
    a.D = d.group_ch;
    a.H = d.height;
    a.W = d.width;
    a.kh = d.kernel_h;
    a.kw = d.kernel_w;
    a.K = plan->K;
    a.ph = d.pad_h;
    a.pw = d.pad_w;
    a.Ho = plan->Ho;
    a.Wo = plan->Wo;
    a.HoWo = plan->Ho * plan->Wo;
    a.softmax = d.softmax ? 1 : 0;
    a.tiles_per_img = plan->tiles_per_img;
    a.n_ctiles = plan->n_ctiles;
    a.x_bytes = plan->x_bytes;
    a.offset_bytes = plan->offset_bytes;
    a.weights_bytes = plan->weights_bytes;
    hipError_t e = dcn::launch_dsample(a, d.dtype == DCN_BF16, d.out_layout == DCN_OUT_NHWC,
                                       static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "dsample launch");
    return ok();
  } catch (...) {
    return fail(DCN_E_INTERNAL, "dcn_dsample_forward: unexpected exception");
  }
}

dcn_status dcn_nchw_to_nhwc(const void* src, void* dst, int32_t batch, int32_t channels,
                            int32_t height, int32_t width, int32_t dtype, void* stream) {
  try {
    if (dtype != DCN_F32 && dtype != DCN_BF16)
      return fail(DCN_E_DTYPE, "dcn_nchw_to_nhwc: dtype %d", dtype);
    if (batch < 0 || channels < 0 || height < 0 || width < 0)
      return fail(DCN_E_SHAPE, "dcn_nchw_to_nhwc: negative size");
    const int64_t n = (int64_t)batch * channels * height * width;
    if (n >= kLimit31) return fail(DCN_E_SHAPE, "dcn_nchw_to_nhwc: %lld elements", (long long)n);
    if (n == 0) return ok();
    if (!src || !dst) return fail(DCN_E_NULL, "dcn_nchw_to_nhwc: src and dst are required");
    if (!aligned(src, 16) || !aligned(dst, 16))
      return fail(DCN_E_ALIGN, "dcn_nchw_to_nhwc: src and dst must be 16-byte aligned");
    hipError_t e = dcn::launch_nchw_to_nhwc(dtype == DCN_BF16, src, dst, batch, channels,
                                            height * width, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "transpose launch");
    return ok();
  } catch (...) {
    return fail(DCN_E_INTERNAL, "dcn_nchw_to_nhwc: unexpected exception");
  }
}

dcn_status dcn_forward(dcn_plan plan, const void* x, const void* offset, const void* mask,
                       const void* weight, const void* bias, void* out, void* workspace,
                       size_t workspace_bytes, void* stream) {
  if (!plan) return fail(DCN_E_NULL, "dcn_forward: plan is NULL");
  if (plan->d.batch == 0) return ok();
  dcn_status s = dcn_pack_weight(plan, weight, workspace, workspace_bytes, stream);
  if (s != DCN_OK) return s;
  return dcn_forward_packed(plan, x, offset, mask, workspace, workspace_bytes, bias, out,
                            stream);
}

namespace {

// Workspace of dcn_forward_noalloc: one array per GPU, resident for the life
// of the process.  Host code never passes `scratch` itself to a kernel (on the
// host the name is a stand-in, not a device address): it asks the runtime for
// the array's address on the current device once and keeps that pointer.
static __device__ __align__(256) char scratch[DCN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (resolved on the first
// call made with that device current).
dcn_status scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "dcn_forward_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(DCN_E_UNSUPPORTED, "dcn_forward_noalloc: device %d (at most %d devices)", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol,
                      "dcn_forward_noalloc: hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return DCN_OK;
}

}  // namespace

dcn_status dcn_forward_noalloc(dcn_plan plan, const void* x, const void* offset, const void* mask,
                               const void* weight, const void* bias, void* out, void* stream) {
  try {
    if (!plan) return fail(DCN_E_NULL, "dcn_forward_noalloc: plan is NULL");
    if (plan->d.batch == 0) return ok();
    if (plan->wpack_bytes > DCN_NOALLOC_SCRATCH_BYTES)
      return fail(DCN_E_UNSUPPORTED,
                  "dcn_forward_noalloc: the packed weight needs %zu bytes, more than the %u "
                  "bytes of the library's static scratch; use dcn_forward with a workspace",
                  plan->wpack_bytes, (unsigned)DCN_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    dcn_status s = scratch_on_current_device(&ws);
    if (s != DCN_OK) return s;
    // the tap split's partial sums only when they fit beside the weight
    const size_t bytes = plan->ws_bytes <= DCN_NOALLOC_SCRATCH_BYTES ? plan->ws_bytes
                                                                     : plan->wpack_bytes;
    s = dcn_pack_weight(plan, weight, ws, bytes, stream);
    if (s != DCN_OK) return s;
    return dcn_forward_packed(plan, x, offset, mask, ws, bytes, bias, out, stream);
  } catch (...) {
    return fail(DCN_E_INTERNAL, "dcn_forward_noalloc: unexpected exception");
  }
}

dcn_status dcn_debug_corner_table(dcn_plan plan, const void* x, const void* offset,
                                  const void* mask, void* workspace, size_t workspace_bytes,
                                  const void* bias, void* out, int32_t* corner_index,
                                  float* corner_weight, void* stream) {
  if (!plan) return fail(DCN_E_NULL, "dcn_debug_corner_table: plan is NULL");
  if (plan->d.batch == 0) return ok();
  if (!corner_index || !corner_weight)
    return fail(DCN_E_NULL, "dcn_debug_corner_table: corner_index and corner_weight are required");
  if (!aligned(corner_index, 4) || !aligned(corner_weight, 4))
    return fail(DCN_E_ALIGN, "dcn_debug_corner_table: misaligned corner arrays");
  return forward_band("dcn_debug_corner_table", plan, 0, plan->Ho, x, offset, mask, workspace,
                      workspace_bytes, bias, out, stream, corner_index, corner_weight);
}

dcn_status dcn_debug_coords(dcn_plan plan, const void* offset, int32_t* y0x0, uint8_t* valid4,
                            void* stream) {
  try {
    if (!plan) return fail(DCN_E_NULL, "dcn_debug_coords: plan is NULL");
    const dcn_desc& d = plan->d;
    if (d.batch == 0) return ok();
    if (!offset || !y0x0 || !valid4)
      return fail(DCN_E_NULL, "dcn_debug_coords: offset, y0x0 and valid4 are required");
    const size_t E = plan->kc.bf16 ? 2 : 4;
    if (!aligned(offset, E) || !aligned(y0x0, 4))
      return fail(DCN_E_ALIGN, "dcn_debug_coords: misaligned pointer");
    hipError_t e = dcn::launch_coords(plan->kc.bf16, offset, y0x0, valid4, d.batch, plan->K,
                                      d.kernel_w, plan->Ho, plan->Wo, d.pad_h, d.pad_w,
                                      d.height, d.width, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "coords launch");
    return ok();
  } catch (...) {
    return fail(DCN_E_INTERNAL, "dcn_debug_coords: unexpected exception");
  }
}

}  // extern "C"
