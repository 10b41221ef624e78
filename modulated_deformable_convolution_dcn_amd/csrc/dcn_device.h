// dcn_device.h -- device-side building blocks of the gfx950 DCNv2 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "dcn_launch.h"

namespace dcn {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Byte offset that no buffer load may reach: the x buffer descriptor's size
// is kept below 2^31, and every in-kernel addition to this value stays below
// 2^32, so a load at it returns zero without touching memory.
constexpr uint32_t kNoCorner = 0x80000000u;

// The corner stage of every kernel: the sampling point of one (pixel, tap)
// and its four corners -- page 1 ("deform_conv.py", deform_conv2d_gather):
// the base grid coordinate (ho - pad_h + i, wo - pad_w + j) is an exact
// integer, the point is that integer plus the learned offset in ONE fp32 add,
// then floor and fraction in fp32; corner (a, b) = (y0 + a, x0 + b) counts
// only when 0 <= y0+a <= H-1 and 0 <= x0+b <= W-1 (page 1's `valid`).
// Every forward and backward kernel and the corner-export test hooks form
// their corner tables from these two functions, so the bit-exact corner test
// runs this code.
struct SamplePoint {
  float fy, fx;  // floor of the sampling row / column
  float ly, lx;  // fractions in [0, 1)
};

// gy, gx: the integer grid coordinate as a float (exact: |value| < 2^24).
__device__ __forceinline__ SamplePoint sample_point(float gy, float gx, float dy, float dx) {
  SamplePoint p;
  const float py = __fadd_rn(gy, dy);
  const float px = __fadd_rn(gx, dx);
  p.fy = floorf(py);
  p.fx = floorf(px);
  p.ly = __fsub_rn(py, p.fy);
  p.lx = __fsub_rn(px, p.fx);
  return p;
}

// Corner row a (0: row y0, 1: row y0 + 1) of a sampling point: the row, the
// first column x0 and whether corners (row, x0) and (row, x0 + 1) are inside.
// The floor is clamped to [-2, H] x [-2, W] before the integer conversion:
// that keeps every outside corner outside (a row or column of -2, -1, H or
// H + 1 is out of range) and every conversion exact, also for points far
// outside or infinite (a NaN point clamps to -2: outside).  Inside corners
// keep their exact floor.
struct CornerRow {
  int ry, ix;    // row y0 + a and column x0 (clamped as above)
  bool ok0, ok1; // (ry, ix) and (ry, ix + 1) inside the image
};

__device__ __forceinline__ CornerRow corner_row(const SamplePoint& p, int a, int H, int W) {
  CornerRow r;
  const int iy = (int)fminf(fmaxf(p.fy, -2.0f), (float)H);
  r.ix = (int)fminf(fmaxf(p.fx, -2.0f), (float)W);
  r.ry = iy + a;
  const bool rok = (uint32_t)r.ry < (uint32_t)H;
  r.ok0 = rok && (uint32_t)r.ix < (uint32_t)W;
  r.ok1 = rok && (uint32_t)(r.ix + 1) < (uint32_t)W;
  return r;
}

// Both corner rows at once: the point, its clamped top-left corner and the
// validity bit (2a + b) of corner (y0 + a, x0 + b).
struct TapCorners {
  SamplePoint p;
  int y0, x0;      // clamped floor (exact for any point with an inside corner)
  uint32_t valid;  // bit (2a + b): corner (y0 + a, x0 + b) inside the image
};

__device__ __forceinline__ TapCorners tap_corners(float gy, float gx, float dy, float dx, int H,
                                                  int W) {
  TapCorners t;
  t.p = sample_point(gy, gx, dy, dx);
  const CornerRow r0 = corner_row(t.p, 0, H, W);
  const CornerRow r1 = corner_row(t.p, 1, H, W);
  t.y0 = r0.ry;
  t.x0 = r0.ix;
  t.valid = (uint32_t)r0.ok0 | ((uint32_t)r0.ok1 << 1) | ((uint32_t)r1.ok0 << 2) |
            ((uint32_t)r1.ok1 << 3);
  return t;
}

// float -> int32 that saturates (the floor of a far point may exceed int32).
__device__ __forceinline__ int32_t sat_i32(float v) {
  if (v >= 2147483648.0f) return 2147483647;
  if (v < -2147483648.0f) return -2147483647 - 1;
  return static_cast<int32_t>(v);
}

template <class T>
__device__ __forceinline__ float to_f32(T v);
template <>
__device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <>
__device__ __forceinline__ float to_f32<__bf16>(__bf16 v) { return static_cast<float>(v); }

// Raw buffer descriptor over `base` with `bytes` valid bytes (dword 3 is the
// gfx9-family default format word).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}

// One operand element through a buffer descriptor, as fp32 (0 when the byte
// offset is past the descriptor's size).
template <class T>
__device__ __forceinline__ float load_scalar(__amdgpu_buffer_rsrc_t r, uint32_t byte_off);
template <>
__device__ __forceinline__ float load_scalar<float>(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0));
}
template <>
__device__ __forceinline__ float load_scalar<__bf16>(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  const uint32_t u = __builtin_amdgcn_raw_buffer_load_b16(r, byte_off, 0, 0);
  return __uint_as_float(u << 16);
}

// ---- shared by the fused kernels

// Calls f(std::integral_constant<int, i>) for i = 0 .. N-1, fully unrolled, so
// that the body can select registers and instructions at compile time.
template <class F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}


template <class T>
struct Ops;

template <>
struct Ops<float> {
  typedef f32x4 frag;
  static constexpr int VEC = 4;
  // blended = w0*c0 + w1*c1 + w2*c2 + w3*c3 on 4 fp32 channels
  __device__ static __forceinline__ u32x4 blend(f32x4 w, u32x4 c0, u32x4 c1, u32x4 c2,
                                                u32x4 c3) {
    const f32x4 v0 = __builtin_bit_cast(f32x4, c0), v1 = __builtin_bit_cast(f32x4, c1);
    const f32x4 v2 = __builtin_bit_cast(f32x4, c2), v3 = __builtin_bit_cast(f32x4, c3);
    f32x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float s = w[0] * v0[e];
      s = __builtin_fmaf(w[1], v1[e], s);
      s = __builtin_fmaf(w[2], v2[e], s);
      s = __builtin_fmaf(w[3], v3[e], s);
      r[e] = s;
    }
    return __builtin_bit_cast(u32x4, r);
  }
};

template <>
struct Ops<__bf16> {
  typedef bf16x8 frag;
  static constexpr int VEC = 8;
  __device__ static __forceinline__ float lo(uint32_t u) { return __uint_as_float(u << 16); }
  __device__ static __forceinline__ float hi(uint32_t u) {
    return __uint_as_float(u & 0xffff0000u);
  }
  // Blend 8 bf16 channels in fp32, round the result to bf16 (nearest-even).
  __device__ static __forceinline__ u32x4 blend(f32x4 w, u32x4 c0, u32x4 c1, u32x4 c2,
                                                u32x4 c3) {
    bf16x8 r;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float sl = w[0] * lo(c0[q]);
      sl = __builtin_fmaf(w[1], lo(c1[q]), sl);
      sl = __builtin_fmaf(w[2], lo(c2[q]), sl);
      sl = __builtin_fmaf(w[3], lo(c3[q]), sl);
      float sh = w[0] * hi(c0[q]);
      sh = __builtin_fmaf(w[1], hi(c1[q]), sh);
      sh = __builtin_fmaf(w[2], hi(c2[q]), sh);
      sh = __builtin_fmaf(w[3], hi(c3[q]), sh);
      r[2 * q] = static_cast<__bf16>(sl);
      r[2 * q + 1] = static_cast<__bf16>(sh);
    }
    return __builtin_bit_cast(u32x4, r);
  }
};

// One 16-byte fragment read from LDS.
template <class T>
__device__ __forceinline__ u32x4 lds16(const T* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// XCD-aware block order: the dispatcher deals consecutive workgroup ids to
// the 8 XCDs in turn, so logical tile t is given to hardware id
// (t % per_xcd) * 8 + t / per_xcd -- each XCD then walks one contiguous run
// of tiles and its private L2 holds one band of the input map.
__device__ __forceinline__ int xcd_logical_block(int bid, int nblk) {
  const int full = (nblk / 8) * 8;
  if (bid >= full) return bid;
  const int per_xcd = full / 8;
  return (bid % 8) * per_xcd + bid / 8;
}

// Kernel-argument source: a kernel runs either one problem (FusedArgs) or a
// table of branches (MultiArgs) in one launch.  Both give the workgroup's
// problem and its logical tile index within that problem; logical indices
// are XCD-remapped before the branch is found, so each XCD walks one
// contiguous run of tiles across the branches.
__device__ __forceinline__ const FusedArgs& resolve_args(const FusedArgs& a, int& logical) {
  logical = xcd_logical_block(blockIdx.x, gridDim.x);
  return a;
}
__device__ __forceinline__ const FusedArgs& resolve_args(const MultiArgs& m, int& logical) {
  const int g = xcd_logical_block(blockIdx.x, gridDim.x);
  int br = 0;
  for (int i = 1; i < m.n; ++i)
    if (g >= m.start[i]) br = i;
  logical = g - m.start[br];
  return m.a[br];
}

}  // namespace dcn
