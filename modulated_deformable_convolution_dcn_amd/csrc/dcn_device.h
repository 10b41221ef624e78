// dcn_device.h -- device-side building blocks of the gfx950 DCNv2 forward.
//
// The sampling-point stage lives here as one __device__ function used by both
// the fused kernel and the corner-export test hook, so the bit-exact corner
// test covers the code that runs on the timed path.
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

// Sampling point of one (pixel, tap) -- page 1 ("deform_conv.py",
// deform_conv2d_gather): the base grid row (ho - pad_h + i) is an exact
// integer, the point is that integer plus the learned offset in ONE fp32
// add, then floor and fraction in fp32.  Corner (a, b) = (y0 + a, x0 + b) is
// inside when 0 <= y0+a <= H-1 and 0 <= x0+b <= W-1, compared in float (a far
// point never goes through an integer conversion).
struct TapPoint {
  float y0, x0;   // floor of the sampling row / column
  float ly, lx;   // fractions in [0, 1)
  uint32_t valid; // bit (2a + b): corner (y0 + a, x0 + b) inside the image
};

__device__ __forceinline__ TapPoint tap_point(float dy, float dx, int grid_y, int grid_x, int H,
                                              int W) {
  TapPoint t;
  const float py = __fadd_rn(static_cast<float>(grid_y), dy);
  const float px = __fadd_rn(static_cast<float>(grid_x), dx);
  t.y0 = floorf(py);
  t.x0 = floorf(px);
  t.ly = __fsub_rn(py, t.y0);
  t.lx = __fsub_rn(px, t.x0);
  const float y1 = __fadd_rn(t.y0, 1.0f);
  const float x1 = __fadd_rn(t.x0, 1.0f);
  const float hmax = static_cast<float>(H - 1);
  const float wmax = static_cast<float>(W - 1);
  const bool vy0 = (t.y0 >= 0.0f) && (t.y0 <= hmax);
  const bool vy1 = (y1 >= 0.0f) && (y1 <= hmax);
  const bool vx0 = (t.x0 >= 0.0f) && (t.x0 <= wmax);
  const bool vx1 = (x1 >= 0.0f) && (x1 <= wmax);
  t.valid = (uint32_t)(vy0 && vx0) | ((uint32_t)(vy0 && vx1) << 1) |
            ((uint32_t)(vy1 && vx0) << 2) | ((uint32_t)(vy1 && vx1) << 3);
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
