// dcn_device.h -- device-side building blocks of the gfx950 DCNv2 forward.
//
// The sampling-point stage lives here as one __device__ function used by both
// the fused kernel and the corner-export test hook, so the bit-exact corner
// test covers the code that runs on the timed path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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

}  // namespace dcn
