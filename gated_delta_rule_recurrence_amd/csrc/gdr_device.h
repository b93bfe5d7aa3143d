// Internal device helpers for the gfx950 gated delta rule kernels.
// Not part of the public ABI (that is include/gdr.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr {

// bfloat16 is carried as its 16-bit pattern.
struct bf16 {
  uint16_t bits;
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) {
  return __uint_as_float(static_cast<uint32_t>(x.bits) << 16);
}

template <typename T>
__device__ __forceinline__ T from_f32(float x);

template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }

// float -> bfloat16, round to nearest, ties to even; NaN stays a quiet NaN.
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t rounded = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  const uint32_t quiet = (u >> 16) | 0x0040u;
  const bool nan = (u & 0x7fffffffu) > 0x7f800000u;
  bf16 r;
  r.bits = static_cast<uint16_t>(nan ? quiet : rounded);
  return r;
}

template <typename T>
__device__ __forceinline__ float ld(const T* p, int64_t i) {
  return to_f32(p[i]);
}

template <typename T>
__device__ __forceinline__ void st(T* p, int64_t i, float x) {
  p[i] = from_f32<T>(x);
}

// One DPP lane permutation inside a row of 16 lanes (gfx9 DPP controls).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                         0xF, 0xF, true));
}

constexpr int kDppQuadSwap1 = 0xB1;   // quad_perm [1,0,3,2]: lane ^ 1
constexpr int kDppQuadSwap2 = 0x4E;   // quad_perm [2,3,0,1]: lane ^ 2
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7 - i within 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15 - i within 16

// Sum over the 16 lanes of a DPP row; every lane of the row receives the
// same bits (each stage adds two operands that are swapped between the two
// partner lanes, and IEEE addition is commutative).
// The last stage is written as one v_add_f32_dpp (the compiler keeps a
// separate v_mov_dpp for row_mirror); the s_nop covers the two wait states
// gfx9 requires between a VALU write and a DPP read of the same VGPR.
__device__ __forceinline__ float rowsum16(float x) {
  x += dpp<kDppQuadSwap1>(x);
  x += dpp<kDppQuadSwap2>(x);
  x += dpp<kDppHalfMirror>(x);
  float r;
  asm("s_nop 1\n\tv_add_f32_dpp %0, %1, %1 row_mirror row_mask:0xf bank_mask:0xf"
      : "=v"(r)
      : "v"(x));
  return r;
}

}  // namespace gdr
