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

// The decay g_t from what the g tensor holds: g_t itself, or its log
// (g_t = exp(lg_t), the fp32 exponential).
__device__ __forceinline__ float decay_of(float x, bool log_g) { return log_g ? expf(x) : x; }

// Whether step t of batch row b is an identity step (mask byte 0).
__device__ __forceinline__ bool skipped(const uint8_t* mask, int b, int T, int t) {
  return mask != nullptr && mask[(int64_t)b * T + t] == 0;
}

// A byte that reads as a valid step: the address a mask load uses when there
// is no mask (or the step is out of range), so that the load needs no branch.
__device__ const uint8_t kValidStep = 1;

// The mask byte of step t (1 without a mask or out of range), loaded without
// a branch around it.
__device__ __forceinline__ const uint8_t* mask_byte(const uint8_t* mask, int b, int T, int t,
                                                    bool in_range) {
  return mask != nullptr && in_range ? mask + (int64_t)b * T + t : &kValidStep;
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

// Four fp32 lanes of an MFMA 16x16x4 accumulator.
typedef float f4 __attribute__((ext_vector_type(4)));

// D = A B + C on one 16x16 tile with k = 4: lane l supplies A[l % 16][l / 16]
// and B[l / 16][l % 16]; C and D hold row 4 (l / 16) + v, column l % 16 in
// register v.
__device__ __forceinline__ f4 mfma(float a, float b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// D = A B + C on one 16x16 tile with k = 32, bf16 operands, fp32 accumulate:
// lane l supplies A[l % 16][8 (l / 16) + e] and B[8 (l / 16) + e][l % 16]
// for e = 0..7 (eight bf16 bit patterns, element e in bits 16e..16e+15 of
// the 128-bit operand); C and D as for mfma().  Products of two bf16 values
// are exact in fp32.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f4 mfma_bf16(uint4 a, uint4 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Two floats as packed bf16 (element 0 in the low half), each rounded to
// nearest even by one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// x = hi + mid + lo with three bf16 values, each rounded to nearest even
// from the remainder (the two remainders are exact in fp32).  The three
// 8-bit significands cover fp32's 24, so the sum reproduces x (away from the
// bottom of the exponent range), and products of the pieces with a bf16
// value are exact: three bf16 MFMAs give an fp32-accurate product.  Four
// values at once, as three 8-byte blocks of packed bf16.
// The residuals x - piece come from v_dot2_f32_bf16 against (-1, 0) or
// (0, -1): one instruction instead of unpacking the piece and subtracting.
// The residual is representable, so it is exact however the dot product
// rounds (the pieces match the subtracting form bit for bit wherever the
// leading piece does not overflow bf16).  The (-1, 0) pair is kept in a
// register: folded, it becomes the inline constant -1.0, which the
// instruction reads as the fp32 pattern, i.e. the pair (0, -1).
__device__ __forceinline__ float minus_bf16_lo(uint32_t pk, float x) {  // x - low half
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  uint32_t m = 0x0000bf80u;
  asm("" : "+v"(m));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, pk),
                                         __builtin_bit_cast(bf16x2v, m), x, false);
}
__device__ __forceinline__ float minus_bf16_hi(uint32_t pk, float x) {  // x - high half
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, pk),
                                         __builtin_bit_cast(bf16x2v, 0xbf800000u), x, false);
}
__device__ __forceinline__ void split3_quad(f4 v, uint2& hi, uint2& mid, uint2& lo) {
  hi = uint2{cvt_pk_bf16(v[0], v[1]), cvt_pk_bf16(v[2], v[3])};
  const f4 r = {minus_bf16_lo(hi.x, v[0]), minus_bf16_hi(hi.x, v[1]),
                minus_bf16_lo(hi.y, v[2]), minus_bf16_hi(hi.y, v[3])};
  mid = uint2{cvt_pk_bf16(r[0], r[1]), cvt_pk_bf16(r[2], r[3])};
  lo = uint2{cvt_pk_bf16(minus_bf16_lo(mid.x, r[0]), minus_bf16_hi(mid.x, r[1])),
             cvt_pk_bf16(minus_bf16_lo(mid.y, r[2]), minus_bf16_hi(mid.y, r[3]))};
}

// ds_read_b64_tr_b16: each lane names an 8-byte block of four bf16; inside
// every group of 16 lanes, lane i receives element i % 4 of the blocks named
// by lanes i / 4, 4 + i / 4, 8 + i / 4 and 12 + i / 4, in that order.  When
// lane s of group G names row k0 + 8 G + s / 4, columns n0 + 4 (s % 4) .. +3
// of a [k][n] tile, lane l receives rows k0 + 8 G + 0..3 of column
// n0 + l % 16: half of an MFMA 16x16x32 bf16 operand (rows 4..7 from a
// second read 4 rows further on).
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t* p) {
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p)));
}

// Swizzled bf16 tiles read through lds_read_tr16.  A tile is row-major
// [k][n] (k the MFMA reduction index), its row stride an odd multiple of 128
// bytes (rows of opposite parity in opposite halves of the 64 banks), and
// 4-element (8-byte) block c of row r stored at block c ^ tile_swz(r): the
// blocks one transposing read touches (rows k0 + 8 G + 0..3 and 4 blocks per
// row, G over a half-wave) then fall on distinct banks, and so do the
// 8-byte writes of 16 consecutive blocks of a row.  Rows hold at least 16
// blocks.
__device__ __forceinline__ int tile_swz(int r) {
  return (((r >> 1) & 1) << 2) | (((r >> 3) & 1) << 3);
}

// The operand of a 16x16x32 bf16 MFMA whose lane l holds rows k0 + 8 (l / 16)
// + 0..7 of column n0 + l % 16 of a swizzled tile with row stride RS (n0 a
// multiple of 16): the B operand of a [k][n] tile, or the A operand of a
// tile holding A^T.
template <int RS>
__device__ __forceinline__ uint4 tile_operand(const uint16_t* tile, int k0, int n0, int lr,
                                              int lq) {
  const int tl = k0 + 8 * lq + (lr >> 2), th = tl + 4;
  const int cb = (n0 >> 2) + (lr & 3);
  const uint2 lo = lds_read_tr16(tile + tl * RS + 4 * (cb ^ tile_swz(tl)));
  const uint2 hi = lds_read_tr16(tile + th * RS + 4 * (cb ^ tile_swz(th)));
  return uint4{lo.x, lo.y, hi.x, hi.y};
}

// 4x4 transpose across the four lanes of each DPP quad: lane b holds
// v[u] = M[u][b] before and M[b][u] after (two stages, each swapping the
// elements whose lane and index differ in one bit with the partner lane).
__device__ __forceinline__ f4 quad_transpose(f4 v, int lane) {
  const int b = lane & 3;
  f4 t;
  t[0] = dpp<kDppQuadSwap1>(v[1]);
  t[1] = dpp<kDppQuadSwap1>(v[0]);
  t[2] = dpp<kDppQuadSwap1>(v[3]);
  t[3] = dpp<kDppQuadSwap1>(v[2]);
#pragma unroll
  for (int u = 0; u < 4; ++u) v[u] = ((b ^ u) & 1) ? t[u] : v[u];
  t[0] = dpp<kDppQuadSwap2>(v[2]);
  t[1] = dpp<kDppQuadSwap2>(v[3]);
  t[2] = dpp<kDppQuadSwap2>(v[0]);
  t[3] = dpp<kDppQuadSwap2>(v[1]);
#pragma unroll
  for (int u = 0; u < 4; ++u) v[u] = ((b ^ u) & 2) ? t[u] : v[u];
  return v;
}

// DPP move with 1.0 in the lanes that get no source (the product identity).
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_or1(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, 1.f),
                                         __builtin_bit_cast(int, x), CTRL, ROWS,
                                         0xF, false));
}

// Inclusive product over lanes 0..l of a wave: a Hillis-Steele scan with
// row_shr inside each 16-lane row, then row_bcast:15 and row_bcast:31 across
// rows.  Only products of the inputs are formed (no division).
__device__ __forceinline__ float wave_prefix_product(float x) {
  x *= dpp_or1<0x111, 0xF>(x);  // row_shr:1
  x *= dpp_or1<0x112, 0xF>(x);  // row_shr:2
  x *= dpp_or1<0x114, 0xF>(x);  // row_shr:4
  x *= dpp_or1<0x118, 0xF>(x);  // row_shr:8
  x *= dpp_or1<0x142, 0xA>(x);  // row_bcast:15 into rows 1 and 3
  x *= dpp_or1<0x143, 0xC>(x);  // row_bcast:31 into rows 2 and 3
  return x;
}


// Four consecutive elements p[o .. o+3] held as the raw loaded bits, so that
// issuing the load does not wait for it: the validity mask depends on the
// indices only, and zeroing and bf16 widening happen in get(), where the
// block is consumed.  VEC: one vector load (o a multiple of 4, the four
// all valid or all invalid); else four element loads.
template <typename T, bool VEC>
struct Quad;

template <>
struct Quad<float, true> {
  float4 v;
  __device__ __forceinline__ void load(const float* __restrict__ p, int64_t o, bool ok, int) {
    v = *reinterpret_cast<const float4*>(p + (ok ? o : 0));
  }
  __device__ __forceinline__ static uint32_t mask(bool ok, int) { return ok ? 15u : 0u; }
  __device__ __forceinline__ f4 get(uint32_t m) const {
    return m ? f4{v.x, v.y, v.z, v.w} : f4{0.f, 0.f, 0.f, 0.f};
  }
};

template <>
struct Quad<bf16, true> {
  uint2 v;
  __device__ __forceinline__ void load(const bf16* __restrict__ p, int64_t o, bool ok, int) {
    v = *reinterpret_cast<const uint2*>(p + (ok ? o : 0));
  }
  __device__ __forceinline__ static uint32_t mask(bool ok, int) { return ok ? 15u : 0u; }
  __device__ __forceinline__ f4 get(uint32_t m) const {
    const f4 r = {__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
                  __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u)};
    return m ? r : f4{0.f, 0.f, 0.f, 0.f};
  }
};

template <typename T>
struct Quad<T, false> {
  T v[4];
  __device__ __forceinline__ void load(const T* __restrict__ p, int64_t o, bool ok, int lim) {
#pragma unroll
    for (int x = 0; x < 4; ++x) v[x] = p[(ok && x < lim) ? o + x : 0];
  }
  __device__ __forceinline__ static uint32_t mask(bool ok, int lim) {
    uint32_t m = 0;
#pragma unroll
    for (int x = 0; x < 4; ++x) m |= (uint32_t)(ok && x < lim) << x;
    return m;
  }
  __device__ __forceinline__ f4 get(uint32_t m) const {
    f4 r;
#pragma unroll
    for (int x = 0; x < 4; ++x) r[x] = ((m >> x) & 1) ? to_f32(v[x]) : 0.f;
    return r;
  }
};

}  // namespace gdr
