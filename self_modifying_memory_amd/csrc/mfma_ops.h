// Matrix-core operand helpers shared by the MFMA chain kernels (gfx950, wave64).
//
// Layouts (16 x 16 tiles, lane l = 16 g + c, g = l >> 4, c = l & 15):
//   v_mfma_f32_16x16x16_bf16   A: lane holds A[c][4g + i], B: B[4g + i][c], i < 4
//   v_mfma_f32_16x16x32_bf16   A: lane holds A[c][k] and B: B[k][c] for the 8 k values
//                              {4g + i} and {16 + 4g + i} (this library's pairing of the 32:
//                              any pairing used on both sides gives the same contraction)
//   accumulator (both shapes)  lane holds C[4g + i][c]
// so a 16 x 16 result is already the B operand of a 16-deep product.
//
// fp32 operands are split as x = hi + lo with hi = bf16(x), lo = bf16(x - hi)
// (|x - hi - lo| <= 2^-17 |x|); a product of two split operands takes three bf16 products
// (hi*hi + hi*lo + lo*hi; lo*lo is below fp32 resolution).
#pragma once

#include <hip/hip_runtime.h>

namespace hope {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mma32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(short4v, a),
                                                   __builtin_bit_cast(short4v, b), c, 0, 0, 0);
}
// c += a b with a, b given as hi/lo pairs.  An accumulation chain never mixes the 16x16x32
// and 16x16x16 shapes: a 16x16x16 that takes a just-issued 16x16x32 result as its
// accumulator was seen to read the accumulator from before that product (no wait states
// are inserted between the two shapes).
__device__ __forceinline__ f32x4 mma32x3(bf16x8 ah, bf16x8 al, bf16x8 bh, bf16x8 bl, f32x4 c) {
  c = mma32(al, bh, c);
  c = mma32(ah, bl, c);
  return mma32(ah, bh, c);
}
__device__ __forceinline__ f32x4 mma16x3(bf16x4 ah, bf16x4 al, bf16x4 bh, bf16x4 bl, f32x4 c) {
  c = mma16(al, bh, c);
  c = mma16(ah, bl, c);
  return mma16(ah, bh, c);
}

// hi = bf16(x) (round to nearest even), lo = bf16(x - hi), for a pair of floats: one packed
// conversion for hi, its two halves widened back by a shift and a mask, two subtractions and
// one packed conversion for lo
__device__ __forceinline__ void split_pair(float x0, float x1, unsigned& hi, unsigned& lo) {
  typedef float f32x2v __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  const f32x2v x = {x0, x1};
  const unsigned h = __builtin_bit_cast(unsigned, __builtin_convertvector(x, bf16x2v));
  const f32x2v r = {x0 - __uint_as_float(h << 16), x1 - __uint_as_float(h & 0xffff0000u)};
  hi = h;
  lo = __builtin_bit_cast(unsigned, __builtin_convertvector(r, bf16x2v));
}
__device__ __forceinline__ void split8(const f32x4 v0, const f32x4 v1, bf16x8& hi, bf16x8& lo) {
  unsigned h0, h1, h2, h3, l0, l1, l2, l3;
  split_pair(v0[0], v0[1], h0, l0);
  split_pair(v0[2], v0[3], h1, l1);
  split_pair(v1[0], v1[1], h2, l2);
  split_pair(v1[2], v1[3], h3, l3);
  const u32x4 h = {h0, h1, h2, h3}, l = {l0, l1, l2, l3};
  hi = __builtin_bit_cast(bf16x8, h);
  lo = __builtin_bit_cast(bf16x8, l);
}
__device__ __forceinline__ void split4(const f32x4 v, bf16x4& hi, bf16x4& lo) {
  unsigned h0, h1, l0, l1;
  split_pair(v[0], v[1], h0, l0);
  split_pair(v[2], v[3], h1, l1);
  const u32x2 h = {h0, h1}, l = {l0, l1};
  hi = __builtin_bit_cast(bf16x4, h);
  lo = __builtin_bit_cast(bf16x4, l);
}

// The k slots of lane group g for 32-deep step s of a token-major bf16 row (8 values:
// columns 32 s + 4 g .. + 3 and 32 s + 16 + 4 g .. + 3, no conversion)
__device__ __forceinline__ bf16x8 load_row_pair_bf16(const unsigned short* row, int s, int g) {
  const u32x2 lo4 = *reinterpret_cast<const u32x2*>(row + 32 * s + 4 * g);
  const u32x2 hi4 = *reinterpret_cast<const u32x2*>(row + 32 * s + 16 + 4 * g);
  const u32x4 both = {lo4[0], lo4[1], hi4[0], hi4[1]};
  return __builtin_bit_cast(bf16x8, both);
}
// The k slots of lane group g for a 16-deep step: columns 16 s + 4 g .. + 3
__device__ __forceinline__ bf16x4 load_row_quad_bf16(const unsigned short* row, int s, int g) {
  return __builtin_bit_cast(bf16x4, *reinterpret_cast<const u32x2*>(row + 16 * s + 4 * g));
}

}  // namespace hope
