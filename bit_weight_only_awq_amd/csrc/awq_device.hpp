// Device-side helpers shared by the gfx950 kernels of the W4A16 layer.
//
// Packed weight word (8 input channels of one output row): channel c of the
// word sits at bit 16*(c & 1) + 4*(c >> 1), so the low halfword holds the even
// channels 0,2,4,6 and the high halfword the odd channels 1,3,5,7.  That
// placement lets one AND pick the pair (2t, 2t+1) into the two halves of a
// 32-bit register, ready to be turned into a half2 without any shuffling.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace awq {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Bit offset of channel c (0..7) inside its packed word.
__host__ __device__ constexpr int nibble_shift(int c) { return 16 * (c & 1) + 4 * (c >> 1); }

__device__ __forceinline__ half2_t as_half2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }
__device__ __forceinline__ uint32_t as_u32(half2_t v) { return __builtin_bit_cast(uint32_t, v); }

// Subtrahends that turn the biased halves produced by decode_pairs into q - z.
struct ZeroBias {
  half2_t hi;  // (1024 + z, 1024 + z): pairs taken from nibble bits 0..3
  half2_t lo;  // (  64 + z,   64 + z): pairs taken from nibble bits 4..7
};

__device__ __forceinline__ ZeroBias zero_bias(uint32_t z) {
  ZeroBias b;
  b.hi = as_half2((0x6400u + z) * 0x00010001u);
  b.lo = as_half2((0x5400u + (z << 4)) * 0x00010001u);
  return b;
}

// v_and_or_b32 (a & m) | o with both constants in VGPRs: a VOP3 instruction on
// gfx9 cannot encode literal operands and reads at most one SGPR, so left to
// itself the compiler splits the pattern into v_and_b32 + v_or_b32.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t o) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "v"(o));
  return r;
}

// Masks and fp16 bias patterns of decode_pairs, kept in registers.
struct DecodeConsts {
  uint32_t mask_lo, mask_hi, bias_1024, bias_64;
  __device__ __forceinline__ DecodeConsts()
      : mask_lo(0x000F000Fu), mask_hi(0x00F000F0u), bias_1024(0x64006400u), bias_64(0x54005400u) {}
};

// Decode one packed word into four half2 values (q - z), pair t holding
// channels (2t, 2t+1).  Every step is exact:
//   * a nibble in bits 0..3 OR-ed under the fp16 pattern 0x6400 (1024.0) reads
//     as 1024 + q (the fp16 spacing at 1024 is 1);
//   * a nibble in bits 4..7 OR-ed under 0x5400 (64.0) reads as 64 + q (the
//     spacing at 64 is 1/16 and the nibble sits 4 bits up);
//   * subtracting 1024 + z or 64 + z leaves the small integer q - z, which
//     fp16 represents exactly.
__device__ __forceinline__ void decode_pairs(uint32_t w, const ZeroBias& b, const DecodeConsts& k, half2_t d[4]) {
  const uint32_t w8 = w >> 8;
  d[0] = as_half2(and_or(w, k.mask_lo, k.bias_1024)) - b.hi;
  d[1] = as_half2(and_or(w, k.mask_hi, k.bias_64)) - b.lo;
  d[2] = as_half2(and_or(w8, k.mask_lo, k.bias_1024)) - b.hi;
  d[3] = as_half2(and_or(w8, k.mask_hi, k.bias_64)) - b.lo;
}

// Decoded weights w' = (q - z) * s of one word as 8 halves in channel order,
// each rounded once to fp16 (the product q - z times s is formed exactly and
// rounded by the fp16 multiply).
__device__ __forceinline__ half8_t decode_word_scaled(uint32_t w, const ZeroBias& b, const DecodeConsts& k,
                                                      half2_t s2) {
  half2_t d[4];
  decode_pairs(w, b, k, d);
  half2_t p0 = d[0] * s2, p1 = d[1] * s2, p2 = d[2] * s2, p3 = d[3] * s2;
  half8_t r;
  r[0] = p0[0]; r[1] = p0[1];
  r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1];
  r[6] = p3[0]; r[7] = p3[1];
  return r;
}

__device__ __forceinline__ half8_t as_half8(u32x4 v) { return __builtin_bit_cast(half8_t, v); }

__device__ __forceinline__ half2_t splat2(_Float16 h) {
  half2_t r;
  r[0] = h;
  r[1] = h;
  return r;
}

// Index of the scale of row n, group j in the row-octet-major scale array
// [N/8][G][8], and of the zero-point word of that octet and group in [N/8][G].
__host__ __device__ __forceinline__ size_t scale_index(int n, int j, int G) {
  return ((size_t)(n >> 3) * G + j) * 8 + (n & 7);
}
__host__ __device__ __forceinline__ size_t zero_word_index(int n, int j, int G) { return (size_t)(n >> 3) * G + j; }

// Sum four per-lane row partials over the 64 lanes of a wave without LDS.
// v_permlane32_swap exchanges the upper half-wave of its first operand with
// the lower half-wave of its second, so adding its two results gives, in
// lanes 0-31, row a summed over lanes l and l + 32 and, in lanes 32-63, row b
// summed the same way.  v_permlane16_swap does the same between the odd
// 16-lane rows of its first operand and the even rows of its second.  After
// the two exchanges lane group r = lane / 16 carries partials of row r only;
// a DPP rotation by 8 adds the partial 8 lanes away (the same pair in either
// rotation direction), and a mirror within 8 lanes and two quad swaps finish
// the sum.  Returns row lane / 16's total in lanes with lane % 8 == 0 (the
// others hold it in another order of additions).  The order is fixed, and the
// eight-row version below adds every row in exactly the same order, so a row
// gets the same bits from either.
// (The two results are copied to named scalars before the bit casts: a bit
// cast applied directly to an element of the returned vector has been compiled
// as a cast of one and the same element for both.)
__device__ __forceinline__ float swap_sum32(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                                                  false, false);
  const uint32_t r0 = r[0], r1 = r[1];
  return __builtin_bit_cast(float, r0) + __builtin_bit_cast(float, r1);
}
__device__ __forceinline__ float swap_sum16(float a, float b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                                                  false, false);
  const uint32_t r0 = r[0], r1 = r[1];
  return __builtin_bit_cast(float, r0) + __builtin_bit_cast(float, r1);
}
template <int CTRL>
__device__ __forceinline__ float row_rotate(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
// the sum over each 8-lane half-row of a 16-lane row
__device__ __forceinline__ float octet_sum(float u) {
  u += row_rotate<0x141>(u);  // row_half_mirror
  u += row_rotate<0x4E>(u);   // quad_perm [2, 3, 0, 1]
  u += row_rotate<0xB1>(u);   // quad_perm [1, 0, 3, 2]
  return u;
}
__device__ __forceinline__ float wave_reduce_quad_rows(const float (&v)[4]) {
  const float a = swap_sum32(v[0], v[2]);  // lanes 0-31: row 0, lanes 32-63: row 2
  const float b = swap_sum32(v[1], v[3]);  // lanes 0-31: row 1, lanes 32-63: row 3
  const float s = swap_sum16(a, b);        // lanes 16 r .. 16 r + 15: row r
  return octet_sum(s + row_rotate<0x128>(s));  // row_ror:8
}

// The same for eight rows: the same two levels of lane-half swaps leave rows
// r and r + 4 in 16-lane group r; after the rotation by 8 a lane select puts
// row r in lanes 0-7 of the group and row r + 4 in lanes 8-15, and the same
// 8-lane sum completes both.  Returns the total of row
// (lane / 16) + 4 ((lane / 8) mod 2) in lanes with lane % 8 == 0.
__device__ __forceinline__ float wave_reduce_oct_rows(const float (&v)[8]) {
  const float a0 = swap_sum32(v[0], v[2]);  // lanes 0-31: row 0, 32-63: row 2
  const float a1 = swap_sum32(v[1], v[3]);
  const float a2 = swap_sum32(v[4], v[6]);  // lanes 0-31: row 4, 32-63: row 6
  const float a3 = swap_sum32(v[5], v[7]);
  const float s0 = swap_sum16(a0, a1);      // 16-lane group r: row r
  const float s1 = swap_sum16(a2, a3);      // 16-lane group r: row r + 4
  const float t0 = s0 + row_rotate<0x128>(s0);
  const float t1 = s1 + row_rotate<0x128>(s1);
  return octet_sum((__lane_id() & 8) ? t1 : t0);
}

// The hardware dispatches workgroup b of a 1-D grid to XCD (b mod 8).  This
// returns a tile index such that each XCD works on one contiguous range of
// tiles, so tiles that share operands also share that XCD's L2.
__device__ __forceinline__ int xcd_contiguous_tile(int b, int nblocks) {
  const int q = nblocks >> 3, r = nblocks & 7;
  const int x = b & 7, local = b >> 3;
  return x * q + (x < r ? x : r) + local;
}

}  // namespace awq
