// The group quantizer shared by the packing kernel and the search kernels:
// group statistics across the lanes of a wave, the fp16 scale and zero point
// of a group, and the 4-bit codes of its weights.
//
// "AI-Research-SKILLs AWQ 高级使用指南", section 分组大小与零点量化: every group
// of g consecutive input channels of one output row shares one scale and one
// zero point.  The arithmetic is IEEE fp32 in one fixed order (each function
// turns off contraction into fused multiply-adds for its own body), with round-half-to-even and correctly rounded
// division, so every caller gets the same bits:
//   zero_point:  r = max(max - min, 1e-5); s = fp16(r / 15); z = clamp(rne(-min / s), 0, 15)
//   symmetric:   a = max(max|w|, 1e-5);    s = fp16(a / 7);  z = 8
//   q = clamp(rne(w / s) + z, 0, 15)
#pragma once

#include "awq_device.hpp"

namespace awq {
namespace {

constexpr float kRangeFloor = 1e-5f;

// Combine v over the GW consecutive lanes of a group (GW = 4, 8, 16 or 32,
// aligned); every lane gets the result.  Partners come by DPP lane swaps
// inside the 16-lane rows (xor 1 and xor 2 within quads, then mirrored
// halves of 8 lanes, then the mirrored halves of the row) and, for 32-lane
// groups, one permute across the two rows.  The min / max is taken on an
// order-preserving integer image of the (finite) floats: integer min / max
// needs no NaN canonicalization of the permuted operand, so each step is one
// DPP-fused instruction.  -0 orders below +0 there, which changes no scale,
// zero point or code.
__device__ __forceinline__ int ord_of(float x) {
  const int i = __builtin_bit_cast(int, x);
  return i ^ ((i >> 31) & 0x7FFFFFFF);
}
__device__ __forceinline__ float float_of(int o) { return __builtin_bit_cast(float, o ^ ((o >> 31) & 0x7FFFFFFF)); }

template <int CTRL>
__device__ __forceinline__ int dpp_mov(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false);
}

template <int GW, class Op>
__device__ __forceinline__ float group_all(float v, Op op) {
  int o = ord_of(v);
  if constexpr (GW >= 2) o = op(o, dpp_mov<0xB1>(o));   // quad_perm [1, 0, 3, 2]
  if constexpr (GW >= 4) o = op(o, dpp_mov<0x4E>(o));   // quad_perm [2, 3, 0, 1]
  if constexpr (GW >= 8) o = op(o, dpp_mov<0x141>(o));  // row_half_mirror
  if constexpr (GW >= 16) o = op(o, dpp_mov<0x140>(o)); // row_mirror
  if constexpr (GW >= 32) o = op(o, __shfl_xor(o, 16));
  return float_of(o);
}

struct MinOp {
  __device__ int operator()(int a, int b) const { return a < b ? a : b; }
};
struct MaxOp {
  __device__ int operator()(int a, int b) const { return a > b ? a : b; }
};

// Scale and zero point of a group from its lanes' own extremes: with a zero
// point, mn and mx are the smallest and largest of the lane's weights;
// without, mx is the lane's largest magnitude (mn unused).  A group of g
// channels is GW consecutive lanes of one row, reduced with butterfly
// shuffles (GW divides 32, so a group never leaves its half-wave, and all
// lanes of a group are active or inactive together).  s16 is the fp16 scale,
// s its fp32 value, zf the zero point as a float.
// ... from the group's own extremes (mn, mx: smallest and largest weight with
// a zero point; mx the largest magnitude without).
template <bool ZP>
__device__ __forceinline__ void scale_zero_of_extremes(float mn, float mx, _Float16& s16, float& s, float& zf) {
#pragma clang fp contract(off)
  if constexpr (ZP) {
    float rng = mx - mn;
    if (rng < kRangeFloor) rng = kRangeFloor;
    s16 = (_Float16)(rng / 15.0f);
    s = (float)s16;
    zf = rintf(-mn / s);
    zf = fminf(fmaxf(zf, 0.0f), 15.0f);
  } else {
    const float am = mx < kRangeFloor ? kRangeFloor : mx;
    s16 = (_Float16)(am / 7.0f);
    s = (float)s16;
    zf = 8.0f;
  }
}

template <int GW, bool ZP>
__device__ __forceinline__ void group_scale_zero_of(float mn, float mx, _Float16& s16, float& s, float& zf) {
  if constexpr (ZP) {
    mn = group_all<GW>(mn, MinOp());
    mx = group_all<GW>(mx, MaxOp());
  } else {
    mx = group_all<GW>(mx, MaxOp());
  }
  scale_zero_of_extremes<ZP>(mn, mx, s16, s, zf);
}

// The same from the lane's NV weights (one or two packed words).
template <int GW, bool ZP, int NV>
__device__ __forceinline__ void group_scale_zero(const float (&a)[NV], _Float16& s16, float& s, float& zf) {
  if constexpr (ZP) {
    float mn = a[0], mx = a[0];
#pragma unroll
    for (int c = 1; c < NV; ++c) {
      mn = fminf(mn, a[c]);
      mx = fmaxf(mx, a[c]);
    }
    group_scale_zero_of<GW, ZP>(mn, mx, s16, s, zf);
  } else {
    float m = fabsf(a[0]);
#pragma unroll
    for (int c = 1; c < NV; ++c) m = fmaxf(m, fabsf(a[c]));
    group_scale_zero_of<GW, ZP>(0.0f, m, s16, s, zf);
  }
}

// Transposed reduction over the GW consecutive lanes of a group: lane p of
// the group enters with v[0..GW) (one value per item, here per candidate) and
// leaves with v[0] = op over the group's lanes of item p.  At the step over
// lane bit b (b = GW/2, ..., 1) a lane keeps the half of its items selected
// by that bit and combines it with its partner's copy of the same half; the
// partners (lane ^ 1, ^ 2, ^ 7, ^ 15 by DPP swaps and mirrors) flip bit b and
// no higher bit, and together they span all GW lanes.  Values are the
// order-preserving integer images of ord_of.  A group's place p is lane % GW,
// so bit b of it is a fixed lane pattern; the selects take it as a constant
// lane mask (left to itself the compiler rewrites the chain of selects as a
// switch on p, eight compares and selects per value).
__device__ __forceinline__ int select_lanes(uint64_t mask, int if_set, int if_clear) {
  int r;
  asm("v_cndmask_b32 %0, %1, %2, %3" : "=v"(r) : "v"(if_clear), "v"(if_set), "s"(mask));
  return r;
}

template <int GW, class Op>
__device__ __forceinline__ void group_transpose(int (&v)[GW], Op op) {
#pragma unroll
  for (int b = GW / 2; b >= 1; b /= 2) {
    const uint64_t m = b == 1 ? 0xAAAAAAAAAAAAAAAAull
                     : b == 2 ? 0xCCCCCCCCCCCCCCCCull
                     : b == 4 ? 0xF0F0F0F0F0F0F0F0ull
                              : 0xFF00FF00FF00FF00ull;
#pragma unroll
    for (int i = 0; i < b; ++i) {
      const int send = select_lanes(m, v[i], v[i + b]);
      const int keep = select_lanes(m, v[i + b], v[i]);
      int recv;
      if (b == 1) recv = dpp_mov<0xB1>(send);        // quad_perm [1, 0, 3, 2]
      else if (b == 2) recv = dpp_mov<0x4E>(send);   // quad_perm [2, 3, 0, 1]
      else if (b == 4) recv = dpp_mov<0x141>(send);  // row_half_mirror
      else recv = dpp_mov<0x140>(send);              // row_mirror
      v[i] = op(keep, recv);
    }
  }
}

// fp16(fp32(a * b)): the fp32 product, rounded to fp16 (a weight scaled by a
// per-channel factor, as the quantizer sees it).  The empty asm keeps the
// product an fp32 value: left alone, the compiler fuses the multiply and the
// conversion into one mixed-precision instruction (v_fma_mixlo_f16) that
// rounds the exact product to fp16 once, which differs from rounding the fp32
// product wherever that lands on an fp16 midpoint (measured on gfx950).
__device__ __forceinline__ float fp32_product(float a, float b) {
  float p = a * b;
  asm("" : "+v"(p));
  return p;
}

// 768 + rne(a / s) for NE weights of one group, as floats, where a and s
// are fp16 values (a weight and its group's scale) and rs = rcp(s), computed
// without a division and without a branch: k = rint(fma(a, rs, 768)).
// The fused multiply-add rounds a * rs + 768 once, to fp32's grid of 2^-14 on
// [512, 1024), which snaps the quotient q = a / s to that grid: rcp's error
// leaves |a * rs - q| <= |q| 2^-23 < 2^-19 while |q| < 16, so an exact
// half-integer quotient j + 1/2 (a point of the grid) is recovered exactly
// and rint's ties-to-even then rounds it as rne(q) does (768 is even).  A
// quotient of two fp16 values that is not a half-integer lies at least about
// 2^-12 from one (with a = A 2^e, s = S 2^f and 11-bit A, S, the gap
// |2a - (2j + 1) s| / 2s is at least min(1 / 2S, |q| / A)), far more than
// the snapped value can move it (2^-15 + 2^-19), so rint rounds it to the
// same integer as q.  Beyond |q| = 16 every code saturates (the caller clamps
// k - 768 to [-z, 15 - z] with 0 <= z <= 15), and the sum stays on the right
// side of the clamp.  (Half-integer quotients are common: fp16 weights are
// coarse against a 16-level grid, about 1 in 250 weights.)
constexpr float kCodeBias = 768.0f;

template <int NE>
__device__ __forceinline__ void biased_quotients(const float (&a)[NE], float rs, float (&k)[NE]) {
#pragma clang fp contract(off)
#pragma unroll
  for (int c = 0; c < NE; ++c) k[c] = rintf(__builtin_fmaf(a[c], rs, kCodeBias));
}

// Codes of a lane's 8 weights of one group, clamp(rne(a / s) + z, 0, 15) as
// floats.
__device__ __forceinline__ void codes_of(const float (&a)[8], float s, float zf, float (&q)[8]) {
#pragma clang fp contract(off)
  float k[8];
  biased_quotients(a, __builtin_amdgcn_rcpf(s), k);
  const float shift = zf - kCodeBias;  // exact: small integers
#pragma unroll
  for (int c = 0; c < 8; ++c) q[c] = fminf(fmaxf(k[c] + shift, 0.0f), 15.0f);
}

// The packed word of 8 codes (small integers held as floats): two codes per
// byte, byte b holding the codes of channels 2b' and 2b' + 2 in the order of
// nibble_shift, each byte inserted by one float-to-u8 conversion.
__device__ __forceinline__ uint32_t pack_word(const float (&q)[8]) {
  uint32_t w = 0;
  // nibble_shift: c = 0, 2 -> byte 0; 4, 6 -> byte 1; 1, 3 -> byte 2; 5, 7 -> byte 3
  // (exact: small integers)
  w = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(q[2], 16.0f, q[0]), 0, w);
  w = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(q[6], 16.0f, q[4]), 1, w);
  w = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(q[3], 16.0f, q[1]), 2, w);
  w = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(q[7], 16.0f, q[5]), 3, w);
  return w;
}

// Range of the group a lane's 8 weights belong to, shrunk by `r` (weight
// clipping): [r * min, r * max] with a zero point, [-r * amax, r * amax]
// without (fp32 products).
template <int GW, bool ZP, int NV>
__device__ __forceinline__ void group_clip_bounds(const float (&a)[NV], float r, float& lo, float& hi) {
#pragma clang fp contract(off)
  if constexpr (ZP) {
    float mn = a[0], mx = a[0];
#pragma unroll
    for (int c = 1; c < NV; ++c) {
      mn = fminf(mn, a[c]);
      mx = fmaxf(mx, a[c]);
    }
    mn = group_all<GW>(mn, MinOp());
    mx = group_all<GW>(mx, MaxOp());
    lo = r * mn;
    hi = r * mx;
  } else {
    float amax = fabsf(a[0]);
#pragma unroll
    for (int c = 1; c < NV; ++c) amax = fmaxf(amax, fabsf(a[c]));
    amax = group_all<GW>(amax, MaxOp());
    hi = r * amax;
    lo = -hi;
  }
}

}  // namespace
}  // namespace awq
