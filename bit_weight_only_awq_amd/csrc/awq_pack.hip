// Group-wise 4-bit quantization and packing (awq_pack) and the fp16 decoder
// used to inspect packed weights (awq_dequant).
//
// The quantizer follows "AI-Research-SKILLs AWQ 高级使用指南", section
// 分组大小与零点量化: every group of g consecutive input channels of one
// output row shares one scale and one zero point; with zero_point the grid is
// shifted to cover an asymmetric range, without it the grid is symmetric.
// The codes are q = clamp(round(w/s) + z, 0, 15).  The arithmetic is IEEE
// fp32 in one fixed order, with round-half-to-even and correctly rounded
// division, so the output is bit-reproducible:
//   zero_point:  r = max(max - min, 1e-5); s = fp16(r / 15); z = clamp(rne(-min / s), 0, 15)
//   symmetric:   a = max(max|w|, 1e-5);    s = fp16(a / 7);  z = 8
//   q = clamp(rne(w / s) + z, 0, 15)
#include "awq_device.hpp"
#include "awq_launch.hpp"

#pragma clang fp contract(off)


namespace awq {
namespace {

constexpr int kPackThreads = 256;  // 8 rows x 32 lanes
constexpr int kPackWords = 2;      // packed words (8 channels each) per lane and pass of pack_kernel
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

// Scale and zero point of the group a lane's NV weights (one or two packed
// words) belong to.  A group of g channels is GW = g / NV consecutive lanes of
// one row, reduced with butterfly shuffles (GW divides 32, so a group never
// leaves its half-wave, and all lanes of a group are active or inactive
// together).  s16 is the fp16 scale,
// s its fp32 value, zf the zero point as a float.
// amax is the group's largest magnitude (a bound for every |a[c]|).
template <int GW, bool ZP, int NV>
__device__ __forceinline__ void group_scale_zero(const float (&a)[NV], _Float16& s16, float& s, float& zf,
                                                 float& amax) {
  if constexpr (ZP) {
    float mn = a[0], mx = a[0];
#pragma unroll
    for (int c = 1; c < NV; ++c) {
      mn = fminf(mn, a[c]);
      mx = fmaxf(mx, a[c]);
    }
    mn = group_all<GW>(mn, MinOp());
    mx = group_all<GW>(mx, MaxOp());
    amax = fmaxf(fabsf(mn), fabsf(mx));
    float rng = mx - mn;
    if (rng < kRangeFloor) rng = kRangeFloor;
    s16 = (_Float16)(rng / 15.0f);
    s = (float)s16;
    zf = rintf(-mn / s);
    zf = fminf(fmaxf(zf, 0.0f), 15.0f);
  } else {
    float m = fabsf(a[0]);
#pragma unroll
    for (int c = 1; c < NV; ++c) m = fmaxf(m, fabsf(a[c]));
    amax = group_all<GW>(m, MaxOp());
    const float am = amax < kRangeFloor ? kRangeFloor : amax;
    s16 = (_Float16)(am / 7.0f);
    s = (float)s16;
    zf = 8.0f;
  }
}

// Codes of a lane's 8 weights of one group, clamp(rne(a / s) + z, 0, 15) as
// floats, with a / s the correctly rounded fp32 quotient.  The quotient is
// first taken as x = a * rcp(s): the reciprocal is within 1 ulp and the
// product adds half an ulp, so x lies within |x| * 2^-21 of the correctly
// rounded quotient f, and rint(x) and rne(f) can differ only if a
// half-integer lies within that distance of x.  With m = amax * rcp(s) *
// 2^-20, at least twice that distance for every weight of the group, a lane
// keeps rint(x) when all its 8 products lie more than m from a half-integer
// (|x - rint(x)| < 0.5 - m; about 2^-15 of the weights of a Gaussian group
// fail it), and divides all 8 weights exactly otherwise (every weight of a
// group on an exact half-step grid, every group whose quotients pass 2^19).
// Bit-identical to dividing every weight.
__device__ __forceinline__ void codes_of(const float (&a)[8], float s, float zf, float amax, float (&q)[8]) {
  const float rs = __builtin_amdgcn_rcpf(s);
  const float lim = 0.5f - amax * rs * 0x1p-20f;
  float k[8];
  float dmax = 0.0f;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const float x = a[c] * rs;
    k[c] = rintf(x);
    dmax = fmaxf(dmax, fabsf(x - k[c]));
  }
  if (!(dmax < lim)) {
#pragma unroll
    for (int c = 0; c < 8; ++c) k[c] = rintf(a[c] / s);
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) q[c] = fminf(fmaxf(k[c] + zf, 0.0f), 15.0f);
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

// One block quantizes one octet of rows (n0 .. n0+7) over one slice of K
// (blockIdx.y: packed words [chunk_words * y, + chunk_words), a multiple of a
// 512-channel pass, so slices end on group boundaries; several slices per row
// keep enough blocks in flight when the rows are few).  Thread t works on row
// n0 + (t >> 5); its lane l = t & 31 owns two consecutive packed words (16
// channels, always in one group) of each 512-channel pass over the slice, so
// wave w holds rows 2w (lanes 0..31) and 2w + 1 (lanes 32..63) and a group
// of g channels is GW = g / 16 consecutive lanes: the group statistics and
// the scale and zero point, computed alike by every lane of a group, are
// shared by 16 weights per lane (with one word per lane, 9-12% slower with
// zero points: the group reductions and the two divisions of the scale and
// zero point are per wave instruction, whatever a lane holds).  The first lane of each group stores its
// row's fp16 scale into the octet's 16-byte scale vector, and the rows 2w and
// 2w + 1 share one byte of the octet's zero-point word (two nibbles), written
// by the row-2w lane after one exchange: no LDS, no barriers.
template <int GW, bool ZP>
__global__ __launch_bounds__(kPackThreads) void pack_kernel(const u32x4* __restrict__ w, int N, int K,
                                                            int chunk_words, uint32_t* __restrict__ qweight,
                                                            uint16_t* __restrict__ scales,
                                                            uint32_t* __restrict__ qzeros) {
  constexpr int WPL = kPackWords;
  typedef uint32_t wordsT __attribute__((ext_vector_type(WPL)));
  constexpr int kPass = 32 * WPL;   // words per row and pass
  const int t = threadIdx.x;
  const int r = t >> 5, l = t & 31;
  const int n = blockIdx.x * 8 + r;
  const int kw = K >> 3;            // packed words per row
  const int G = kw / (WPL * GW);    // groups per row
  uint16_t* soct = scales + (size_t)blockIdx.x * G * 8;
  uint8_t* zoct = reinterpret_cast<uint8_t*>(qzeros + (ZP ? (size_t)blockIdx.x * G : 0));

  const int j_begin = blockIdx.y * chunk_words;
  const int j_end = min(kw, j_begin + chunk_words);  // multiples of WPL: no lane's words straddle j_end

  // the next pass's weights are loaded while this one is quantized (deeper
  // rings, 2-4 passes ahead, were 1-4% slower: the grid alone keeps enough
  // loads in flight)
  constexpr int kDepth = 1;
  const u32x4* wrow = w + (size_t)n * kw;
  u32x4 ring[kDepth][WPL];
#pragma unroll
  for (int u = 0; u < kDepth; ++u) {
    const int j = j_begin + kPass * u + WPL * l;
#pragma unroll
    for (int i = 0; i < WPL; ++i) ring[u][i] = j < j_end ? wrow[j + i] : u32x4{0u, 0u, 0u, 0u};
  }
  for (int w0 = j_begin; w0 < j_end; w0 += kPass * kDepth) {
#pragma unroll
    for (int u = 0; u < kDepth; ++u) {
      if (w0 + kPass * u >= j_end) break;  // uniform: no pass left
      const int j = w0 + kPass * u + WPL * l;
      const bool active = j < j_end;
      u32x4 raw[WPL];
      const int jn = j + kPass * kDepth;
#pragma unroll
      for (int i = 0; i < WPL; ++i) {
        raw[i] = ring[u][i];
        ring[u][i] = jn < j_end ? wrow[jn + i] : u32x4{0u, 0u, 0u, 0u};
      }

      float a[8 * WPL], aw[WPL][8];
#pragma unroll
      for (int i = 0; i < WPL; ++i) {
        const half8_t h = as_half8(raw[i]);
#pragma unroll
        for (int c = 0; c < 8; ++c) aw[i][c] = a[8 * i + c] = (float)h[c];
      }

      float s, zf, amax;
      _Float16 s16;
      group_scale_zero<GW, ZP>(a, s16, s, zf, amax);

      wordsT out;
#pragma unroll
      for (int i = 0; i < WPL; ++i) {
        float q[8];
        codes_of(aw[i], s, zf, amax, q);
        out[i] = pack_word(q);
      }
      if (active) *reinterpret_cast<wordsT*>(qweight + (size_t)n * kw + j) = out;

      const int grp = j / (WPL * GW);
      const bool leader = active && (l % GW) == 0;
      if (leader) soct[(size_t)grp * 8 + r] = __builtin_bit_cast(uint16_t, s16);
      if constexpr (ZP) {
        const float zpartner = __shfl_xor(zf, 32);  // row 2w + 1's zero point, same group
        if (leader && (r & 1) == 0)
          zoct[(size_t)grp * 4 + (r >> 1)] = (uint8_t)((uint32_t)zf | ((uint32_t)zpartner << 4));
      }
    }
  }
}

// Weight error of the activation-aware scaling, for the objective
//   L(s) = || Q(W diag(s)) (diag(s)^-1 X) - W X ||
// ("AI-Research-SKILLs AWQ 高级使用指南", section 算法原理).  For candidate c
// (blockIdx.y) with per-input-channel scales s_c:
//   e[n][k] = fp16( w'[n][k] / s_c[k] - w[n][k] ),  w' = Dq(Q(fp16(w[n][k] * s_c[k])))
// so that L(s_c) = || X e^T ||_F: one dense product instead of two.  The
// quantizer is the one of pack_kernel (same code, same fp32 order); w * s is
// an fp32 product rounded to fp16, w' = (q - z) * s is exact, and the
// product by the reciprocal of s_c[k] (1 ulp) and the subtraction are fp32
// roundings far below the final fp16 one.  Same block shape as pack_kernel:
// one octet of rows per block.
template <int GW, bool ZP>
__global__ __launch_bounds__(kPackThreads) void scale_error_kernel(const u32x4* __restrict__ w,
                                                                   const float* __restrict__ s_all, int N, int K,
                                                                   u32x4* __restrict__ e_all) {
  constexpr int WPL = kPackWords;  // lane l of a row owns words 2l, 2l + 1 of each 64-word pass
  const int t = threadIdx.x;
  const int r = t >> 5, l = t & 31;
  const int n = blockIdx.x * 8 + r;
  const int kw = K >> 3;
  const float* sc = s_all + (size_t)blockIdx.y * K;
  u32x4* e = e_all + (size_t)blockIdx.y * N * kw;

  // the next pass's weights and scales are loaded while this pass is processed
  const u32x4* wrow = w + (size_t)n * kw;
  u32x4 nraw[WPL];
  float4_t ns[2 * WPL];
  auto fetch = [&](int j) {
#pragma unroll
    for (int i = 0; i < WPL; ++i) nraw[i] = j < kw ? wrow[j + i] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 2 * WPL; ++i)
      ns[i] = j < kw ? *reinterpret_cast<const float4_t*>(sc + 8 * j + 4 * i) : float4_t{1.f, 1.f, 1.f, 1.f};
  };
  fetch(WPL * l);
  for (int w0 = 0; w0 < kw; w0 += 32 * WPL) {
    const int j = w0 + WPL * l;  // kw is a multiple of 4: a lane's words are all in or all out
    const bool active = j < kw;
    u32x4 raw[WPL];
    float sv[8 * WPL];
#pragma unroll
    for (int i = 0; i < WPL; ++i) raw[i] = nraw[i];
#pragma unroll
    for (int i = 0; i < 2 * WPL; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c) sv[4 * i + c] = ns[i][c];
    fetch(j + 32 * WPL);
    float hv[8 * WPL], a[8 * WPL];
#pragma unroll
    for (int i = 0; i < WPL; ++i) {
      const half8_t h = as_half8(raw[i]);
#pragma unroll
      for (int c = 0; c < 8; ++c) hv[8 * i + c] = (float)h[c];
    }
#pragma unroll
    for (int c = 0; c < 8 * WPL; ++c) a[c] = (float)(_Float16)(hv[c] * sv[c]);

    float s, zf, amax;
    _Float16 s16;
    group_scale_zero<GW, ZP>(a, s16, s, zf, amax);

    // e only needs fp16 accuracy: w' / s by a reciprocal (1 ulp in fp32)
#pragma unroll
    for (int i = 0; i < WPL; ++i) {
      float ai[8], q[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) ai[c] = a[8 * i + c];
      codes_of(ai, s, zf, amax, q);
      half8_t out;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float wq = (q[c] - zf) * s;
        out[c] = (_Float16)(wq * __builtin_amdgcn_rcpf(sv[8 * i + c]) - hv[8 * i + c]);
      }
      if (active) e[(size_t)n * kw + j + i] = __builtin_bit_cast(u32x4, out);
    }
  }
}

// Output error of weight clipping, for the search of apply_clip ("AI-Research-
// SKILLs AWQ 高级使用指南", section 自定义校准策略 (校准参数全景): clip the weights to reduce
// the effect of outliers on the quantization error).  For candidate ratio
// r_c (blockIdx.y): every group is clamped to its range shrunk by r_c (fp32,
// then fp16), quantized as by pack_kernel, decoded, and compared with the
// unclipped weight:  e[c][n][k] = fp16(Dq(Q(clip_c(w)))[n][k] - w[n][k]).
template <int GW, bool ZP>
__global__ __launch_bounds__(kPackThreads) void clip_error_kernel(const u32x4* __restrict__ w, ClipRatios ratios,
                                                                  int N, int K, u32x4* __restrict__ e_all) {
  constexpr int WPL = kPackWords;  // lane l of a row owns words 2l, 2l + 1 of each 64-word pass
  const int t = threadIdx.x;
  const int r = t >> 5, l = t & 31;
  const int n = blockIdx.x * 8 + r;
  const int kw = K >> 3;
  const float ratio = ratios.v[blockIdx.y];
  u32x4* e = e_all + (size_t)blockIdx.y * N * kw;
  const u32x4* wrow = w + (size_t)n * kw;
  u32x4 next[WPL];
#pragma unroll
  for (int i = 0; i < WPL; ++i) next[i] = WPL * l < kw ? wrow[WPL * l + i] : u32x4{0u, 0u, 0u, 0u};
  for (int w0 = 0; w0 < kw; w0 += 32 * WPL) {
    const int j = w0 + WPL * l;  // kw is a multiple of 4: a lane's words are all in or all out
    const bool active = j < kw;
    const int jn = j + 32 * WPL;
    float a[8 * WPL];
#pragma unroll
    for (int i = 0; i < WPL; ++i) {
      const half8_t h = as_half8(next[i]);
#pragma unroll
      for (int c = 0; c < 8; ++c) a[8 * i + c] = (float)h[c];
      next[i] = jn < kw ? wrow[jn + i] : u32x4{0u, 0u, 0u, 0u};
    }
    float lo, hi;
    group_clip_bounds<GW, ZP>(a, ratio, lo, hi);
    float cl[8 * WPL];
#pragma unroll
    for (int c = 0; c < 8 * WPL; ++c) cl[c] = (float)(_Float16)fminf(fmaxf(a[c], lo), hi);
    float s, zf, amax;
    _Float16 s16;
    group_scale_zero<GW, ZP>(cl, s16, s, zf, amax);
#pragma unroll
    for (int i = 0; i < WPL; ++i) {
      float ci[8], q[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) ci[c] = cl[8 * i + c];
      codes_of(ci, s, zf, amax, q);
      half8_t out;
#pragma unroll
      for (int c = 0; c < 8; ++c) out[c] = (_Float16)((q[c] - zf) * s - a[8 * i + c]);
      if (active) e[(size_t)n * kw + j + i] = __builtin_bit_cast(u32x4, out);
    }
  }
}

// The clipping ratio of each weight group (n, j): the error of the group under
// ratio c is the sum, in a fixed order (fp64), of the per-tile partials
// part[c][tm][h][j][n] (tile rows tm, half h of a tile's rows), and the group
// keeps the first ratio with the smallest error.  One thread per group,
// consecutive threads on consecutive rows n, so the partial reads coalesce.
__global__ __launch_bounds__(256) void clip_choose_kernel(const float* __restrict__ part, int parts, int G, int N,
                                                          int count, int32_t* __restrict__ choice) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)G * N) return;
  const int grp = (int)(idx / N), n = (int)(idx - (size_t)grp * N);
  double best_v = __builtin_huge_val();
  int best = 0;
  for (int c = 0; c < count; ++c) {
    double v = 0.0;
    for (int p = 0; p < parts; ++p) v += (double)part[(((size_t)c * parts + p) * G + grp) * N + n];
    if (v < best_v) {
      best_v = v;
      best = c;
    }
  }
  choice[(size_t)n * G + grp] = best;
}

// Writes the clipped weights: every group clamped to its range shrunk by its
// chosen ratio choice[n][j].
template <int GW, bool ZP>
__global__ __launch_bounds__(kPackThreads) void clip_apply_kernel(const u32x4* __restrict__ w, int N, int K,
                                                                  ClipRatios ratios,
                                                                  const int32_t* __restrict__ choice,
                                                                  u32x4* __restrict__ w_out) {
  const int t = threadIdx.x;
  const int r = t >> 5, l = t & 31;
  const int n = blockIdx.x * 8 + r;
  const int kw = K >> 3;
  const int G = kw / GW;
  for (int w0 = 0; w0 < kw; w0 += 32) {
    const int j = w0 + l;
    const bool active = j < kw;
    const int grp = j / GW;
    const int best = active ? choice[(size_t)n * G + grp] : 0;
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (active) raw = w[(size_t)n * kw + j];
    const half8_t h = as_half8(raw);
    float a[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) a[c] = (float)h[c];
    float lo, hi;
    group_clip_bounds<GW, ZP>(a, ratios.v[best], lo, hi);
    half8_t out;
#pragma unroll
    for (int c = 0; c < 8; ++c) out[c] = (_Float16)fminf(fmaxf(a[c], lo), hi);
    if (active) w_out[(size_t)n * kw + j] = __builtin_bit_cast(u32x4, out);
  }
}

// One thread per packed word: w_out[n][8j .. 8j+7] = fp16((q - z) * s).
// (q - z) * s is exact in fp32 (a 5-bit by 11-bit product), so the single
// conversion to fp16 is the only rounding.
__global__ __launch_bounds__(256) void dequant_kernel(const uint32_t* __restrict__ qweight,
                                                      const uint16_t* __restrict__ scales,
                                                      const uint32_t* __restrict__ qzeros,
                                                      u32x4* __restrict__ w_out, int N, int K, int gshift,
                                                      int zero_point) {
  const int kw = K >> 3;
  const size_t total = (size_t)N * kw;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    const int n = (int)(idx / kw), j = (int)(idx % kw);
    const int G = K >> gshift;
    const int grp = (j << 3) >> gshift;
    const float s = (float)__builtin_bit_cast(_Float16, scales[scale_index(n, grp, G)]);
    int z = 8;
    if (zero_point) z = (int)((qzeros[zero_word_index(n, grp, G)] >> (4 * (n & 7))) & 15u);
    const uint32_t word = qweight[idx];
    half8_t out;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int q = (int)((word >> nibble_shift(c)) & 15u);
      out[c] = (_Float16)((float)(q - z) * s);
    }
    w_out[idx] = __builtin_bit_cast(u32x4, out);
  }
}

template <bool ZP>
hipError_t launch_pack_zp(const void* w, int N, int K, int group_size, uint32_t* qweight, void* scales,
                          uint32_t* qzeros, hipStream_t stream) {
  // K is cut into slices of whole 512-channel passes (64 words, a multiple of
  // every group) until the grid has about 16384 blocks, which on the Llama-7B
  // layers makes every slice a single pass: one block per row octet streams
  // a row with too few loads in flight (243 us per Llama-7B block of 7
  // linears with the first quantizer, against 206-212 us with slices of 1024
  // channels).  With two words per lane, 16384 target blocks are 3-6% faster
  // than 8192 (a 4096-row layer then already has one-pass slices, the
  // 11008-row ones had two) and 2048 are 7% slower.
  constexpr int kTargetBlocks = 16384, kRingWords = 32 * kPackWords;
  const int kw = K >> 3, octets = N / 8;
  const int rings = (kw + kRingWords - 1) / kRingWords;
  int slices = (kTargetBlocks + octets - 1) / octets;
  if (slices > rings) slices = rings;
  if (slices < 1) slices = 1;
  const int chunk = ((rings + slices - 1) / slices) * kRingWords;
  const dim3 grid(octets, (kw + chunk - 1) / chunk), block(kPackThreads);
  const u32x4* wv = static_cast<const u32x4*>(w);
  uint16_t* sc = static_cast<uint16_t*>(scales);
  switch (group_size) {
    case 32: hipLaunchKernelGGL((pack_kernel<4 / kPackWords, ZP>), grid, block, 0, stream, wv, N, K, chunk, qweight, sc, qzeros); break;
    case 64: hipLaunchKernelGGL((pack_kernel<8 / kPackWords, ZP>), grid, block, 0, stream, wv, N, K, chunk, qweight, sc, qzeros); break;
    case 128: hipLaunchKernelGGL((pack_kernel<16 / kPackWords, ZP>), grid, block, 0, stream, wv, N, K, chunk, qweight, sc, qzeros); break;
    case 256: hipLaunchKernelGGL((pack_kernel<32 / kPackWords, ZP>), grid, block, 0, stream, wv, N, K, chunk, qweight, sc, qzeros); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

int log2_group(int g) { return g == 32 ? 5 : g == 64 ? 6 : g == 128 ? 7 : 8; }

template <bool ZP>
hipError_t launch_scale_error_zp(const void* w, const float* s, int count, int N, int K, int group_size, void* e,
                                 hipStream_t stream) {
  const dim3 grid(N / 8, count), block(kPackThreads);
  const u32x4* wv = static_cast<const u32x4*>(w);
  u32x4* ev = static_cast<u32x4*>(e);
  switch (group_size) {
    case 32: hipLaunchKernelGGL((scale_error_kernel<4 / kPackWords, ZP>), grid, block, 0, stream, wv, s, N, K, ev); break;
    case 64: hipLaunchKernelGGL((scale_error_kernel<8 / kPackWords, ZP>), grid, block, 0, stream, wv, s, N, K, ev); break;
    case 128: hipLaunchKernelGGL((scale_error_kernel<16 / kPackWords, ZP>), grid, block, 0, stream, wv, s, N, K, ev); break;
    case 256: hipLaunchKernelGGL((scale_error_kernel<32 / kPackWords, ZP>), grid, block, 0, stream, wv, s, N, K, ev); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool ZP>
hipError_t launch_clip_zp(const void* w, const ClipRatios& ratios, int count, int N, int K, int group_size, void* e,
                          const int32_t* choice, void* w_out, bool apply, hipStream_t stream) {
  const u32x4* wv = static_cast<const u32x4*>(w);
  const dim3 block(kPackThreads);
#define AWQ_CLIP_CASE(G_, GW_)                                                                                   \
  case G_:                                                                                                     \
    if (!apply)                                                                                                \
      hipLaunchKernelGGL((clip_error_kernel<GW_ / kPackWords, ZP>), dim3(N / 8, count), block, 0, stream, wv,     \
                         ratios, N, K,                                                                         \
                         static_cast<u32x4*>(e));                                                              \
    else                                                                                                       \
      hipLaunchKernelGGL((clip_apply_kernel<GW_, ZP>), dim3(N / 8), block, 0, stream, wv, N, K, ratios, choice,  \
                         static_cast<u32x4*>(w_out));                                                          \
    break;
  switch (group_size) {
    AWQ_CLIP_CASE(32, 4)
    AWQ_CLIP_CASE(64, 8)
    AWQ_CLIP_CASE(128, 16)
    AWQ_CLIP_CASE(256, 32)
    default: return hipErrorInvalidValue;
  }
#undef AWQ_CLIP_CASE
  return hipGetLastError();
}

}  // namespace

hipError_t launch_clip_error(const void* w, const ClipRatios& ratios, int count, int N, int K, int group_size,
                             bool zero_point, void* e, hipStream_t stream) {
  return zero_point ? launch_clip_zp<true>(w, ratios, count, N, K, group_size, e, nullptr, nullptr, false, stream)
                    : launch_clip_zp<false>(w, ratios, count, N, K, group_size, e, nullptr, nullptr, false, stream);
}

hipError_t launch_clip_apply(const void* w, const float* part, int parts, const ClipRatios& ratios, int count, int N,
                             int K, int group_size, bool zero_point, void* w_out, int32_t* choice, hipStream_t stream) {
  const int G = K / group_size;
  const size_t groups = (size_t)G * N;
  hipLaunchKernelGGL(clip_choose_kernel, dim3((unsigned)((groups + 255) / 256)), dim3(256), 0, stream, part, parts, G,
                     N, count, choice);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return zero_point ? launch_clip_zp<true>(w, ratios, count, N, K, group_size, nullptr, choice, w_out, true, stream)
                    : launch_clip_zp<false>(w, ratios, count, N, K, group_size, nullptr, choice, w_out, true, stream);
}

hipError_t launch_scale_error(const void* w, const float* s, int count, int N, int K, int group_size, bool zero_point,
                              void* e, hipStream_t stream) {
  return zero_point ? launch_scale_error_zp<true>(w, s, count, N, K, group_size, e, stream)
                    : launch_scale_error_zp<false>(w, s, count, N, K, group_size, e, stream);
}

hipError_t launch_pack(const void* w, int N, int K, int group_size, bool zero_point, uint32_t* qweight,
                       void* scales, uint32_t* qzeros, hipStream_t stream) {
  return zero_point ? launch_pack_zp<true>(w, N, K, group_size, qweight, scales, qzeros, stream)
                    : launch_pack_zp<false>(w, N, K, group_size, qweight, scales, qzeros, stream);
}

hipError_t launch_dequant(const uint32_t* qweight, const void* scales, const uint32_t* qzeros, void* w_out,
                          int N, int K, int group_size, bool zero_point, hipStream_t stream) {
  const size_t words = (size_t)N * (K >> 3);
  size_t blocks = (words + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(dequant_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, qweight,
                     static_cast<const uint16_t*>(scales), qzeros, static_cast<u32x4*>(w_out), N, K,
                     log2_group(group_size), zero_point ? 1 : 0);
  return hipGetLastError();
}

}  // namespace awq
