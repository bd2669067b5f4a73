// Activation-aware scale search: candidate per-channel scales from activation
// statistics (awq_scale_candidates) and the reconstruction error L(s) of each
// candidate (awq_scale_loss).
//
// "AI-Research-SKILLs AWQ 高级使用指南", section 算法原理: AWQ finds the ~1% of
// salient weight channels from the distribution of the activations, multiplies
// them by a scaling factor before quantization, and chooses the scaling to
// make the reconstruction error
//   L(s) = || Q(W * s)(s^-1 * X) - W * X ||
// small.  "AWQ Activation-aware Weight Quantization (Lin 2023年)" lists the
// ingredients as activation statistics and per-channel scaling.  The pages do
// not give the family of candidate scales; the one used here is
//   s_k = a_k ^ alpha,  a_k = max(mean_m |x_mk|, 1e-4)
// for a grid of exponents alpha (alpha = 0 is plain round-to-nearest), or,
// with duo scaling (the calibration parameter duo_scaling, "scale weights and
// activations", section 自定义校准策略 / 校准参数全景), also divided by a
// weight statistic of the channel:
//   s_k = a_k ^ alpha / b_k ^ (1 - alpha),  b_k = max(mean_n |w_nk|, 1e-4).
//
// L(s) is evaluated as || X e^T ||_F with e = Q(W s) s^-1 - W (the same
// quantity, one dense product instead of two), written as
//   X e^T = (X diag(s)^-1) (Q(W s) - W diag(s))^T:
// the activations are scaled once per candidate and the weight error
// Q(W s) - W s is built tile by tile next to the matrix cores
// (loss_fused_kernel) and never stored.  The product runs on the fp16 matrix
// cores with fp32 accumulation; the squares are summed per wave and the
// partial sums are added in a fixed order in fp64 (deterministic).
#include "awq_device.hpp"
#include "awq_launch.hpp"
#include "awq_quant.hpp"

#include <type_traits>

namespace awq {
namespace {

// ---------------------------------------------------------------------------
// Activation statistics and candidates.
// ---------------------------------------------------------------------------
constexpr int kStatRows = 64;  // rows of X (or W) summed per partial
constexpr float kActFloor = 1e-4f;
constexpr float kWeightFloor = 1e-4f;

// partial[b][k] = sum over rows 64 b .. 64 b + 63 of |x_mk|, in row order
// (activations, or weights for duo scaling).  One thread per channel;
// consecutive threads read consecutive channels.
__global__ __launch_bounds__(256) void act_partial_kernel(const _Float16* __restrict__ x, int M, int K,
                                                          float* __restrict__ partial) {
  const int k = blockIdx.x * 256 + threadIdx.x;
  if (k >= K) return;
  const int m0 = blockIdx.y * kStatRows, m1 = min(M, m0 + kStatRows);
  float acc = 0.0f;
  for (int m = m0; m < m1; ++m) acc += fabsf((float)x[(size_t)m * K + k]);
  partial[(size_t)blockIdx.y * K + k] = acc;
}

struct Alphas {
  float v[kMaxScaleCandidates];
};

// a_k = max((sum of the partials in order) / M, 1e-4); s[c][k] = a_k ^ alpha_c,
// or with duo scaling (wparts > 0) b_k = max((sum of the weight partials in
// order) / N, 1e-4) and s[c][k] = a_k ^ alpha_c / b_k ^ (1 - alpha_c).
__global__ __launch_bounds__(256) void candidates_kernel(const float* __restrict__ partial, int nparts, int M,
                                                         const float* __restrict__ wpartial, int wparts, int N, int K,
                                                         Alphas alphas, int count, float* __restrict__ s) {
  const int k = blockIdx.x * 256 + threadIdx.x;
  if (k >= K) return;
  float sum = 0.0f;
  for (int b = 0; b < nparts; ++b) sum += partial[(size_t)b * K + k];
  const float a = fmaxf(sum / (float)M, kActFloor);
  if (wparts == 0) {
    for (int c = 0; c < count; ++c) s[(size_t)c * K + k] = alphas.v[c] == 0.0f ? 1.0f : powf(a, alphas.v[c]);
    return;
  }
  float wsum = 0.0f;
  for (int b = 0; b < wparts; ++b) wsum += wpartial[(size_t)b * K + k];
  const float bk = fmaxf(wsum / (float)N, kWeightFloor);
  for (int c = 0; c < count; ++c) {
    const float al = alphas.v[c];
    const float num = al == 0.0f ? 1.0f : al == 1.0f ? a : powf(a, al);
    const float den = al == 1.0f ? 1.0f : al == 0.0f ? bk : powf(bk, 1.0f - al);
    s[(size_t)c * K + k] = num / den;
  }
}

// The search's choice: the first candidate with the smallest loss (a NaN
// loss is never chosen), written to best[0], and its scale vector copied to
// s_best.  Every workgroup finds the same index (count <= 64) and copies
// its share of the K channels.
__global__ __launch_bounds__(256) void scale_choose_kernel(const double* __restrict__ loss, int count,
                                                           const float* __restrict__ s_all, int K,
                                                           float* __restrict__ s_best, int32_t* __restrict__ best) {
  int idx = 0;
  double lo = __builtin_inf();
  for (int c = 0; c < count; ++c) {
    const double v = loss[c];
    if (v < lo) {
      lo = v;
      idx = c;
    }
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) best[0] = idx;
  const float* src = s_all + (size_t)idx * K;
  for (int k = blockIdx.x * 256 + threadIdx.x; k < K; k += gridDim.x * 256) s_best[k] = src[k];
}

// dst[r][k] = fp16(src[r][k] * s[k]) (or / s[k]): fp32 product or correctly
// rounded fp32 quotient, rounded once to fp16.  One thread per 8 channels.
__global__ __launch_bounds__(256) void scale_columns_kernel(const u32x4* __restrict__ src, int rows, int K,
                                                            const float* __restrict__ s, int divide,
                                                            u32x4* __restrict__ dst) {
  const int kw = K >> 3;
  const size_t total = (size_t)rows * kw;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (size_t)gridDim.x * 256) {
    const int j = (int)(i % kw);
    const half8_t h = as_half8(src[i]);
    const float4_t s0 = *reinterpret_cast<const float4_t*>(s + 8 * j);
    const float4_t s1 = *reinterpret_cast<const float4_t*>(s + 8 * j + 4);
    half8_t out;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float sc = c < 4 ? s0[c] : s1[c - 4];
      out[c] = (_Float16)(divide ? (float)h[c] / sc : fp32_product((float)h[c], sc));
    }
    dst[i] = __builtin_bit_cast(u32x4, out);
  }
}

// ---------------------------------------------------------------------------
// Shared by the loss products.
// ---------------------------------------------------------------------------
// Buffer resource over `bytes` bytes at `base`: loads past the end return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
constexpr uint32_t kOutOfRange = 0x80000000u;

constexpr int TK = 64;  // K step

// 16-byte chunk c of LDS row r sits in slot c ^ ((r >> 1) & 7): with 128-byte
// rows, 16 consecutive rows read at the same logical chunk hit 16 distinct
// bank groups, and a 1 KiB run of slots is what one buffer-to-LDS load of 64
// lanes x 16 bytes writes.
__device__ __forceinline__ int swz_chunk(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

// ---------------------------------------------------------------------------
// The loss product with the weight error built in place.
// ---------------------------------------------------------------------------
// xs[c][m][k] = fp16(x[m][k] * rcp(s_c[k])): the activations of candidate c
// (the reciprocal within 1 ulp; the operand only needs fp16 accuracy).  One
// thread per 8 channels.
__global__ __launch_bounds__(256) void scaled_activations_kernel(const u32x4* __restrict__ x,
                                                                 const float* __restrict__ s_all, int M, int K,
                                                                 u32x4* __restrict__ xs) {
  const int kw = K >> 3;
  const size_t words = (size_t)M * kw;
  const int c = blockIdx.y;
  const float* sc = s_all + (size_t)c * K;
  u32x4* out = xs + (size_t)c * words;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < words; i += (size_t)gridDim.x * 256) {
    const int j = (int)(i % kw);
    const half8_t h = as_half8(x[i]);
    const float4_t s0 = *reinterpret_cast<const float4_t*>(sc + 8 * j);
    const float4_t s1 = *reinterpret_cast<const float4_t*>(sc + 8 * j + 4);
    half8_t r;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      r[q] = (_Float16)((float)h[q] * __builtin_amdgcn_rcpf(s0[q]));
      r[4 + q] = (_Float16)((float)h[4 + q] * __builtin_amdgcn_rcpf(s1[q]));
    }
    out[i] = __builtin_bit_cast(u32x4, r);
  }
}

// fp16(fma(-h_lo, b0, c0)) | fp16(fma(-h_hi, b1, c1)) << 16 for the two fp16
// halves of h2: each a single rounding of the exact fused multiply-add,
// written straight into its half of the result (v_fma_mixlo/hi_f16 take the
// fp16 operand as it is packed).
__device__ __forceinline__ uint32_t neg_fma_pair(uint32_t h2, float b0, float c0, float b1, float c1) {
  uint32_t r;
  asm("v_fma_mixlo_f16 %0, -%1, %2, %3 op_sel_hi:[1,0,0]\n\t"
      "v_fma_mixhi_f16 %0, -%1, %4, %5 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
      : "=&v"(r)
      : "v"(h2), "v"(b0), "v"(c0), "v"(b1), "v"(c1));
  return r;
}

// fp16(c0 - h_lo) | fp16(c1 - h_hi) << 16, single roundings, as above.
__device__ __forceinline__ uint32_t neg_add_pair(uint32_t h2, float c0, float c1) {
  uint32_t r;
  asm("v_fma_mixlo_f16 %0, -%1, 1.0, %2 op_sel_hi:[1,0,0]\n\t"
      "v_fma_mixhi_f16 %0, -%1, 1.0, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
      : "=&v"(r)
      : "v"(h2), "v"(c0), "v"(c1));
  return r;
}

// Scaled errors of one row's 8 channels of one group for one candidate:
//   e = fp16( (q - z) * s_g - w * s_c ),  q = clamp(rne(a / s_g) + z, 0, 15),  a = fp16(w * s_c)
// with the group's fp16 scale s_g and zero point z from p = s_g bits |
// z << 16, and q by pack_kernel's rule (a is the fp32 product rounded to
// fp16, as the quantizer sees it).  With k = 768 + rne(a / s_g) from
// biased_quotients, med3(k, 768 - z, 783 - z) - 768 is q - z, and
// fma(med3(..), s_g, -768 s_g) is (q - z) s_g exactly (small integers times
// an fp16 value); the error is then one fused multiply-add rounded once to
// fp16.  The product w * s_c is taken as fma(w, s_c, +0) so that the fp16
// weight enters it without a conversion (the +0 changes only the sign of a
// zero product, and the code of a zero is the zero point either way).
__device__ __forceinline__ u32x4 scaled_error8(u32x4 raw, uint32_t p, float4_t s0, float4_t s1) {
#pragma clang fp contract(off)
  const half8_t h = as_half8(raw);
  const float sv[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
  const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)(p & 0xFFFFu));
  const float zf = (float)(p >> 16);
  const float lob = kCodeBias - zf, hib = kCodeBias + 15.0f - zf, off = -kCodeBias * s;
  float a[8], k[8], d[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    float prod = __builtin_fmaf((float)h[c], sv[c], 0.0f);
    asm("" : "+v"(prod));  // keep the fp32 rounding of the product (see fp32_product)
    a[c] = (float)(_Float16)prod;
  }
  biased_quotients(a, __builtin_amdgcn_rcpf(s), k);
#pragma unroll
  for (int c = 0; c < 8; ++c) d[c] = __builtin_fmaf(__builtin_amdgcn_fmed3f(k[c], lob, hib), s, off);
  u32x4 e;
#pragma unroll
  for (int i = 0; i < 4; ++i) e[i] = neg_fma_pair(raw[i], sv[2 * i], d[2 * i], sv[2 * i + 1], d[2 * i + 1]);
  return e;
}

// Clipped errors of one row's 8 channels of one group for one ratio:
//   e = fp16( (q - z) * s_g - w ),  q = clamp(rne(c / s_g) + z, 0, 15),  c = clamp(w, lo, hi)
// with p = { s_g bits | z << 16, fp16(lo) bits | fp16(hi) bits << 16 }, the
// group's clipped scale, zero point and fp32 bounds rounded to fp16.  For an
// fp16 weight, clamping to the rounded bounds gives the fp16 rounding of the
// clamp to the fp32 bounds (no fp16 value lies strictly between a bound and
// its nearest fp16 value), which is what the quantizer sees.  Codes and
// (q - z) s_g as in scaled_error8.
__device__ __forceinline__ u32x4 clipped_error8(u32x4 raw, u32x2 p) {
#pragma clang fp contract(off)
  const half8_t h = as_half8(raw);
  const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)(p[0] & 0xFFFFu));
  const float zf = (float)(p[0] >> 16);
  const float lo = (float)__builtin_bit_cast(_Float16, (uint16_t)(p[1] & 0xFFFFu));
  const float hi = (float)__builtin_bit_cast(_Float16, (uint16_t)(p[1] >> 16));
  const float lob = kCodeBias - zf, hib = kCodeBias + 15.0f - zf, off = -kCodeBias * s;
  float a[8], k[8], d[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) a[c] = __builtin_amdgcn_fmed3f((float)h[c], lo, hi);
  biased_quotients(a, __builtin_amdgcn_rcpf(s), k);
#pragma unroll
  for (int c = 0; c < 8; ++c) d[c] = __builtin_fmaf(__builtin_amdgcn_fmed3f(k[c], lob, hib), s, off);
  u32x4 e;
#pragma unroll
  for (int i = 0; i < 4; ++i) e[i] = neg_add_pair(raw[i], d[2 * i], d[2 * i + 1]);
  return e;
}

// Scheduling pattern of one step of the loss product: per 16-channel slice
// the slice's fragment reads, then its 8 products each followed by 4 of the
// error build's VALU instructions (the matrix cores take 32 cycles per
// 32x32x16 product, in whose shadow a few independent VALU instructions
// issue for free), then the rest of the build and its LDS writes.
template <int N>
__device__ __forceinline__ void products_with_valu() {
  if constexpr (N > 0) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // four VALU
    products_with_valu<N - 1>();
  }
}

template <int SLICES>
__device__ __forceinline__ void interleave_step() {
  if constexpr (SLICES > 0) {
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);  // the slice's fragment reads
    products_with_valu<8>();
    interleave_step<SLICES - 1>();
  }
}

// The loss products of the two searches, with the weight error built in
// place:
//  * scale search (CLIP false): the sum of the squares of xs_c e_c^T for
//    candidate c, e_c as in scaled_error8 with the group quantities of
//    scale_group_params_kernel (= L(s_c)^2);
//  * clip search (CLIP true): for ratio c, the squares of x e_c^T summed per
//    group of input channels (the output error of each weight group, e_c as
//    in clipped_error8 with the quantities of clip_group_params_kernel).
// e never goes to memory: every K step the workgroup builds the 128 x 64 tile
// of e for the next step from weights already in registers and writes it to
// LDS, where the matrix cores read it as the B operand while the activations
// stream in by buffer-to-LDS loads.  Tile 512 tokens x 128 weight rows, so an
// element of e (about eight fp32 operations) is built once per 512 tokens,
// against 512 multiply-adds on the matrix cores; 8 waves of 128 x 64 (4 x 2
// v_mfma_f32_32x32x16_f16 tiles), two per SIMD, so that one wave's loads,
// build and LDS waits overlap the other's products (one wave per SIMD with
// 128 x 128 tiles was 5-10% slower); 160 KiB of LDS.  Operands through LDS:
// 16-byte chunk c of row r in slot c ^ ((r >> 1) & 7).  For the build, lane l
// of wave w takes channels 8 (l % 8) .. + 7 of the step (LDS chunk l % 8) in
// rows 16 w + l / 8 and 16 w + 8 + l / 8, so each wave load covers whole
// 128-byte lines of 8 rows.  Every load is an unconditional buffer load
// (out-of-range offsets return zero): no branch separates a load from its
// use, and the waits count exactly.  Tiles are ordered candidate-major: the
// workgroups on one XCD share one candidate's activations in its L2.
// Output: scale search, per wave the fp64 value of its fp32 sum of squares,
// partial[(c * tiles + tile) * 8 + wave]; clip search, at every group
// boundary each wave adds the squares of its accumulators over its 128
// tokens per column, writes them to gpart[c][tm][wave % 4][group][n] and
// restarts its accumulators from zero.
constexpr int kLossM = 512, kLossN = 128, kLossWaves = 8, kLossWM = 4;

template <bool KTAIL, bool CLIP, bool MIDFLUSH = false>
__global__ __launch_bounds__(kLossWaves * 64) void loss_fused_kernel(const _Float16* __restrict__ XS,
                                                                   const _Float16* __restrict__ W,
                                                                   const float* __restrict__ s_all,
                                                                   const uint32_t* __restrict__ gp, int M, int N, int K,
                                                                   int gshift, int tiles_m, int tiles,
                                                                   double* __restrict__ partial,
                                                                   float* __restrict__ gpart) {
  constexpr int AM = 4, AN = 2, WM = kLossWM;
  constexpr int XOP = kLossM * TK * 2, EOP = kLossN * TK * 2;
  constexpr int PE = CLIP ? 8 : 4;  // bytes of one group-parameter entry
  typedef typename std::conditional<CLIP, u32x2, uint32_t>::type param_t;
  __shared__ __attribute__((aligned(1024))) char lx0[XOP], lx1[XOP], le0[EOP], le1[EOP];
  // (the wave index is uniform: readfirstlane keeps it, and the LDS addresses
  // derived from it, in scalar registers)
  const int t = threadIdx.x, lane = t & 63, wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int lin = xcd_contiguous_tile(blockIdx.x, gridDim.x);
  const int cand = lin / tiles, tile = lin - cand * tiles;
  const int tm = tile % tiles_m, tn = tile / tiles_m;
  const int m0 = tm * kLossM, n0 = tn * kLossN;
  const int rows_m = min(kLossM, M - m0), rows_n = min(kLossN, N - n0);
  const int nsteps = (K + TK - 1) / TK;
  const int G = K >> gshift;

  // activations (each candidate's scaled copy for the scale search, the one
  // X for the clip search): wave w fills rows 64 w .. 64 w + 63 of the X tile
  // with 8 loads of 8 rows x 128 B (lane l: row 64 w + 8 j + l / 8, slot
  // l % 8).  The swizzled chunk of a lane depends on j only through j's
  // parity, so two lane offsets serve all 8 loads; the row block 8 j and the
  // step go in the scalar offset.
  const __amdgpu_buffer_rsrc_t rx =
      rsrc(XS + ((CLIP ? 0 : (size_t)cand * M) + m0) * K, (uint32_t)rows_m * K * 2);
  const int xrow = 64 * wave + (lane >> 3);
  int xchunk[2];
  uint32_t xoff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    xchunk[j] = swz_chunk(xrow + 8 * j, lane & 7);
    xoff[j] = (uint32_t)xrow * K * 2 + xchunk[j] * 16;
  }
  auto load_x = [&](int step, int buf) {
    char* dx = (buf ? lx1 : lx0) + wave * 8192;
    // (readfirstlane: the step offset stays scalar instead of being shared
    // with the weights' lane offsets, which would make the loads divergent)
    const int sx = __builtin_amdgcn_readfirstlane(step * TK * 2);
    // the scalar offset is outside the hardware's range check: rows past M
    // and a prefetch past the last step take the out-of-range lane offset
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t o = step < nsteps && xrow + 8 * j < rows_m ? xoff[j & 1] : kOutOfRange;
      if constexpr (KTAIL) {
        if (step * TK + 8 * xchunk[j & 1] >= K) o = kOutOfRange;
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (__attribute__((address_space(3))) void*)(dx + 1024 * j), 16, o,
                                               sx + 8 * j * K * 2, 0, 0);
    }
  };

  // the error tile: this lane's two rows and one chunk of 8 channels
  const int ec = lane & 7, er0 = 16 * wave + (lane >> 3), er1 = er0 + 8;
  const bool ok0 = er0 < rows_n, ok1 = er1 < rows_n;
  const __amdgpu_buffer_rsrc_t rw = rsrc(W + (size_t)n0 * K, (uint32_t)rows_n * K * 2);
  const __amdgpu_buffer_rsrc_t rsv = rsrc(s_all + (CLIP ? 0 : (size_t)cand * K), CLIP ? 0u : (uint32_t)K * 4);
  // group parameters of this candidate (G * N * PE <= 2^31 bytes, checked by the caller)
  const __amdgpu_buffer_rsrc_t rg =
      rsrc(reinterpret_cast<const char*>(gp) + (size_t)cand * G * N * PE, (uint32_t)G * N * PE);
  const uint32_t wo0 = (uint32_t)er0 * K * 2 + 16 * ec, wo1 = (uint32_t)er1 * K * 2 + 16 * ec;
  const uint32_t go0 = (uint32_t)(n0 + er0) * PE, go1 = (uint32_t)(n0 + er1) * PE;
  struct Rows {
    u32x4 w0, w1;
    param_t p0, p1;
  };
  struct Scales {
    float4_t s0, s1;
  };
  // The loads below need no guards: past the last step or past K a scale or
  // group-parameter offset lies past its resource's range (zero), and a
  // weight offset reads the next row or nothing (the last row); the build
  // masks channels past K, and a tile built past the last step is never read.
  // the candidate's scales of the lane's 8 channels (the same for all rows:
  // L2-resident, loaded in the step that uses them)
  auto fetch_scales = [&](int step, Scales& c) {
    if constexpr (!CLIP) {
      const uint32_t so = (uint32_t)(step * TK + 8 * ec) * 4;
      c.s0 = __builtin_bit_cast(float4_t, __builtin_amdgcn_raw_buffer_load_b128(rsv, so, 0, 0));
      c.s1 = __builtin_bit_cast(float4_t, __builtin_amdgcn_raw_buffer_load_b128(rsv, so, 16, 0));
    }
  };
  auto fetch = [&](int step, Rows& f) {
    f.w0 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, wo0 + step * TK * 2, 0, 0));
    f.w1 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, wo1 + step * TK * 2, 0, 0));
    const uint32_t go = (uint32_t)((step * TK + 8 * ec) >> gshift) * N * PE;
    if constexpr (CLIP) {
      f.p0 = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rg, go + go0, 0, 0));
      f.p1 = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rg, go + go1, 0, 0));
    } else {
      f.p0 = __builtin_amdgcn_raw_buffer_load_b32(rg, go + go0, 0, 0);
      f.p1 = __builtin_amdgcn_raw_buffer_load_b32(rg, go + go1, 0, 0);
    }
  };
  const int es0 = er0 * 128 + 16 * swz_chunk(er0, ec), es1 = er1 * 128 + 16 * swz_chunk(er1, ec);
  // Rows past N and channels past K must hold zeros.  A row past N loads
  // zero weights (past its resource's range) but another row's group
  // parameters; given the parameters { scale 1, zero point 0, clip bounds 0 }
  // instead, its error is exactly zero (code 0, (q - z) s = 0, e = -0 * s_c + 0).
  // Channels past K (the K-tail variant) read the next row's weights and are
  // zeroed at the store.
  auto build = [&](int step, const Rows& f, const Scales& c, int buf) {
    u32x4 e0, e1;
    param_t p0 = f.p0, p1 = f.p1;
    if constexpr (!KTAIL) {
      if constexpr (CLIP) {
        p0 = ok0 ? p0 : u32x2{0x3C00u, 0u};
        p1 = ok1 ? p1 : u32x2{0x3C00u, 0u};
      } else {
        p0 = ok0 ? p0 : 0x3C00u;
        p1 = ok1 ? p1 : 0x3C00u;
      }
    }
    if constexpr (CLIP) {
      e0 = clipped_error8(f.w0, p0);
      e1 = clipped_error8(f.w1, p1);
    } else {
      e0 = scaled_error8(f.w0, p0, c.s0, c.s1);
      e1 = scaled_error8(f.w1, p1, c.s0, c.s1);
    }
    char* de = buf ? le1 : le0;
    if constexpr (KTAIL) {
      // (with the original parameters, a row past N may give NaN: masked here too)
      const bool kin = step * TK + 8 * ec < K;
      e0 = kin && ok0 ? e0 : u32x4{0u, 0u, 0u, 0u};
      e1 = kin && ok1 ? e1 : u32x4{0u, 0u, 0u, 0u};
    }
    *reinterpret_cast<u32x4*>(de + es0) = e0;
    *reinterpret_cast<u32x4*>(de + es1) = e1;
  };

  float16_t acc[AM][AN];
#pragma unroll
  for (int a = 0; a < AM; ++a)
#pragma unroll
    for (int b = 0; b < AN; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

  const int wm = (wave % WM) * (32 * AM), wn = (wave / WM) * (32 * AN);
  const int fi = lane & 31, fh = lane >> 5;  // fragment row and k-half of this lane
  const int fsw = (fi >> 1) & 7;             // swizzle of the fragment rows (bases are multiples of 32)
  // clip search: squares per column over this wave's 128 tokens; lanes l and
  // l + 32 hold the two halves of column l % 32 of each 32 x 32 tile
  float* gout = CLIP ? gpart + (((size_t)cand * tiles_m + tm) * WM + (wave % WM)) * G * N : nullptr;
  auto flush = [&](int grp) {
#pragma unroll
    for (int b = 0; b < AN; ++b) {
      float v = 0.0f;
#pragma unroll
      for (int a = 0; a < AM; ++a)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          v += acc[a][b][r] * acc[a][b][r];
          acc[a][b][r] = 0.0f;
        }
      v += __shfl_xor(v, 32);
      const int n = n0 + wn + 32 * b + lane;
      if (lane < 32 && n < N) gout[(size_t)grp * N + n] = v;
    }
  };
  auto compute = [&](int buf, int step) {
    const char* xa = (buf ? lx1 : lx0) + (wm + fi) * 128;
    const char* eb = (buf ? le1 : le0) + (wn + fi) * 128;
#pragma unroll
    for (int ks = 0; ks < TK / 16; ++ks) {
      const int slot = 16 * ((2 * ks + fh) ^ fsw);
      half8_t af[AM], bf[AN];
#pragma unroll
      for (int a = 0; a < AM; ++a) af[a] = *reinterpret_cast<const half8_t*>(xa + 32 * 128 * a + slot);
#pragma unroll
      for (int b = 0; b < AN; ++b) bf[b] = *reinterpret_cast<const half8_t*>(eb + 32 * 128 * b + slot);
#pragma unroll
      for (int a = 0; a < AM; ++a)
#pragma unroll
        for (int b = 0; b < AN; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[a], bf[b], acc[a][b], 0, 0, 0);
      if constexpr (CLIP && MIDFLUSH) {
        const int kend = step * TK + (ks + 1) * 16;  // channels done after this slice
        if ((kend & ((1 << gshift) - 1)) == 0 && kend <= K) flush((kend >> gshift) - 1);
      }
    }
  };
  // groups of 64 channels or more end at step boundaries (K is then a
  // multiple of 64): their flush follows the step's products, outside the
  // scheduled region
  auto step_flush = [&](int step) {
    if constexpr (CLIP && !MIDFLUSH) {
      const int kend = (step + 1) * TK;
      if ((kend & ((1 << gshift) - 1)) == 0) flush((kend >> gshift) - 1);
    }
  };
  constexpr bool kInterleave = !(CLIP && MIDFLUSH);

  // Two steps per trip (constant buffer indices).  A step's activation loads,
  // then the candidate scales and the weights two steps ahead, are issued
  // first; the error tile of the next step is then built while the matrix
  // cores work on this one (products first in program order, so that the
  // build's arithmetic fills the matrix cores' shadow).  The barrier at the
  // end of a step waits for the activation loads only: the register loads
  // issued after them stay in flight for a whole step.
  Rows cur, nxt;
  Scales sc, scn;
  fetch(0, cur);
  fetch_scales(0, sc);
  load_x(0, 0);
  fetch(1, nxt);
  fetch_scales(1, scn);
  build(0, cur, sc, 0);
  __syncthreads();
  int step = 0;
  for (; step + 1 < nsteps; step += 2) {
    cur = nxt;
    sc = scn;
    load_x(step + 1, 1);
    fetch_scales(step + 2, scn);
    fetch(step + 2, nxt);
    __builtin_amdgcn_sched_barrier(0);
    compute(0, step);
    build(step + 1, cur, sc, 1);
    if constexpr (kInterleave) {
      interleave_step<TK / 16>();
      __builtin_amdgcn_sched_group_barrier(0x002, 256, 0);  // the rest of the build
      __builtin_amdgcn_sched_group_barrier(0x200, 2, 0);    // its LDS writes
    }
    step_flush(step);
    __syncthreads();
    cur = nxt;
    sc = scn;
    load_x(step + 2, 0);
    fetch_scales(step + 3, scn);
    fetch(step + 3, nxt);
    __builtin_amdgcn_sched_barrier(0);
    compute(1, step + 1);
    // (past the last step this builds a tile that is never read: no branch
    // here, so the waits for the loads above stay exact)
    build(step + 2, cur, sc, 0);
    if constexpr (kInterleave) {
      interleave_step<TK / 16>();
      __builtin_amdgcn_sched_group_barrier(0x002, 256, 0);
      __builtin_amdgcn_sched_group_barrier(0x200, 2, 0);
    }
    step_flush(step + 1);
    __syncthreads();
  }
  if (step < nsteps) {
    compute(0, step);
    step_flush(step);
  }
  if constexpr (CLIP) return;

  float ss = 0.0f;
#pragma unroll
  for (int a = 0; a < AM; ++a)
#pragma unroll
    for (int b = 0; b < AN; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) ss += acc[a][b][r] * acc[a][b][r];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
  if (lane == 0) partial[((size_t)cand * tiles + tile) * kLossWaves + wave] = (double)ss;
}

// loss[c] = sqrt(sum of candidate c's tile partials), summed by one workgroup
// in a fixed order.
__global__ __launch_bounds__(256) void loss_finalize_kernel(const double* __restrict__ partial, int tiles,
                                                            double* __restrict__ loss) {
  __shared__ double red[256];
  const int t = threadIdx.x;
  const double* p = partial + (size_t)blockIdx.x * tiles;
  double v = 0.0;
  for (int i = t; i < tiles; i += 256) v += p[i];
  red[t] = v;
  __syncthreads();
  for (int h = 128; h >= 1; h >>= 1) {
    if (t < h) red[t] += red[t + h];
    __syncthreads();
  }
  if (t == 0) loss[blockIdx.x] = sqrt(red[0]);
}

size_t align256(size_t b) { return (b + 255) / 256 * 256; }

int log2_group(int g) { return g == 32 ? 5 : g == 64 ? 6 : g == 128 ? 7 : 8; }

}  // namespace

size_t scale_candidates_workspace_bytes(int M, int N, int K) {
  return align256((size_t)((M + kStatRows - 1) / kStatRows) * K * 4) +
         (N > 0 ? align256((size_t)((N + kStatRows - 1) / kStatRows) * K * 4) : 0);
}

hipError_t launch_scale_candidates(const void* x, int M, int K, const void* w, int N, const float* alphas, int count,
                                   float* s, void* workspace, hipStream_t stream) {
  const int nparts = (M + kStatRows - 1) / kStatRows;
  const int wparts = w ? (N + kStatRows - 1) / kStatRows : 0;
  float* partial = static_cast<float*>(workspace);
  float* wpartial = reinterpret_cast<float*>(static_cast<char*>(workspace) + align256((size_t)nparts * K * 4));
  hipLaunchKernelGGL(act_partial_kernel, dim3((K + 255) / 256, nparts), dim3(256), 0, stream,
                     static_cast<const _Float16*>(x), M, K, partial);
  if (wparts > 0)
    hipLaunchKernelGGL(act_partial_kernel, dim3((K + 255) / 256, wparts), dim3(256), 0, stream,
                       static_cast<const _Float16*>(w), N, K, wpartial);
  Alphas a;
  for (int c = 0; c < kMaxScaleCandidates; ++c) a.v[c] = c < count ? alphas[c] : 0.0f;
  hipLaunchKernelGGL(candidates_kernel, dim3((K + 255) / 256), dim3(256), 0, stream, partial, nparts, M, wpartial,
                     wparts, N, K, a, count, s);
  return hipGetLastError();
}

// Workspace of the loss: the group parameters (4 bytes per candidate, row and
// group, sized for the smallest group, 32 channels), the scaled activations
// (count x M x K fp16) and the per-wave partial sums.
size_t scale_loss_workspace_bytes(int count, int M, int N, int K) {
  const size_t tiles = (size_t)((M + kLossM - 1) / kLossM) * ((N + kLossN - 1) / kLossN);
  return align256((size_t)count * (K / 32) * N * 4) + align256((size_t)count * M * K * 2) +
         align256((size_t)count * tiles * kLossWaves * 8);
}

hipError_t launch_scale_loss(const void* x, const void* w, const float* s, int count, int M, int N, int K,
                             int group_size, bool zero_point, void* workspace, double* loss, hipStream_t stream) {
  const int tiles_m = (M + kLossM - 1) / kLossM, tiles_n = (N + kLossN - 1) / kLossN;
  const int tiles = tiles_m * tiles_n;
  char* ws = static_cast<char*>(workspace);
  uint32_t* gp = reinterpret_cast<uint32_t*>(ws);
  ws += align256((size_t)count * (K / 32) * N * 4);
  _Float16* xs = reinterpret_cast<_Float16*>(ws);
  ws += align256((size_t)count * M * K * 2);
  double* partial = reinterpret_cast<double*>(ws);
  hipError_t err = launch_scale_group_params(w, s, count, N, K, group_size, zero_point, gp, stream);
  if (err != hipSuccess) return err;
  const size_t words = (size_t)M * (K >> 3);
  size_t blocks = (words + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(scaled_activations_kernel, dim3((unsigned)blocks, count), dim3(256), 0, stream,
                     static_cast<const u32x4*>(x), s, M, K, reinterpret_cast<u32x4*>(xs));
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  const dim3 grid((unsigned)((size_t)tiles * count)), block(kLossWaves * 64);
  const _Float16* wh = static_cast<const _Float16*>(w);
  if (K % TK == 0)
    hipLaunchKernelGGL((loss_fused_kernel<false, false>), grid, block, 0, stream, xs, wh, s, gp, M, N, K,
                       log2_group(group_size), tiles_m, tiles, partial, nullptr);
  else
    hipLaunchKernelGGL((loss_fused_kernel<true, false>), grid, block, 0, stream, xs, wh, s, gp, M, N, K,
                       log2_group(group_size), tiles_m, tiles, partial, nullptr);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(loss_finalize_kernel, dim3(count), dim3(256), 0, stream, partial, tiles * kLossWaves, loss);
  return hipGetLastError();
}

// Workspace of the whole search: every candidate's scales, the candidates'
// statistics, the loss product's workspace and the losses.
size_t scale_search_workspace_bytes(int count, int M, int N, int K) {
  return align256((size_t)count * K * 4) + scale_candidates_workspace_bytes(M, N, K) +
         scale_loss_workspace_bytes(count, M, N, K) + align256((size_t)count * 8);
}

hipError_t launch_scale_search(const void* x, const void* w, int M, int N, int K, int group_size, bool zero_point,
                               const float* alphas, int count, bool duo, float* s_best, int32_t* best, double* losses,
                               void* workspace, hipStream_t stream) {
  char* ws = static_cast<char*>(workspace);
  float* s_all = reinterpret_cast<float*>(ws);
  ws += align256((size_t)count * K * 4);
  void* cand_ws = ws;
  ws += scale_candidates_workspace_bytes(M, N, K);
  void* loss_ws = ws;
  ws += scale_loss_workspace_bytes(count, M, N, K);
  double* L = losses ? losses : reinterpret_cast<double*>(ws);
  hipError_t err = launch_scale_candidates(x, M, K, duo ? w : nullptr, N, alphas, count, s_all, cand_ws, stream);
  if (err != hipSuccess) return err;
  err = launch_scale_loss(x, w, s_all, count, M, N, K, group_size, zero_point, loss_ws, L, stream);
  if (err != hipSuccess) return err;
  int blocks = (K + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(scale_choose_kernel, dim3(blocks), dim3(256), 0, stream, L, count, s_all, K, s_best, best);
  return hipGetLastError();
}

hipError_t launch_scale_columns(const void* src, int rows, int K, const float* s, bool divide, void* dst,
                                hipStream_t stream) {
  const size_t words = (size_t)rows * (K >> 3);
  size_t blocks = (words + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(scale_columns_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<const u32x4*>(src), rows, K, s, divide ? 1 : 0, static_cast<u32x4*>(dst));
  return hipGetLastError();
}

// Clip search workspace: the group parameters of every ratio (8 bytes per
// ratio, row and group) and the per-group partial errors
// part[c][tm][wave % 4][j][n] (4 token quarters of each 512-token tile).
size_t clip_search_workspace_bytes(int count, int M, int N, int K, int group_size) {
  const size_t tiles_m = (M + kLossM - 1) / kLossM, G = K / group_size;
  return align256((size_t)count * G * N * 8) + align256((size_t)count * tiles_m * kLossWM * G * N * 4);
}

hipError_t launch_clip_search(const void* x, const void* w, int M, int N, int K, int group_size, bool zero_point,
                              const float* ratios, int count, void* w_out, int32_t* choice, void* workspace,
                              hipStream_t stream) {
  const int tiles_m = (M + kLossM - 1) / kLossM, tiles_n = (N + kLossN - 1) / kLossN;
  const int tiles = tiles_m * tiles_n;
  const size_t G = K / group_size;
  char* ws = static_cast<char*>(workspace);
  uint32_t* gp = reinterpret_cast<uint32_t*>(ws);
  float* gpart = reinterpret_cast<float*>(ws + align256((size_t)count * G * N * 8));
  ClipRatios r;
  for (int c = 0; c < kMaxClipCandidates; ++c) r.v[c] = c < count ? ratios[c] : 1.0f;
  hipError_t err = launch_clip_group_params(w, r, count, N, K, group_size, zero_point, gp, stream);
  if (err != hipSuccess) return err;
  const dim3 grid((unsigned)((size_t)tiles * count)), block(kLossWaves * 64);
  const _Float16* xh = static_cast<const _Float16*>(x);
  const _Float16* wh = static_cast<const _Float16*>(w);
  // groups of 32 channels flush twice per step (K % 64 != 0 implies them)
  if (K % TK != 0)
    hipLaunchKernelGGL((loss_fused_kernel<true, true, true>), grid, block, 0, stream, xh, wh, nullptr, gp, M, N, K,
                       log2_group(group_size), tiles_m, tiles, nullptr, gpart);
  else if (group_size == 32)
    hipLaunchKernelGGL((loss_fused_kernel<false, true, true>), grid, block, 0, stream, xh, wh, nullptr, gp, M, N, K,
                       log2_group(group_size), tiles_m, tiles, nullptr, gpart);
  else
    hipLaunchKernelGGL((loss_fused_kernel<false, true, false>), grid, block, 0, stream, xh, wh, nullptr, gp, M, N, K,
                       log2_group(group_size), tiles_m, tiles, nullptr, gpart);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  // without a caller's choice buffer the choices go to the start of the
  // workspace: the group parameters there are dead once the product has run
  int32_t* ch = choice ? choice : reinterpret_cast<int32_t*>(ws);
  return launch_clip_apply(w, gpart, tiles_m * kLossWM, r, count, N, K, group_size, zero_point, w_out, ch, stream);
}

}  // namespace awq
