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
#include "awq_quant.hpp"

#pragma clang fp contract(off)


namespace awq {
namespace {

constexpr int kPackThreads = 256;  // 8 rows x 32 lanes
constexpr int kPackWords = 2;      // packed words (8 channels each) per lane and pass of pack_kernel
constexpr int kParamRows = 2;      // rows per lane of scale_group_params_kernel
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

      float s, zf;
      _Float16 s16;
      group_scale_zero<GW, ZP>(a, s16, s, zf);

      wordsT out;
#pragma unroll
      for (int i = 0; i < WPL; ++i) {
        float q[8];
        codes_of(aw[i], s, zf, q);
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

// Group parameters of the candidate-scaled weights, for the objective
//   L(s) = || Q(W diag(s)) (diag(s)^-1 X) - W X ||
// ("AI-Research-SKILLs AWQ 高级使用指南", section 算法原理), which the loss
// product evaluates with the quantization error of W diag(s) built tile by
// tile beside the matrix cores.  What needs a whole group comes from here:
// for every candidate c, row n and group j of the scaled weights
// a = fp16(w[n][k] * s_c[k]) (fp32 product, rounded once to fp16),
//   gp[c][j][n] = fp16 scale bits | zero point << 16,
// the scale and zero point of pack_kernel's quantizer, so that the loss
// product's codes are pack_kernel's codes bit for bit.  The weights are read
// once for all candidates.  The group's extremes of a are the fp16 roundings
// of the extremes of the fp32 products (rounding is monotone), so a lane
// takes the extremes of its 16 products per candidate and rounds only the
// group's two.  Candidates go in sets of GW (the lanes of a group): a
// transposed reduction leaves lane p of the group with the extremes of
// candidate p of the set, and each lane computes one scale and zero point
// (two divisions) per set instead of one per candidate; the set's scale
// vectors are staged in LDS, and each lane holds the same 16 channels of two
// rows, so that every scale it reads serves two products.  Blocks of 16 rows
// x 512-channel passes, K sliced as in pack_kernel.
template <int GW, bool ZP>
__global__ __launch_bounds__(kPackThreads) void scale_group_params_kernel(const u32x4* __restrict__ w,
                                                                          const float* __restrict__ s_all, int count,
                                                                          int N, int K, int chunk_words,
                                                                          uint32_t* __restrict__ gp) {
  constexpr int WPL = kPackWords;
  constexpr int kPass = 32 * WPL;
  constexpr int RPL = kParamRows;  // rows per lane: each scale read from LDS serves RPL products
  const int t = threadIdx.x;
  const int r = t >> 5, l = t & 31;
  const int nb = blockIdx.x * 8 * RPL;  // the block's first row
  const int n0 = nb + RPL * r;          // this lane's rows n0 .. n0 + RPL - 1
  const int kw = K >> 3;
  const int G = kw / (WPL * GW);
  __shared__ float4_t lsc[GW * kPass * 2];  // GW candidates x 512 channels of scales
  const int pos = l % GW;  // the lane's place in its group
  const int j_begin = blockIdx.y * chunk_words;
  const int j_end = min(kw, j_begin + chunk_words);  // multiples of WPL: no lane's words straddle j_end
  // Unconditional buffer loads: a lane past the slice end reads other
  // weights or zeros and writes nothing, and its whole group is past the end
  // with it (no branch around each load); rows past N read zeros.
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<u32x4*>(w + (size_t)nb * kw), 0, min(8 * RPL, N - nb) * kw * 16, 0x00020000);
  for (int w0 = j_begin; w0 < j_end; w0 += kPass) {
    const int j = w0 + WPL * l;
    const bool active = j < j_end;
    float hv[RPL][8 * WPL];
#pragma unroll
    for (int rr = 0; rr < RPL; ++rr)
#pragma unroll
      for (int i = 0; i < WPL; ++i) {
        const half8_t h = __builtin_bit_cast(
            half8_t, __builtin_amdgcn_raw_buffer_load_b128(rw, (uint32_t)((RPL * r + rr) * kw + j + i) * 16, 0, 0));
#pragma unroll
        for (int c = 0; c < 8; ++c) hv[rr][8 * i + c] = (float)h[c];
      }
    const int grp = j / (WPL * GW);
    for (int c0 = 0; c0 < count; c0 += GW) {
      // the set's scales of this pass's 512 channels, staged in LDS once per
      // block: the rows of the block read the same ones (per-lane global
      // loads of them kept the address units busy ~80% of the time)
      __syncthreads();
      for (int q = t; q < GW * kPass * 2; q += kPackThreads) {
        const int i = q / (kPass * 2), f = q % (kPass * 2);  // candidate of the set, float4 of the pass
        const int c = min(c0 + i, count - 1);                 // a short last set repeats the last candidate
        const int k = 8 * w0 + 4 * f;
        lsc[q] = k < K ? *reinterpret_cast<const float4_t*>(s_all + (size_t)c * K + k) : float4_t{1.f, 1.f, 1.f, 1.f};
      }
      __syncthreads();
      int mn[RPL][GW], mx[RPL][GW];  // order-preserving images of the lane's extremes
#pragma unroll
      for (int i = 0; i < GW; ++i) {
        if (c0 + i >= count) {  // a short last set: nothing to compute (uniform branch)
#pragma unroll
          for (int rr = 0; rr < RPL; ++rr) mn[rr][i] = mx[rr][i] = 0;
          continue;
        }
        float sv[8 * WPL];
#pragma unroll
        for (int q4 = 0; q4 < 2 * WPL; ++q4) {
          const float4_t v = lsc[i * kPass * 2 + 2 * WPL * l + q4];
#pragma unroll
          for (int q = 0; q < 4; ++q) sv[4 * q4 + q] = v[q];
        }
#pragma unroll
        for (int rr = 0; rr < RPL; ++rr) {
          if constexpr (ZP) {
            float lo = fp32_product(hv[rr][0], sv[0]), hi = lo;
#pragma unroll
            for (int q = 1; q < 8 * WPL; ++q) {
              const float v = fp32_product(hv[rr][q], sv[q]);
              lo = fminf(lo, v);
              hi = fmaxf(hi, v);
            }
            mn[rr][i] = ord_of(lo);
            mx[rr][i] = ord_of(hi);
          } else {
            float hi = fabsf(fp32_product(hv[rr][0], sv[0]));
#pragma unroll
            for (int q = 1; q < 8 * WPL; ++q) hi = fmaxf(hi, fabsf(fp32_product(hv[rr][q], sv[q])));
            mx[rr][i] = ord_of(hi);
          }
        }
      }
      const int c = c0 + pos;
#pragma unroll
      for (int rr = 0; rr < RPL; ++rr) {
        if constexpr (ZP) group_transpose<GW>(mn[rr], MinOp());
        group_transpose<GW>(mx[rr], MaxOp());
        float s, zf;
        _Float16 s16;
        scale_zero_of_extremes<ZP>(ZP ? (float)(_Float16)float_of(mn[rr][0]) : 0.0f,
                                   (float)(_Float16)float_of(mx[rr][0]), s16, s, zf);
        const int n = n0 + rr;
        if (active && c < count && n < N)
          gp[((size_t)c * G + grp) * N + n] = (uint32_t)__builtin_bit_cast(uint16_t, s16) | ((uint32_t)zf << 16);
      }
    }
  }
}

// Group parameters of weight clipping, for the search of apply_clip
// ("AI-Research-SKILLs AWQ 高级使用指南", section 自定义校准策略 (校准参数全景): clip the
// weights to reduce the effect of outliers on the quantization error).  For
// ratio r_c every group is clamped to its range shrunk by r_c ([r min, r max]
// with a zero point, [-r amax, r amax] without; fp32 products), the clamped
// weights are rounded to fp16 and quantized as by pack_kernel.  Clamping and
// rounding are monotone, so the clamped group's extremes are those of its
// unclamped extremes: one pass over the weights gives every ratio's scale and
// zero point.  Per (ratio c, group j, row n):
//   gp[c][j][n] = { fp16 scale bits | zero point << 16, fp16(lo) bits | fp16(hi) bits << 16 }.
// The GW lanes of a group share its extremes and split the ratios between
// them (lane p takes ratios p, p + GW, ...), so each lane computes about
// count / GW scales.  Same block shape and K slices as pack_kernel.
template <int GW, bool ZP>
__global__ __launch_bounds__(kPackThreads) void clip_group_params_kernel(const u32x4* __restrict__ w,
                                                                         ClipRatios ratios, int count, int N, int K,
                                                                         int chunk_words, u32x2* __restrict__ gp) {
  constexpr int WPL = kPackWords;
  constexpr int kPass = 32 * WPL;
  const int t = threadIdx.x;
  const int r = t >> 5, l = t & 31;
  const int n = blockIdx.x * 8 + r;
  const int kw = K >> 3;
  const int G = kw / (WPL * GW);
  const int pos = l % GW;
  const int j_begin = blockIdx.y * chunk_words;
  const int j_end = min(kw, j_begin + chunk_words);  // multiples of WPL: no lane's words straddle j_end
  // unconditional loads: a lane past the slice end reads other weights or
  // zeros and writes nothing (its whole group is past the end with it)
  const __amdgpu_buffer_rsrc_t rw =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<u32x4*>(w + (size_t)blockIdx.x * 8 * kw), 0, 8 * kw * 16, 0x00020000);
  for (int w0 = j_begin; w0 < j_end; w0 += kPass) {
    const int j = w0 + WPL * l;
    const bool active = j < j_end;
    float a[8 * WPL];
#pragma unroll
    for (int i = 0; i < WPL; ++i) {
      const half8_t h = __builtin_bit_cast(
          half8_t, __builtin_amdgcn_raw_buffer_load_b128(rw, (uint32_t)(r * kw + j + i) * 16, 0, 0));
#pragma unroll
      for (int c = 0; c < 8; ++c) a[8 * i + c] = (float)h[c];
    }
    float mn = 0.0f, mx;
    if constexpr (ZP) {
      mn = mx = a[0];
#pragma unroll
      for (int c = 1; c < 8 * WPL; ++c) {
        mn = fminf(mn, a[c]);
        mx = fmaxf(mx, a[c]);
      }
      mn = group_all<GW>(mn, MinOp());
      mx = group_all<GW>(mx, MaxOp());
    } else {
      mx = fabsf(a[0]);
#pragma unroll
      for (int c = 1; c < 8 * WPL; ++c) mx = fmaxf(mx, fabsf(a[c]));
      mx = group_all<GW>(mx, MaxOp());
    }
    const int grp = j / (WPL * GW);
    for (int c = pos; c < count; c += GW) {
      const float ratio = ratios.v[c];
      float lo, hi, cmn = 0.0f, cmx;
      // (fp32 products kept explicit: the bounds are rounded to fp16 below)
      if constexpr (ZP) {
        lo = fp32_product(ratio, mn);
        hi = fp32_product(ratio, mx);
        cmn = (float)(_Float16)fminf(fmaxf(mn, lo), hi);
        cmx = (float)(_Float16)fminf(fmaxf(mx, lo), hi);
      } else {
        hi = fp32_product(ratio, mx);
        lo = -hi;
        cmx = (float)(_Float16)fminf(mx, hi);
      }
      float s, zf;
      _Float16 s16;
      scale_zero_of_extremes<ZP>(cmn, cmx, s16, s, zf);
      if (active)
        gp[((size_t)c * G + grp) * N + n] =
            u32x2{(uint32_t)__builtin_bit_cast(uint16_t, s16) | ((uint32_t)zf << 16),
                  (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo) |
                      ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16)};
    }
  }
}

// The clipping ratio of each weight group (n, j): the error of the group under
// ratio c is the sum, in a fixed order (fp64), of the per-tile partials
// part[c][tm][q][j][n] (tile rows tm, quarter q of a tile's rows), and the
// group keeps the first ratio with the smallest error.  One thread per four
// groups of consecutive rows n (N is a multiple of 8), so each partial read is
// one 16-byte load and the reads of a wave coalesce; the parts of a ratio are
// loaded together (the loop is unrolled) before their sum.
__global__ __launch_bounds__(256) void clip_choose_kernel(const float4_t* __restrict__ part, int parts, int G, int N,
                                                          int count, int32_t* __restrict__ choice) {
  const int N4 = N >> 2;
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)G * N4) return;
  const int grp = (int)(idx / N4), n4 = (int)(idx - (size_t)grp * N4);
  double best_v[4] = {__builtin_huge_val(), __builtin_huge_val(), __builtin_huge_val(), __builtin_huge_val()};
  int best[4] = {0, 0, 0, 0};
  for (int c = 0; c < count; ++c) {
    double v[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll 4
    for (int p = 0; p < parts; ++p) {
      const float4_t x = part[(((size_t)c * parts + p) * G + grp) * N4 + n4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] += (double)x[i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (v[i] < best_v[i]) {
        best_v[i] = v[i];
        best[i] = c;
      }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) choice[(size_t)(4 * n4 + i) * G + grp] = best[i];
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

// K slices as in launch_pack_zp, to about 4096 blocks (every block loops over
// all candidates).
template <bool ZP>
hipError_t launch_scale_group_params_zp(const void* w, const float* s, int count, int N, int K, int group_size,
                                        void* gp, hipStream_t stream) {
  constexpr int kTargetBlocks = 4096, kRingWords = 32 * kPackWords;
  const int kw = K >> 3, bands = (N + 8 * kParamRows - 1) / (8 * kParamRows);
  const int rings = (kw + kRingWords - 1) / kRingWords;
  int slices = (kTargetBlocks + bands - 1) / bands;
  if (slices > rings) slices = rings;
  if (slices < 1) slices = 1;
  const int chunk = ((rings + slices - 1) / slices) * kRingWords;
  const dim3 grid(bands, (kw + chunk - 1) / chunk), block(kPackThreads);
  const u32x4* wv = static_cast<const u32x4*>(w);
  uint32_t* g = static_cast<uint32_t*>(gp);
  switch (group_size) {
    case 32: hipLaunchKernelGGL((scale_group_params_kernel<4 / kPackWords, ZP>), grid, block, 0, stream, wv, s, count, N, K, chunk, g); break;
    case 64: hipLaunchKernelGGL((scale_group_params_kernel<8 / kPackWords, ZP>), grid, block, 0, stream, wv, s, count, N, K, chunk, g); break;
    case 128: hipLaunchKernelGGL((scale_group_params_kernel<16 / kPackWords, ZP>), grid, block, 0, stream, wv, s, count, N, K, chunk, g); break;
    case 256: hipLaunchKernelGGL((scale_group_params_kernel<32 / kPackWords, ZP>), grid, block, 0, stream, wv, s, count, N, K, chunk, g); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool ZP>
hipError_t launch_clip_zp(const void* w, const ClipRatios& ratios, int count, int N, int K, int group_size, void* gp,
                          const int32_t* choice, void* w_out, bool apply, hipStream_t stream) {
  const u32x4* wv = static_cast<const u32x4*>(w);
  const dim3 block(kPackThreads);
  // parameters: K slices as in launch_pack_zp, to about 4096 blocks
  constexpr int kRingWords = 32 * kPackWords;
  const int kw = K >> 3, octets = N / 8;
  const int rings = (kw + kRingWords - 1) / kRingWords;
  int slices = (4096 + octets - 1) / octets;
  if (slices > rings) slices = rings;
  if (slices < 1) slices = 1;
  const int chunk = ((rings + slices - 1) / slices) * kRingWords;
  const dim3 pgrid(octets, (kw + chunk - 1) / chunk);
#define AWQ_CLIP_CASE(G_, GW_)                                                                                   \
  case G_:                                                                                                     \
    if (!apply)                                                                                                \
      hipLaunchKernelGGL((clip_group_params_kernel<GW_ / kPackWords, ZP>), pgrid, block, 0, stream, wv, ratios,  \
                         count, N, K, chunk, static_cast<u32x2*>(gp));                                         \
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

hipError_t launch_clip_group_params(const void* w, const ClipRatios& ratios, int count, int N, int K, int group_size,
                                    bool zero_point, void* gp, hipStream_t stream) {
  return zero_point ? launch_clip_zp<true>(w, ratios, count, N, K, group_size, gp, nullptr, nullptr, false, stream)
                    : launch_clip_zp<false>(w, ratios, count, N, K, group_size, gp, nullptr, nullptr, false, stream);
}

hipError_t launch_clip_apply(const void* w, const float* part, int parts, const ClipRatios& ratios, int count, int N,
                             int K, int group_size, bool zero_point, void* w_out, int32_t* choice, hipStream_t stream) {
  const int G = K / group_size;
  const size_t groups = (size_t)G * N;
  hipLaunchKernelGGL(clip_choose_kernel, dim3((unsigned)((groups / 4 + 255) / 256)), dim3(256), 0, stream,
                     reinterpret_cast<const float4_t*>(part), parts, G, N, count, choice);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return zero_point ? launch_clip_zp<true>(w, ratios, count, N, K, group_size, nullptr, choice, w_out, true, stream)
                    : launch_clip_zp<false>(w, ratios, count, N, K, group_size, nullptr, choice, w_out, true, stream);
}

hipError_t launch_scale_group_params(const void* w, const float* s, int count, int N, int K, int group_size,
                                     bool zero_point, void* gp, hipStream_t stream) {
  return zero_point ? launch_scale_group_params_zp<true>(w, s, count, N, K, group_size, gp, stream)
                    : launch_scale_group_params_zp<false>(w, s, count, N, K, group_size, gp, stream);
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
