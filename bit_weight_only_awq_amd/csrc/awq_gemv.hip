// Single-token W4A16 layer (awq_gemv): y[n] = sum_k x[k] * (q[n,k] - z) * s.
//
// The GEMV variant of the quantized linear layer ("AI-Research-SKILLs AWQ 高级
// 使用指南", section WQLinear 内核全景: single-token generation, batch 1).  At
// batch 1 every packed weight byte is used exactly once, so the kernel is a
// stream over HBM.  Design for gfx950:
//   * one workgroup per quad of output rows; a lane owns 32-channel chunks of
//     all 4 rows and loads them as 128-bit words, so every weight load of a
//     wave reads 1 KiB of one row contiguously;
//   * the 4 rows share the lane's activations; the quad's 4 scales arrive in
//     one 64-bit load and its zero points in one 32-bit load, and with the
//     row-octet-major scale/zero layout consecutive lanes read consecutive
//     groups, so these side loads stay coalesced;
//   * side loads are issued before the weight loads, so row 0 is decoded as
//     soon as its weights land while rows 1-3 are still in flight;
//   * decoding is exact bit arithmetic (q - z as small fp16 integers) followed
//     by v_dot2_f32_f16 against the fp16 activations; the group scale
//     multiplies the fp32 chunk sum once, so no decoded weight is rounded;
//   * row sums are reduced across the wave in registers (two lane-swap
//     exchanges that leave one row per 16-lane group, then DPP row rotations),
//     then across waves through LDS in a fixed order: bit-reproducible results.
#include "awq_device.hpp"
#include "awq_launch.hpp"

namespace awq {
namespace {

constexpr int kRows = 4;

template <int NW, bool ZP>
__global__ __launch_bounds__(NW * 64) void gemv_kernel(const u32x4* __restrict__ x, const u32x4* __restrict__ qweight,
                                                       const uint16_t* __restrict__ scales,
                                                       const uint32_t* __restrict__ qzeros,
                                                       _Float16* __restrict__ y, int N, int K, int gshift) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  __shared__ float red[NW][kRows];
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int n0 = blockIdx.x * kRows;
  const int chunks = K >> 5;                // 32-channel chunks per row
  const int G = K >> gshift;
  const size_t row_u4 = (size_t)(K >> 5);   // a row is K/2 bytes = K/32 128-bit words
  const int sub = n0 & 7;                   // 0 or 4: position of the quad in its octet

  const u32x4* wrow = qweight + (size_t)n0 * row_u4;
  const uint16_t* squad = scales + scale_index(n0, 0, G);
  const uint32_t* zoct = qzeros + (ZP ? zero_word_index(n0, 0, G) : 0);
  const DecodeConsts kc;

  float acc[kRows];
#pragma unroll
  for (int r = 0; r < kRows; ++r) acc[r] = 0.0f;

  for (int c = t; c < chunks; c += NW * 64) {
    const int grp = (c << 5) >> gshift;
    const u32x2 sv = *reinterpret_cast<const u32x2*>(squad + (size_t)grp * 8);
    const uint32_t zw = ZP ? (zoct[grp] >> (4 * sub)) : 0x88888888u;
    u32x4 xv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) xv[i] = x[(size_t)c * 4 + i];
    u32x4 wv[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r) wv[r] = wrow[(size_t)r * row_u4 + c];
    // every load of the chunk is issued before any decoding: left alone, the
    // scheduler splits them into rounds around the dot products in the
    // variant without zero points (two to three load latencies per chunk)
    __builtin_amdgcn_sched_barrier(0);

#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      const ZeroBias b = zero_bias((zw >> (4 * r)) & 15u);
      float part0 = 0.0f, part1 = 0.0f;
#pragma unroll
      for (int wi = 0; wi < 4; ++wi) {
        half2_t d[4];
        decode_pairs(wv[r][wi], b, kc, d);
        part0 = __builtin_amdgcn_fdot2(d[0], as_half2(xv[wi][0]), part0, false);
        part1 = __builtin_amdgcn_fdot2(d[1], as_half2(xv[wi][1]), part1, false);
        part0 = __builtin_amdgcn_fdot2(d[2], as_half2(xv[wi][2]), part0, false);
        part1 = __builtin_amdgcn_fdot2(d[3], as_half2(xv[wi][3]), part1, false);
      }
      const uint32_t sbits = (sv[r >> 1] >> (16 * (r & 1))) & 0xFFFFu;
      const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)sbits);
      acc[r] += (part0 + part1) * s;
    }
  }

  const float total = wave_reduce_quad_rows(acc);
  constexpr int kLanesPerRow = 64 / kRows;
  if (NW == 1) {
    if ((lane % kLanesPerRow) == 0) y[n0 + lane / kLanesPerRow] = (_Float16)total;
    return;
  }
  if ((lane % kLanesPerRow) == 0) red[wave][lane / kLanesPerRow] = total;
  __syncthreads();
  if (t < kRows) {
    float sum = red[0][t];
#pragma unroll
    for (int w = 1; w < NW; ++w) sum += red[w][t];
    y[n0 + t] = (_Float16)sum;
  }
}

int log2_group(int g) { return g == 32 ? 5 : g == 64 ? 6 : g == 128 ? 7 : 8; }

template <bool ZP>
hipError_t launch_zp(const void* x, const uint32_t* qweight, const void* scales, const uint32_t* qzeros, void* y,
                     int N, int K, int group_size, hipStream_t stream) {
  // one 32-channel chunk per lane where K allows it (K = 4096: 2 waves; K = 11008: 6 waves)
  const int chunks = K >> 5;
  int nw = (chunks + 63) / 64;
  if (nw > 8) nw = 8;
  const dim3 grid(N / kRows);
  const u32x4* xv = static_cast<const u32x4*>(x);
  const u32x4* wv = reinterpret_cast<const u32x4*>(qweight);
  const uint16_t* sc = static_cast<const uint16_t*>(scales);
  _Float16* yv = static_cast<_Float16*>(y);
  const int gs = log2_group(group_size);
#define AWQ_GEMV_CASE(W)                                                                                  \
  case W:                                                                                                 \
    hipLaunchKernelGGL((gemv_kernel<W, ZP>), grid, dim3(W * 64), 0, stream, xv, wv, sc, qzeros, yv, N, K, gs); \
    break;
  switch (nw) {
    AWQ_GEMV_CASE(1)
    AWQ_GEMV_CASE(2)
    AWQ_GEMV_CASE(3)
    AWQ_GEMV_CASE(4)
    AWQ_GEMV_CASE(5)
    AWQ_GEMV_CASE(6)
    AWQ_GEMV_CASE(7)
    AWQ_GEMV_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef AWQ_GEMV_CASE
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv(const void* x, const uint32_t* qweight, const void* scales, const uint32_t* qzeros, void* y,
                       int N, int K, int group_size, bool zero_point, hipStream_t stream) {
  return zero_point ? launch_zp<true>(x, qweight, scales, qzeros, y, N, K, group_size, stream)
                    : launch_zp<false>(x, qweight, scales, qzeros, y, N, K, group_size, stream);
}

}  // namespace awq
