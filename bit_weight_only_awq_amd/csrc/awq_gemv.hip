// Single-token W4A16 layer (awq_gemv): y[n] = sum_k x[k] * (q[n,k] - z) * s.
//
// The GEMV variant of the quantized linear layer ("AI-Research-SKILLs AWQ 高级
// 使用指南", section WQLinear 内核全景: single-token generation, batch 1).  At
// batch 1 every packed weight byte is used exactly once, so the kernel is a
// stream over HBM.  Design for gfx950:
//   * one workgroup per octet of output rows; each lane owns 32-channel chunks
//     of all 8 rows and loads them as 128-bit words, so every load instruction
//     of a wave reads 1 KiB of one row contiguously;
//   * the 8 rows share the lane's activations (loaded once per chunk), the
//     octet's 8 scales arrive in one 128-bit load and its 8 zero points in one
//     32-bit load (scales are [G][N], zeros [G][N/8]);
//   * decoding is exact bit arithmetic (q - z as fp16 integers) followed by
//     v_dot2_f32_f16 against the fp16 activations; the group scale multiplies
//     the fp32 chunk sum once, so no decoded weight is ever rounded;
//   * the 8 per-lane row sums are reduced across the wave with a transposing
//     butterfly (each step halves the rows a lane carries: 4+2+1+3 shuffles
//     instead of 8x6), then across waves through LDS in a fixed order, so the
//     result is bit-reproducible.
#include "awq_device.hpp"
#include "awq_launch.hpp"

namespace awq {
namespace {

template <int NW, bool ZP>
__global__ __launch_bounds__(NW * 64) void gemv_kernel(const u32x4* __restrict__ x, const u32x4* __restrict__ qweight,
                                                       const uint16_t* __restrict__ scales,
                                                       const uint32_t* __restrict__ qzeros,
                                                       _Float16* __restrict__ y, int N, int K, int gshift) {
  __shared__ float red[NW][8];
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int n0 = blockIdx.x * 8;
  const int chunks = K >> 5;       // 32-channel chunks per row
  const size_t row_u4 = (size_t)(K >> 5);  // a row is K/2 bytes = K/32 128-bit words

  const u32x4* wrow = qweight + (size_t)n0 * row_u4;
  float acc[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) acc[r] = 0.0f;

  for (int c = t; c < chunks; c += NW * 64) {
    u32x4 wv[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) wv[r] = wrow[(size_t)r * row_u4 + c];
    u32x4 xv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) xv[i] = x[(size_t)c * 4 + i];
    const int grp = (c << 5) >> gshift;
    const u32x4 sv = *reinterpret_cast<const u32x4*>(scales + (size_t)grp * N + n0);
    const uint32_t zw = ZP ? qzeros[(size_t)grp * (N >> 3) + (n0 >> 3)] : 0x88888888u;

    half2_t xp[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int p = 0; p < 4; ++p) xp[i * 4 + p] = as_half2(xv[i][p]);
    }

#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const ZeroBias b = zero_bias((zw >> (4 * r)) & 15u);
      float part0 = 0.0f, part1 = 0.0f;
#pragma unroll
      for (int wi = 0; wi < 4; ++wi) {
        half2_t d[4];
        decode_pairs(wv[r][wi], b, d);
        part0 = __builtin_amdgcn_fdot2(d[0], xp[wi * 4 + 0], part0, false);
        part1 = __builtin_amdgcn_fdot2(d[1], xp[wi * 4 + 1], part1, false);
        part0 = __builtin_amdgcn_fdot2(d[2], xp[wi * 4 + 2], part0, false);
        part1 = __builtin_amdgcn_fdot2(d[3], xp[wi * 4 + 3], part1, false);
      }
      const uint32_t sbits = (sv[r >> 1] >> (16 * (r & 1))) & 0xFFFFu;
      const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)sbits);
      acc[r] += (part0 + part1) * s;
    }
  }

  // Transposing butterfly: after the xor-32/16/8 steps lane l carries the
  // partial sum of row (l >> 3) over its 8-lane group; xor-4/2/1 finish it.
  float a4[4], a2[2], a1;
  {
    const bool hi = lane & 32;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float give = hi ? acc[i] : acc[i + 4];
      const float keep = hi ? acc[i + 4] : acc[i];
      a4[i] = keep + __shfl_xor(give, 32);
    }
  }
  {
    const bool hi = lane & 16;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const float give = hi ? a4[i] : a4[i + 2];
      const float keep = hi ? a4[i + 2] : a4[i];
      a2[i] = keep + __shfl_xor(give, 16);
    }
  }
  {
    const bool hi = lane & 8;
    const float give = hi ? a2[0] : a2[1];
    const float keep = hi ? a2[1] : a2[0];
    a1 = keep + __shfl_xor(give, 8);
  }
  a1 += __shfl_xor(a1, 4);
  a1 += __shfl_xor(a1, 2);
  a1 += __shfl_xor(a1, 1);

  if (NW == 1) {
    if ((lane & 7) == 0) y[n0 + (lane >> 3)] = (_Float16)a1;
    return;
  }
  if ((lane & 7) == 0) red[wave][lane >> 3] = a1;
  __syncthreads();
  if (t < 8) {
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
  const int chunks = K >> 5;
  int nw = (chunks + 63) / 64;
  if (nw > 8) nw = 8;
  const dim3 grid(N / 8);
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
