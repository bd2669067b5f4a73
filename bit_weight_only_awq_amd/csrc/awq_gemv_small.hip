// Few-token W4A16 layer (awq_gemv / awq_gemm with 2-8 tokens):
//   y[m][n] = sum_k x[m][k] * (q[n,k] - z) * s,  2 <= M <= 8.
//
// The GEMVFast idea of "AI-Research-SKILLs AWQ 高级使用指南" (section WQLinear
// 内核全景: the fastest few-token decoding), built for gfx950.  Every packed
// weight byte is used once per call, so the kernel is a stream over HBM.
//
// gemv_small_kernel (M = 2..8) keeps the single-token GEMV's load pattern
// (every load of a lane issued up front, one memory round trip per wave),
// with the products on the matrix cores.  v_mfma_f32_4x4x4_16b_f16 runs 16 independent 4 x 4 x 4
// products per wave; here its 16 blocks are 16 different 32-channel slices of
// the same rows, so lane (b, q) = (lane / 4, lane % 4) holds A = 4 channels of
// weight row q and B = the same 4 channels of token q.  A 128-bit load of a
// lane (32 channels of one row) feeds 8 MFMAs, and one activation load feeds
// four weight rows, as in the single-token kernel; a workgroup owns 16 rows
// (each lane 4 of them) so that activations are read once per 16 rows.  The
// decoded weights enter the MFMA as exact small integers q - z; the slice's
// fp32 sum is multiplied by the row's group scale once.  The 16 slices are
// summed by the same lane-swap reduction, then the waves through LDS.
#include "awq_device.hpp"
#include "awq_launch.hpp"

namespace awq {
namespace {

int log2_group(int g) { return g == 32 ? 5 : g == 64 ? 6 : g == 128 ? 7 : 8; }

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
constexpr uint32_t kOutOfRange = 0x80000000u;  // a buffer offset past every resource: loads return 0
constexpr int kSmallRows = 16;                 // output rows per workgroup

// One workgroup: 16 output rows, all M <= 4 TS tokens, all of K.  Sub-chunk c
// (512 channels) is 16 slices of 32 channels, slice b at channels 512 c + 32 b;
// wave w takes sub-chunks (round * nw + w) * S + s.  Lane (b, q) loads, per
// sub-chunk, 32 channels of rows 4 r + q (r < 4), the two row octets' scales
// and zero-point words of its slice's group, and the same 32 channels of
// tokens 4 t + q (t < TS); MFMA (word, half) then multiplies 4 channels.  The
// accumulator of lane (b, q) for row quad r and token set t holds, in register
// i, row 4 r + i and token 4 t + q (the 4x4x4 output layout).
// MULTI: K takes more than one round.  A single round is a separate
// instance: with the loop in place the compiler stages the loads less
// aggressively and a Llama-7B layer took ~1 us (10-20%) longer.
template <int TS, int S, int MAXW, bool ZP, bool MULTI>
__global__ __launch_bounds__(MAXW * 64) void gemv_small_kernel(
    const _Float16* __restrict__ X, int M, const uint32_t* __restrict__ qweight, const uint16_t* __restrict__ scales,
    const uint32_t* __restrict__ qzeros, _Float16* __restrict__ y, int N, int K, int gshift, int rounds) {
  constexpr int RS = kSmallRows / 4, OCT = kSmallRows / 8;
  __shared__ float red[MAXW][kSmallRows][TS * 4];
  const int nw = blockDim.x >> 6;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int b = lane >> 2, q = lane & 3;
  const int n0 = blockIdx.x * kSmallRows;
  const int rows_n = min(kSmallRows, N - n0);  // a multiple of 8
  const int G = K >> gshift;
  const DecodeConsts kc;
  // rows past rows_n (and their octet) lie past the resources and read as 0
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(qweight + (size_t)n0 * (K >> 3), (uint32_t)rows_n * (K >> 1));
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(scales + scale_index(n0, 0, G), (uint32_t)(rows_n >> 3) * G * 16);
  const __amdgpu_buffer_rsrc_t rz = make_rsrc(ZP ? qzeros + zero_word_index(n0, 0, G) : qzeros,
                                              ZP ? (uint32_t)(rows_n >> 3) * G * 4 : 0u);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(X, (uint32_t)M * K * 2);  // tokens past M read as 0

  float4_t acc[RS][TS];
#pragma unroll
  for (int r = 0; r < RS; ++r)
#pragma unroll
    for (int ts = 0; ts < TS; ++ts) acc[r][ts] = float4_t{0.f, 0.f, 0.f, 0.f};

  for (int round = 0; round < (MULTI ? rounds : 1); ++round) {
    u32x4 wv[S][RS];
    u32x4 sv[S][OCT];
    uint32_t zv[S][OCT];
    u32x4 xv[S][TS][4];
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int k0 = ((round * nw + wave) * S + s) * 512 + 32 * b;
      const bool kin = k0 < K;  // K is a multiple of 32: a slice is wholly in or out
      const int grp = k0 >> gshift;
#pragma unroll
      for (int r = 0; r < RS; ++r)
        wv[s][r] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                       rw, kin ? (uint32_t)(4 * r + q) * (K >> 1) + (k0 >> 1) : kOutOfRange, 0, 0));
#pragma unroll
      for (int o = 0; o < OCT; ++o) {
        sv[s][o] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 rs, kin ? (uint32_t)((o * G + grp) * 16) : kOutOfRange, 0, 0));
        zv[s][o] = ZP ? __builtin_amdgcn_raw_buffer_load_b32(rz, kin ? (uint32_t)((o * G + grp) * 4) : kOutOfRange,
                                                             0, 0)
                      : 0x88888888u;
      }
#pragma unroll
      for (int ts = 0; ts < TS; ++ts) {
        const uint32_t xo = kin ? ((uint32_t)(4 * ts + q) * K + k0) * 2 : kOutOfRange;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          xv[s][ts][e] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, xo, e * 16, 0));
      }
    }
    // every load of the round is in flight before any decoding
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < S; ++s) {
#pragma unroll
      for (int r = 0; r < RS; ++r) {
        const ZeroBias zb = zero_bias((zv[s][r >> 1] >> (4 * (4 * (r & 1) + q))) & 15u);
        float4_t tmp[TS];
#pragma unroll
        for (int ts = 0; ts < TS; ++ts) tmp[ts] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          half2_t d[4];
          decode_pairs(wv[s][r][w], zb, kc, d);
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            // channels 8 w + 4 h .. + 3 of the slice, in order, for A and B alike
            half4_t a;
            a[0] = d[2 * h][0];
            a[1] = d[2 * h][1];
            a[2] = d[2 * h + 1][0];
            a[3] = d[2 * h + 1][1];
#pragma unroll
            for (int ts = 0; ts < TS; ++ts) {
              const half2_t x0 = as_half2(xv[s][ts][w][2 * h]), x1 = as_half2(xv[s][ts][w][2 * h + 1]);
              half4_t bx;
              bx[0] = x0[0];
              bx[1] = x0[1];
              bx[2] = x1[0];
              bx[3] = x1[1];
              tmp[ts] = __builtin_amdgcn_mfma_f32_4x4x4f16(a, bx, tmp[ts], 0, 0, 0);
            }
          }
        }
        // register i of tmp is row 4 r + i: its scale for this slice's group
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int pos = 4 * (r & 1) + i;  // place of row 4 r + i in octet r / 2
          const uint32_t bits = (sv[s][r >> 1][pos >> 1] >> (16 * (pos & 1))) & 0xFFFFu;
          const float sc = (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
#pragma unroll
          for (int ts = 0; ts < TS; ++ts) acc[r][ts][i] += tmp[ts][i] * sc;
        }
      }
    }
  }

  // Sum over the 16 slices (lane bits 2-5): the two lane-half swaps leave, in
  // 16-lane group g, register (0, 2, 1, 3)[g] summed over bits 4 and 5; two
  // DPP rotations within the 16 lanes add bits 3 and 2.  Lane 16 g + q then
  // holds the wave's total of that register for token q.
#pragma unroll
  for (int r = 0; r < RS; ++r)
#pragma unroll
    for (int ts = 0; ts < TS; ++ts) {
      const float a01 = swap_sum32(acc[r][ts][0], acc[r][ts][1]);
      const float a23 = swap_sum32(acc[r][ts][2], acc[r][ts][3]);
      float v = swap_sum16(a01, a23);
      v += row_rotate<0x128>(v);  // row_ror:8
      v += row_rotate<0x124>(v);  // row_ror:4
      const int g = lane >> 4;
      const int reg = g == 0 ? 0 : g == 1 ? 2 : g == 2 ? 1 : 3;
      if ((lane & 12) == 0) red[wave][4 * r + reg][4 * ts + q] = v;
    }
  __syncthreads();
  for (int i = t; i < kSmallRows * TS * 4; i += nw * 64) {
    const int row = i / (TS * 4), m = i - row * (TS * 4);
    float sum = red[0][row][m];
    for (int w = 1; w < nw; ++w) sum += red[w][row][m];
    if (m < M && row < rows_n) y[(size_t)m * N + n0 + row] = (_Float16)sum;
  }
}

// Launch shape of the few-token kernel: S sub-chunks per wave, nw waves, and
// rounds of nw * S sub-chunks until K is covered.  Up to 4 tokens: S = 2 and
// up to 12 waves (124 VGPRs); 5-8 tokens hold twice the activations, so at
// most 8 waves (a 256-register budget) with S = 2, or 3 once K needs more
// than 16 sub-chunks.  Measured on the Llama-7B shapes at 2-8 tokens: 4
// waves of two sub-chunks on K = 4096, 11 on K = 11008 (one sub-chunk per
// wave, or three or four per wave on fewer waves, are 1-4% slower).
struct SmallPlan {
  int s, nw, rounds;
};
SmallPlan plan_small(int M, int K) {
  const int nsub = (K + 511) / 512;
  const int maxw = M <= 4 ? 12 : 8;
  SmallPlan p;
  p.s = M <= 4 || nsub <= 2 * maxw ? 2 : 3;
  p.nw = (nsub + p.s - 1) / p.s;
  if (p.nw > maxw) p.nw = maxw;
  p.rounds = (nsub + p.nw * p.s - 1) / (p.nw * p.s);
  return p;
}

template <int TS, int S, int MAXW, bool ZP>
hipError_t launch_small_ts(const void* x, int M, const uint32_t* qweight, const uint16_t* scales,
                           const uint32_t* qzeros, void* y, int N, int K, int gs, const SmallPlan& p,
                           hipStream_t stream) {
  if (p.s != S || p.nw > MAXW) return hipErrorInvalidValue;  // the plan must match the instance
  const dim3 grid((N + kSmallRows - 1) / kSmallRows), block(p.nw * 64);
  const _Float16* xv = static_cast<const _Float16*>(x);
  _Float16* yv = static_cast<_Float16*>(y);
  if (p.rounds == 1)
    hipLaunchKernelGGL((gemv_small_kernel<TS, S, MAXW, ZP, false>), grid, block, 0, stream, xv, M, qweight, scales,
                       qzeros, yv, N, K, gs, p.rounds);
  else
    hipLaunchKernelGGL((gemv_small_kernel<TS, S, MAXW, ZP, true>), grid, block, 0, stream, xv, M, qweight, scales,
                       qzeros, yv, N, K, gs, p.rounds);
  return hipGetLastError();
}

template <bool ZP>
hipError_t launch_small(const void* x, int M, const uint32_t* qweight, const uint16_t* scales,
                        const uint32_t* qzeros, void* y, int N, int K, int gs, hipStream_t stream) {
  const SmallPlan p = plan_small(M, K);
  if (M <= 4) return launch_small_ts<1, 2, 12, ZP>(x, M, qweight, scales, qzeros, y, N, K, gs, p, stream);
  return p.s == 2 ? launch_small_ts<2, 2, 8, ZP>(x, M, qweight, scales, qzeros, y, N, K, gs, p, stream)
                  : launch_small_ts<2, 3, 8, ZP>(x, M, qweight, scales, qzeros, y, N, K, gs, p, stream);
}

}  // namespace

hipError_t launch_gemv_small(const void* x, const uint32_t* qweight, const void* scales, const uint32_t* qzeros,
                             void* y, int M, int N, int K, int group_size, bool zero_point, hipStream_t stream) {
  const uint16_t* sc = static_cast<const uint16_t*>(scales);
  const int gs = log2_group(group_size);
  return zero_point ? launch_small<true>(x, M, qweight, sc, qzeros, y, N, K, gs, stream)
                    : launch_small<false>(x, M, qweight, sc, qzeros, y, N, K, gs, stream);
}

}  // namespace awq
