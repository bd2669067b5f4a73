// Single-token W4A16 layer (awq_gemv): y[n] = sum_k x[k] * (q[n,k] - z) * s.
//
// The GEMV variant of the quantized linear layer ("AI-Research-SKILLs AWQ 高级
// 使用指南", section WQLinear 内核全景: single-token generation, batch 1).  At
// batch 1 every packed weight byte is used exactly once, so the kernel is a
// stream over HBM.  Design for gfx950:
//   * NW waves per quad (or, on layers large enough to fill the chip with half
//     as many workgroups, per octet) of output rows, two quads per workgroup
//     (4% faster on the 4096 x 4096 layers than one: fewer, fuller
//     workgroups, the quads' activation reads served by one compute unit's
//     L1); a lane owns
//     32-channel chunks of all its rows and loads them as 128-bit words, so
//     every weight load of a wave reads 1 KiB of one row contiguously;
//   * the rows share the lane's activations; their scales arrive in one 64-bit
//     (quad) or 128-bit (octet) load and their zero points in one 32-bit
//     load, and with the row-octet-major scale/zero layout consecutive lanes
//     read consecutive groups, so these side loads stay coalesced;
//   * side loads are issued before the weight loads, so row 0 is decoded as
//     soon as its weights land while rows 1-3 are still in flight;
//   * decoding is exact bit arithmetic (q - z as small fp16 integers) followed
//     by v_dot2_f32_f16 against the fp16 activations; the group scale
//     multiplies the fp32 chunk sum once, so no decoded weight is rounded;
//   * row sums are reduced across the wave in registers (lane-swap exchanges
//     that leave one row per 16- or 8-lane group, then DPP lane rotations),
//     then across waves through LDS in a fixed order: bit-reproducible results;
//   * workgroups are laid out so that each line of y is written from one
//     XCD's L2.
#include "awq_device.hpp"
#include "awq_launch.hpp"

namespace awq {
namespace {

// QPW row groups (quads or octets) per workgroup, NW waves each.
template <int NW, bool ZP, int ROWS, int QPW>
__global__ __launch_bounds__(NW * QPW * 64) void gemv_kernel(const u32x4* __restrict__ x,
                                                             const u32x4* __restrict__ qweight,
                                                             const uint16_t* __restrict__ scales,
                                                             const uint32_t* __restrict__ qzeros,
                                                             _Float16* __restrict__ y, int N, int K, int gshift) {
  static_assert(ROWS == 4 || ROWS == 8, "row quads or octets");
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  __shared__ float red[QPW][NW][ROWS];
  // (the wave index is uniform: readfirstlane keeps it, the row group and
  // the row addresses derived from it in scalar registers)
  const int lane = threadIdx.x & 63, wave_all = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int part = QPW == 1 ? 0 : wave_all / NW, wave = wave_all - part * NW;  // row group of the wave, wave within it
  const int t = wave * 64 + lane;                               // thread within the row group
  // The hardware deals workgroups to the 8 XCDs round robin, which would spread the 8 workgroups
  // of 8 rows (two quads or an octet) that write one 128-byte line of y (64 rows) over all 8 L2s.
  // Within each group of 64 workgroups the row groups are transposed: the group's workgroups on
  // XCD j (j, j + 8, ..., j + 56) take its row groups 8 j .. 8 j + 7, one line of y, so each line
  // is written from one L2 (the 7B decode step 2.5% faster) while the XCDs still sweep
  // neighbouring rows together.  A ragged last group keeps the dealt order.
  const int bid = blockIdx.x < (gridDim.x & ~63u)
                      ? (int)((blockIdx.x & ~63u) | ((blockIdx.x & 7u) << 3) | ((blockIdx.x >> 3) & 7u))
                      : (int)blockIdx.x;
  const int n0 = (bid * QPW + part) * ROWS;
  const int chunks = K >> 5;                // 32-channel chunks per row
  const int G = K >> gshift;
  const size_t row_u4 = (size_t)(K >> 5);   // a row is K/2 bytes = K/32 128-bit words
  const int sub = n0 & 7;                   // quads: 0 or 4, the position of the quad in its octet

  const u32x4* wrow = qweight + (size_t)n0 * row_u4;
  const uint16_t* sq = scales + scale_index(n0, 0, G);
  const uint32_t* zoct = qzeros + (ZP ? zero_word_index(n0, 0, G) : 0);
  const DecodeConsts kc;

  float acc[ROWS];
#pragma unroll
  for (int r = 0; r < ROWS; ++r) acc[r] = 0.0f;

  for (int c = t; c < chunks; c += NW * 64) {
    const int grp = (c << 5) >> gshift;
    // the rows' scales: 8 (16 bytes, an octet) or 4 (8 bytes) consecutive fp16
    uint32_t sw[ROWS / 2];
    if constexpr (ROWS == 8) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(sq + (size_t)grp * 8);
#pragma unroll
      for (int i = 0; i < 4; ++i) sw[i] = v[i];
    } else {
      const u32x2 v = *reinterpret_cast<const u32x2*>(sq + (size_t)grp * 8);
      sw[0] = v[0];
      sw[1] = v[1];
    }
    const uint32_t zw = ZP ? (zoct[grp] >> (ROWS == 8 ? 0 : 4 * sub)) : 0x88888888u;
    u32x4 xv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) xv[i] = x[(size_t)c * 4 + i];
    u32x4 wv[ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) wv[r] = wrow[(size_t)r * row_u4 + c];
    // every load of the chunk is issued before any decoding: left alone, the
    // scheduler splits them into rounds around the dot products in the
    // variant without zero points (two to three load latencies per chunk)
    __builtin_amdgcn_sched_barrier(0);

#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
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
      const uint32_t sbits = (sw[r >> 1] >> (16 * (r & 1))) & 0xFFFFu;
      const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)sbits);
      acc[r] += (part0 + part1) * s;
    }
  }

  float total;
  int row;  // the row whose total this lane holds
  if constexpr (ROWS == 8) {
    total = wave_reduce_oct_rows(acc);
    row = (lane >> 4) + 4 * ((lane >> 3) & 1);
  } else {
    total = wave_reduce_quad_rows(acc);
    row = lane >> 4;
  }
  // quads: lanes 0, 16, 32, 48; octets: every eighth lane
  const bool writer = (lane % (64 / ROWS)) == 0;
  if (NW == 1) {
    if (writer) y[n0 + row] = (_Float16)total;
    return;
  }
  if (writer) red[part][wave][row] = total;
  __syncthreads();
  if (threadIdx.x < QPW * ROWS) {
    const int p = threadIdx.x / ROWS, r = threadIdx.x - p * ROWS;
    float sum = red[p][0][r];
#pragma unroll
    for (int w = 1; w < NW; ++w) sum += red[p][w][r];
    y[(bid * QPW + p) * ROWS + r] = (_Float16)sum;
  }
}

int log2_group(int g) { return g == 32 ? 5 : g == 64 ? 6 : g == 128 ? 7 : 8; }

// Waves per workgroup: one 32-channel chunk per lane where K allows it
// (K = 4096: 2 waves; K = 11008: 6); past 512 chunks 12 waves, so that on
// K = 28672 (896 chunks) most lanes take one chunk instead of two (2% faster
// than 8 waves; 7 or 14 waves are slower).
int gemv_waves(int K) {
  const int chunks = K >> 5;
  return chunks > 8 * 64 ? 12 : (chunks + 63) / 64;
}

bool gemv_uses_octets(int N, int K) { return (long)(N / 8) * gemv_waves(K) >= 32 * 256; }

// Quads go two per workgroup while that fits 1024 threads (N is a multiple
// of 8, so the quads always pair up); octets and 12-wave quads one.
template <bool ZP, int ROWS>
hipError_t launch_rows(const u32x4* xv, const u32x4* wv, const uint16_t* sc, const uint32_t* qzeros, _Float16* yv,
                       int N, int K, int gs, int nw, hipStream_t stream) {
#define AWQ_GEMV_CASE(W)                                                                                        \
  case W:                                                                                                       \
    if (ROWS == 4 && W <= 8)                                                                                    \
      hipLaunchKernelGGL((gemv_kernel<W, ZP, ROWS, (ROWS == 4 && W <= 8) ? 2 : 1>), dim3(N / (2 * ROWS)),      \
                         dim3(W * 128), 0, stream, xv, wv, sc, qzeros, yv, N, K, gs);                           \
    else                                                                                                        \
      hipLaunchKernelGGL((gemv_kernel<W, ZP, ROWS, 1>), dim3(N / ROWS), dim3(W * 64), 0, stream, xv, wv, sc,    \
                         qzeros, yv, N, K, gs);                                                                 \
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
    AWQ_GEMV_CASE(12)
    default: return hipErrorInvalidValue;
  }
#undef AWQ_GEMV_CASE
  return hipGetLastError();
}

template <bool ZP>
hipError_t launch_zp(const void* x, const uint32_t* qweight, const void* scales, const uint32_t* qzeros, void* y,
                     int N, int K, int group_size, hipStream_t stream) {
  const int nw = gemv_waves(K);
  const u32x4* xv = static_cast<const u32x4*>(x);
  const u32x4* wv = reinterpret_cast<const u32x4*>(qweight);
  const uint16_t* sc = static_cast<const uint16_t*>(scales);
  _Float16* yv = static_cast<_Float16*>(y);
  const int gs = log2_group(group_size);
  // row octets halve the activation loads per weight byte, but take half as
  // many workgroups: they pay once the octets alone give ~32 waves per compute
  // unit (the 70B MLP layers, 48-56: 10-12% faster), quads stay faster below
  // (the 7B layers: 2-15%; the fused 4096 -> 22016 gate_up layer at 21.5: 7%)
  if (gemv_uses_octets(N, K))
    return launch_rows<ZP, 8>(xv, wv, sc, qzeros, yv, N, K, gs, nw, stream);
  return launch_rows<ZP, 4>(xv, wv, sc, qzeros, yv, N, K, gs, nw, stream);
}

}  // namespace

hipError_t launch_gemv(const void* x, const uint32_t* qweight, const void* scales, const uint32_t* qzeros, void* y,
                       int N, int K, int group_size, bool zero_point, hipStream_t stream) {
  return zero_point ? launch_zp<true>(x, qweight, scales, qzeros, y, N, K, group_size, stream)
                    : launch_zp<false>(x, qweight, scales, qzeros, y, N, K, group_size, stream);
}

}  // namespace awq
