// Batched W4A16 layer (awq_gemm): Y[M][N] = X[M][K] . W'^T, W' = (q - z) * s.
//
// The GEMM variant of the quantized linear layer ("AI-Research-SKILLs AWQ 高级
// 使用指南", section WQLinear 内核全景: general matrix multiplication for
// batches).  Weights are decoded to fp16 on the fly (exact q - z, one fp16
// rounding of the product with the group scale) and multiplied on the gfx950
// fp16 matrix cores with fp32 accumulation.  Two kernels:
//
//   * gemm_skinny_kernel (M <= 64): still bound by the weight stream.  A wave
//     owns NT tiles of 16 output rows and all (<= 4) tiles of 16 tokens; its
//     lanes load packed weights straight into MFMA B-operand registers (one
//     128-bit load = 32 channels of one row = four 16x16x32 B fragments), so
//     no LDS round trip sits on the weight path.  The NW waves of a workgroup
//     split K and are summed through LDS in a fixed order (deterministic, no
//     workspace, no atomics).
//
//   * gemm_large_kernel (M > 64): compute-bound.  256x256 output tile per
//     workgroup of 4 waves (2x2, 128x128 each, 4x4 v_mfma_f32_32x32x16_f16
//     tiles), K in steps of 64.  The next step's X tile and packed weights are
//     fetched into registers while the current step multiplies out of LDS; the
//     weights are then decoded and written to LDS as fp16 next to the X tile.
//     LDS rows are padded to 72 halves so that the 128-bit fragment reads of 8
//     consecutive rows hit distinct banks.  Workgroups are mapped so that each
//     XCD (and its L2) works on a contiguous band of tiles.
//
// MFMA operand placement: a lane's 8 fp16 values of A and of B cover the same
// 8 reduction indices, so any assignment of channels to (lane group, element)
// slots gives the same product as long as A and B use the same one.  Both
// kernels give a lane whole packed words (8 consecutive channels).
#include "awq_device.hpp"
#include "awq_launch.hpp"

namespace awq {
namespace {

int log2_group(int g) { return g == 32 ? 5 : g == 64 ? 6 : g == 128 ? 7 : 8; }

// --------------------------------------------------------------------------
// Skinny M: weight-stream bound.
// --------------------------------------------------------------------------
// Buffer resource over `bytes` bytes at `base`: loads past the end return 0
// and stores past the end are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

constexpr uint32_t kOutOfRange = 0x80000000u;  // a buffer offset past every resource: loads return 0

// Global data of one 128-channel step for one lane: its 32 channels of one
// weight row (4 packed words), the matching activations of its MT token rows,
// and the row's raw scale and zero-point word for the lane's group.
template <int MT>
struct SkinnyStep {
  u32x4 w;
  u32x4 x[MT][4];
  uint32_t s, z;
};

// One workgroup per 16 output rows, KS waves splitting K.  Wave w handles the
// 128-channel steps w, w + KS, ... in rounds of SPW steps; the loads of round
// r + 1 are in flight while round r is multiplied.  A lane (i, h) = (lane % 16,
// lane / 16) loads the 32 channels 128 c + 32 h .. +32 of row n0 + i as one
// 16-byte word, which is exactly its B operand for four 16x16x32 MFMAs, and
// the same channels of token rows 16 mt + i as the A operands.  The waves'
// partial sums meet in LDS and are added in wave order (deterministic).
template <int MT, int KS, int SPW, bool ZP>
__global__ __launch_bounds__(KS * 64) void gemm_skinny_kernel(const _Float16* __restrict__ X,
                                                              const uint32_t* __restrict__ qweight,
                                                              const uint16_t* __restrict__ scales,
                                                              const uint32_t* __restrict__ qzeros,
                                                              _Float16* __restrict__ Y, int M, int N, int K,
                                                              int gshift) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int li = lane & 15, lh = lane >> 4;
  const int n0 = blockIdx.x * 16;
  const int nrows = min(16, N - n0);  // 16, or 8 at the end of an N that is not a multiple of 16
  const int steps = (K + 127) >> 7;
  const int G = K >> gshift;
  const DecodeConsts kc;

  const __amdgpu_buffer_rsrc_t rw = make_rsrc(qweight + (size_t)n0 * (K >> 3), (uint32_t)nrows * (K >> 1));
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(X, (uint32_t)M * K * 2);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(scales + scale_index(n0, 0, G), (uint32_t)(nrows >> 3) * G * 16);
  const __amdgpu_buffer_rsrc_t rz = make_rsrc(ZP ? qzeros + zero_word_index(n0, 0, G) : qzeros,
                                              ZP ? (uint32_t)(nrows >> 3) * G * 4 : 0u);
  const uint32_t wbase = (uint32_t)li * (K >> 1) + lh * 16;
  const uint32_t sbase = (uint32_t)(((li >> 3) * G * 8 + (li & 7)) * 2);
  const uint32_t zbase = (uint32_t)((li >> 3) * G * 4);
  const int zshift = 4 * (li & 7);

  auto fetch = [&](SkinnyStep<MT>& r, int c) {
    const int k0 = (c << 7) + (lh << 5);  // first channel of the lane's 32
    const bool kin = c < steps && k0 < K;
    const int grp = k0 >> gshift;
    r.w = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, kin ? wbase + c * 64 : kOutOfRange, 0, 0));
    r.s = __builtin_amdgcn_raw_buffer_load_b16(rs, kin ? sbase + grp * 16 : kOutOfRange, 0, 0);
    r.z = ZP ? __builtin_amdgcn_raw_buffer_load_b32(rz, kin ? zbase + grp * 4 : kOutOfRange, 0, 0) : 0u;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      // token rows past M lie past the end of the X resource and read as 0
      const uint32_t xo = kin ? ((uint32_t)(16 * mt + li) * K + k0) * 2 : kOutOfRange;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        r.x[mt][e] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, xo, e * 16, 0));
    }
  };

  float4_t acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = float4_t{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const SkinnyStep<MT>& r) {
    const uint32_t z = ZP ? ((r.z >> zshift) & 15u) : 8u;
    const ZeroBias zb = zero_bias(z);
    const half2_t s2 = splat2(__builtin_bit_cast(_Float16, (uint16_t)r.s));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const half8_t b = decode_word_scaled(r.w[e], zb, kc, s2);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(r.x[mt][e]), b, acc[mt], 0, 0, 0);
    }
  };

  // rounds of SPW steps, double-buffered
  const int per_round = KS * SPW;
  const int rounds = (steps + per_round - 1) / per_round;
  SkinnyStep<MT> ra[SPW], rb[SPW];
#pragma unroll
  for (int u = 0; u < SPW; ++u) fetch(ra[u], wave + KS * u);
  int r = 0;
  for (; r + 1 < rounds; r += 2) {
#pragma unroll
    for (int u = 0; u < SPW; ++u) fetch(rb[u], wave + KS * (SPW * (r + 1) + u));
#pragma unroll
    for (int u = 0; u < SPW; ++u) compute(ra[u]);
    if (r + 2 < rounds) {
#pragma unroll
      for (int u = 0; u < SPW; ++u) fetch(ra[u], wave + KS * (SPW * (r + 2) + u));
    }
#pragma unroll
    for (int u = 0; u < SPW; ++u) compute(rb[u]);
  }
  if (r < rounds) {
#pragma unroll
    for (int u = 0; u < SPW; ++u) compute(ra[u]);
  }

  // 16x16 accumulator layout: lane (li, lh) holds column li, rows 4 lh + j.
  __shared__ float red[KS][MT * 4][64];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int j = 0; j < 4; ++j) red[wave][mt * 4 + j][lane] = acc[mt][j];
  __syncthreads();
  for (int o = t; o < MT * 4 * 64; o += KS * 64) {
    const int idx = o >> 6, ln = o & 63;
    float sum = red[0][idx][ln];
#pragma unroll
    for (int w = 1; w < KS; ++w) sum += red[w][idx][ln];
    const int m = 16 * (idx >> 2) + 4 * (ln >> 4) + (idx & 3), n = n0 + (ln & 15);
    if (m < M && n < N) Y[(size_t)m * N + n] = (_Float16)sum;
  }
}

// --------------------------------------------------------------------------
// Large M: matrix-core bound.
// --------------------------------------------------------------------------
constexpr int BM = 256, BN = 256, BK = 64;
constexpr int LDS_STRIDE = BK + 8;  // halves per LDS row (padding breaks bank conflicts)
constexpr int TILE_HALVES = BM * LDS_STRIDE;

// Registers holding one K step of global data on its way to LDS.
struct StepRegs {
  u32x4 x[4];    // X: 4 x 16 B
  u32x4 w;       // 32 channels of packed weights
  uint32_t s;    // raw fp16 scale (low half)
  uint32_t z;    // zero-point word
};

// 2 x 4 waves of 128 x 64 outputs (two waves per SIMD).  Every global access
// goes through a buffer resource based at the tile: a thread's 32-bit offsets
// are fixed for the whole K loop and the step advances an SGPR offset, rows
// past M or N read as zero and loads past the end of a tile return zero.
// Software pipeline, one barrier per K step:
//   iteration s: issue the global loads of step s + 2 (register set s & 1),
//   multiply step s out of LDS buffer s & 1, and, interleaved with those
//   MFMAs, decode step s + 1 (register set (s + 1) & 1) into LDS buffer
//   (s + 1) & 1.
// The loop has no branches: loads for steps past the end stay inside the
// buffers (or return zero) and land in an LDS buffer no one reads again.
template <bool ZP, bool KTAIL>
__global__ __launch_bounds__(512) void gemm_large_kernel(const _Float16* __restrict__ X,
                                                         const uint32_t* __restrict__ qweight,
                                                         const uint16_t* __restrict__ scales,
                                                         const uint32_t* __restrict__ qzeros,
                                                         _Float16* __restrict__ Y, int M, int N, int K, int gshift,
                                                         int tiles_m) {
  constexpr int WN = 64;                      // wave tile width (N)
  constexpr int NB = WN / 32;                 // 32x32 MFMA tiles per wave along N
  constexpr int XROWS = 512 / (BK / 8);       // X rows covered by one load round (64)
  __shared__ __attribute__((aligned(16))) _Float16 lds[2][2][TILE_HALVES];  // [buffer][X | W'][row * 72 + k]

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int tile = xcd_contiguous_tile(blockIdx.x, gridDim.x);
  const int tm = tile % tiles_m, tn = tile / tiles_m;
  const int m0 = tm * BM, n0 = tn * BN;
  const int rows_m = min(BM, M - m0), rows_n = min(BN, N - n0);  // rows_n is a multiple of 8
  const int wm = (wave & 1) * 128, wn = (wave >> 1) * WN;
  const int nsteps = (K + BK - 1) / BK;
  const int G = K >> gshift;
  const DecodeConsts kc;

  const __amdgpu_buffer_rsrc_t rx = make_rsrc(X + (size_t)m0 * K, (uint32_t)rows_m * K * 2);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(qweight + (size_t)n0 * (K >> 3), (uint32_t)rows_n * (K >> 1));
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(scales + scale_index(n0, 0, G), (uint32_t)(rows_n >> 3) * G * 16);
  const __amdgpu_buffer_rsrc_t rz = make_rsrc(ZP ? qzeros + zero_word_index(n0, 0, G) : qzeros,
                                              ZP ? (uint32_t)(rows_n >> 3) * G * 4 : 0u);

  // X: thread t loads 4 x 16 B: rows (t >> 3) + 64 i, channels 8 (t & 7) .. +8.
  // W: thread t loads one 16-byte piece (32 channels) of row t >> 1, plus the
  // scale and zero-point word of the piece's group.
  const int xr = t >> 3, xc = t & 7;
  const int wr = t >> 1, piece = t & 1;
  uint32_t xoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) xoff[i] = (uint32_t)(xr + XROWS * i) * K * 2 + xc * 16;
  const uint32_t woff = (uint32_t)wr * (K >> 1) + piece * 16;
  const bool g32 = gshift == 5;  // with g = 32 the two pieces of a step are two groups
  const uint32_t soff = (uint32_t)(((wr >> 3) * G * 8 + (wr & 7)) * 2) + (g32 ? piece * 16 : 0);
  const uint32_t zoff = (uint32_t)((wr >> 3) * G * 4) + (g32 ? piece * 4 : 0);
  const int zshift = 4 * (wr & 7);

  auto fetch = [&](StepRegs& r, int step) {
    const int grp = (step * BK) >> gshift;  // group of piece 0
#pragma unroll
    for (int i = 0; i < 4; ++i)
      r.x[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, xoff[i], step * BK * 2, 0));
    r.w = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, woff, step * (BK / 2), 0));
    r.s = __builtin_amdgcn_raw_buffer_load_b16(rs, soff, grp * 16, 0);
    r.z = ZP ? __builtin_amdgcn_raw_buffer_load_b32(rz, zoff, grp * 4, 0) : 0u;
  };

  // One quarter (q = 0..3) of the LDS stash of a step: one X vector and one
  // decoded packed word per thread.
  auto stash_part = [&](const StepRegs& r, int buf, int step, int q) {
    _Float16* xa = lds[buf][0];
    _Float16* wb = lds[buf][1];
    u32x4 xv = r.x[q];
    if constexpr (KTAIL) {  // zero the channels past K of the last step
      if (step * BK + 8 * xc >= K) xv = u32x4{0u, 0u, 0u, 0u};
    }
    *reinterpret_cast<u32x4*>(xa + (xr + XROWS * q) * LDS_STRIDE + 8 * xc) = xv;
    const uint32_t z = ZP ? ((r.z >> zshift) & 15u) : 8u;
    const half8_t v = decode_word_scaled(r.w[q], zero_bias(z), kc, splat2(__builtin_bit_cast(_Float16, (uint16_t)r.s)));
    *reinterpret_cast<half8_t*>(wb + wr * LDS_STRIDE + 32 * piece + 8 * q) = v;
  };

  float16_t acc[4][NB];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

  const int fi = lane & 31, fh = lane >> 5;  // fragment row and k-half of this lane

  // Multiply step `step` out of LDS buffer `buf`, and stash `nxt` (the data of
  // step + 1) into the other buffer, a quarter after each 16-channel slice.
  auto compute = [&](int step, const StepRegs& nxt) {
    const int buf = step & 1;
    const _Float16* xa = lds[buf][0] + (wm + fi) * LDS_STRIDE + 8 * fh;
    const _Float16* wb = lds[buf][1] + (wn + fi) * LDS_STRIDE + 8 * fh;
    half8_t af[2][4], bf[2][NB];
#pragma unroll
    for (int a = 0; a < 4; ++a) af[0][a] = *reinterpret_cast<const half8_t*>(xa + 32 * a * LDS_STRIDE);
#pragma unroll
    for (int b = 0; b < NB; ++b) bf[0][b] = *reinterpret_cast<const half8_t*>(wb + 32 * b * LDS_STRIDE);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int cur = ks & 1, nx = cur ^ 1;
      if (ks + 1 < BK / 16) {
#pragma unroll
        for (int a = 0; a < 4; ++a)
          af[nx][a] = *reinterpret_cast<const half8_t*>(xa + 32 * a * LDS_STRIDE + 16 * (ks + 1));
#pragma unroll
        for (int b = 0; b < NB; ++b)
          bf[nx][b] = *reinterpret_cast<const half8_t*>(wb + 32 * b * LDS_STRIDE + 16 * (ks + 1));
      }
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < NB; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[cur][a], bf[cur][b], acc[a][b], 0, 0, 0);
      stash_part(nxt, buf ^ 1, step + 1, ks);
    }
  };

  StepRegs ra, rb;
  fetch(ra, 0);
#pragma unroll
  for (int q = 0; q < 4; ++q) stash_part(ra, 0, 0, q);
  fetch(rb, 1);
  __syncthreads();

  // two steps per trip so that the register sets keep static names
  int step = 0;
  for (; step + 1 < nsteps; step += 2) {
    fetch(ra, step + 2);
    compute(step, rb);
    __syncthreads();
    fetch(rb, step + 3);
    compute(step + 1, ra);
    __syncthreads();
  }
  if (step < nsteps) compute(step, rb);

  // 32x32 accumulator layout: lane l holds column l % 32 and, in register r,
  // row 8 * (r / 4) + 4 * (l / 32) + r % 4.  Rows past M fall outside the
  // buffer and are dropped; columns past N are skipped.
  const __amdgpu_buffer_rsrc_t ry = make_rsrc(Y + (size_t)m0 * N, (uint32_t)rows_m * N * 2);
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int col = wn + 32 * b + fi;
      if (col >= rows_n) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm + 32 * a + 8 * (r >> 2) + 4 * fh + (r & 3);
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (_Float16)acc[a][b][r]), ry,
                                              (uint32_t)(row * N + n0 + col) * 2, 0, 0);
      }
    }
}

template <int MT, int KS, int SPW, bool ZP>
hipError_t launch_skinny(const void* x, const uint32_t* qw, const uint16_t* sc, const uint32_t* qz, _Float16* Y, int M,
                         int N, int K, int gs, hipStream_t stream) {
  hipLaunchKernelGGL((gemm_skinny_kernel<MT, KS, SPW, ZP>), dim3((N + 15) / 16), dim3(KS * 64), 0, stream,
                     static_cast<const _Float16*>(x), qw, sc, qz, Y, M, N, K, gs);
  return hipGetLastError();
}

template <bool ZP>
hipError_t launch_zp(const void* x, const uint32_t* qweight, const void* scales, const uint32_t* qzeros, void* y,
                     int M, int N, int K, int group_size, hipStream_t stream) {
  const uint16_t* sc = static_cast<const uint16_t*>(scales);
  _Float16* Y = static_cast<_Float16*>(y);
  const int gs = log2_group(group_size);
  if (M <= 64) {
    // up to 32 tokens: 8 waves of 2 steps per round; more tokens: 8 waves of 1 step
    switch ((M + 15) / 16) {
      case 1: return launch_skinny<1, 8, 2, ZP>(x, qweight, sc, qzeros, Y, M, N, K, gs, stream);
      case 2: return launch_skinny<2, 8, 2, ZP>(x, qweight, sc, qzeros, Y, M, N, K, gs, stream);
      case 3: return launch_skinny<3, 8, 1, ZP>(x, qweight, sc, qzeros, Y, M, N, K, gs, stream);
      default: return launch_skinny<4, 8, 1, ZP>(x, qweight, sc, qzeros, Y, M, N, K, gs, stream);
    }
  }
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  if (K % BK == 0)
    hipLaunchKernelGGL((gemm_large_kernel<ZP, false>), dim3(tiles_m * tiles_n), dim3(512), 0, stream,
                       static_cast<const _Float16*>(x), qweight, sc, qzeros, Y, M, N, K, gs, tiles_m);
  else
    hipLaunchKernelGGL((gemm_large_kernel<ZP, true>), dim3(tiles_m * tiles_n), dim3(512), 0, stream,
                       static_cast<const _Float16*>(x), qweight, sc, qzeros, Y, M, N, K, gs, tiles_m);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const void* x, const uint32_t* qweight, const void* scales, const uint32_t* qzeros, void* y,
                       int M, int N, int K, int group_size, bool zero_point, hipStream_t stream) {
  return zero_point ? launch_zp<true>(x, qweight, scales, qzeros, y, M, N, K, group_size, stream)
                    : launch_zp<false>(x, qweight, scales, qzeros, y, M, N, K, group_size, stream);
}

}  // namespace awq
