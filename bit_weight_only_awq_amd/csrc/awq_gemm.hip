// Batched W4A16 layer (awq_gemm): Y[M][N] = X[M][K] . W'^T, W' = (q - z) * s.
//
// The GEMM variant of the quantized linear layer ("AI-Research-SKILLs AWQ 高级
// 使用指南", section WQLinear 内核全景: general matrix multiplication for
// batches).  Weights are decoded to fp16 on the fly (exact q - z, one fp16
// rounding of the product with the group scale) and multiplied on the gfx950
// fp16 matrix cores with fp32 accumulation.  Two kernels:
//
//   * up to 8 tokens: the single- and few-token kernels of awq_gemv (one
//     token: the GEMV; 2-8: 4x4x4 MFMA blocks over 32-channel slices).
//
//   * gemm_skinny_kernel (9-64 tokens, but 33-64 tokens on layers with
//     N >= 8192 and 49-64 tokens on layers with K >= 8192 go to the
//     matrix-core kernel): bound by the weight stream (and, from
//     ~16 tokens on, by the activation loads).  A workgroup owns NT tiles of
//     16 output rows, all (<= 4) tiles of 16 tokens and one slice of K; its
//     lanes load packed weights straight into MFMA B-operand registers (one
//     128-bit load = 32 channels of one row = four 16x16x32 B fragments), so
//     no LDS round trip sits on the weight path.  The waves of a workgroup
//     split its slice and are summed through LDS in a fixed order; when K is
//     split across workgroups, fp32 partial tiles go through the caller's
//     workspace and the last workgroup of each tile adds them in slice order
//     (deterministic, one launch).
//
//   * gemm_large_kernel (M > 64, and the 33-64 token cases above on 64 x 128
//     tiles): matrix-core bound.  TBM x 256 output tile per
//     workgroup of 4 waves, one per SIMD, each TBM x 64
//     (v_mfma_f32_32x32x16_f16, accumulators in the AGPRs), K in steps of 64;
//     TBM = 256, or 128 / 64 where 256-row tiles are too few to fill the chip
//     (then with K split across workgroups and a reduction launch), and
//     TBM x 128 tiles for a last wave of tiles that would run half empty.  X tiles go from HBM straight into LDS
//     (buffer-to-LDS loads); packed weights are fetched two steps ahead into
//     registers and decoded once per workgroup straight into MFMA B operands
//     (no LDS on the weight path); the K loop is software-pipelined by hand.
//     LDS tiles use an XOR swizzle instead of padding; workgroups are mapped
//     so that each XCD (and its L2) works on a contiguous band of tiles, in
//     groups of 4 tile rows.
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

// Global data of one 128-channel step for one lane: its 32 channels of NT
// weight rows (4 packed words each) with each row's raw scale and zero-point
// word for the lane's group, and the matching activations of its MT token rows.
template <int MT, int NT>
struct SkinnyStep {
  u32x4 w[NT];
  uint32_t s[NT], z[NT];
  u32x4 x[MT][4];
};

// One workgroup computes a tile of 16 NT output rows x 16 MT token rows over
// one slice of K (split-K across workgroups).  Its KS waves take the slice's
// 128-channel steps round robin, in rounds of SPW steps whose loads are in
// flight while the previous round is multiplied.  Lane (i, h) = (lane % 16,
// lane / 16) loads the 32 channels 128 c + 32 h .. +32 of row 16 nt + i as one
// 16-byte word, which is exactly its B operand for four 16x16x32 MFMAs, and
// the same channels of token rows 16 mt + i as the A operands; one X fragment
// serves NT weight tiles.  The waves' partial sums meet in LDS and are added
// in wave order.  With one slice the tile is written to Y; with several, each
// workgroup writes its fp32 partial tile to the workspace and the last of the
// tile's workgroups to finish (an agent-scope counter per tile) adds the
// partials in slice order and writes Y, then resets the counter to zero.  The
// result does not depend on which workgroup finishes last.
template <int MT, int NT, int KS, int SPW, bool ZP>
__global__ __launch_bounds__(KS * 64) void gemm_skinny_kernel(const _Float16* __restrict__ X,
                                                              const uint32_t* __restrict__ qweight,
                                                              const uint16_t* __restrict__ scales,
                                                              const uint32_t* __restrict__ qzeros,
                                                              _Float16* __restrict__ Y, int M, int N, int K,
                                                              int gshift, int splits, int steps_per_split,
                                                              uint32_t* __restrict__ counters,
                                                              float* __restrict__ partials) {
  constexpr int kTileElems = MT * NT * 256;          // fp32 values of one 16 MT x 16 NT tile
  constexpr int kPerThread = (kTileElems + KS * 64 - 1) / (KS * 64);  // tile values per thread (o < kTileElems)
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int li = lane & 15, lh = lane >> 4;
  // consecutive ids on one XCD: the slices of a tile share that XCD's L2
  const int id = xcd_contiguous_tile(blockIdx.x, gridDim.x);
  const int tile = id / splits, split = id - tile * splits;
  const int n0 = tile * 16 * NT;
  const int nrows = min(16 * NT, N - n0);  // a multiple of 8
  const int steps = (K + 127) >> 7;
  const int c_begin = split * steps_per_split;
  const int c_end = min(steps, c_begin + steps_per_split);
  const int G = K >> gshift;
  const DecodeConsts kc;

  const __amdgpu_buffer_rsrc_t rw = make_rsrc(qweight + (size_t)n0 * (K >> 3), (uint32_t)nrows * (K >> 1));
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(X, (uint32_t)M * K * 2);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(scales + scale_index(n0, 0, G), (uint32_t)(nrows >> 3) * G * 16);
  const __amdgpu_buffer_rsrc_t rz = make_rsrc(ZP ? qzeros + zero_word_index(n0, 0, G) : qzeros,
                                              ZP ? (uint32_t)(nrows >> 3) * G * 4 : 0u);
  // row 16 nt + li of the tile: rows past nrows lie past the resources and read as 0
  uint32_t wbase[NT], sbase[NT], zbase[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = 16 * nt + li;
    wbase[nt] = (uint32_t)r * (K >> 1) + lh * 16;
    sbase[nt] = (uint32_t)(((r >> 3) * G * 8 + (r & 7)) * 2);
    zbase[nt] = (uint32_t)((r >> 3) * G * 4);
  }
  const int zshift = 4 * (li & 7);

  auto fetch = [&](SkinnyStep<MT, NT>& r, int c) {
    const int k0 = (c << 7) + (lh << 5);  // first channel of the lane's 32
    const bool kin = c < c_end && k0 < K;
    const int grp = k0 >> gshift;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      r.w[nt] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, kin ? wbase[nt] + c * 64 : kOutOfRange, 0, 0));
      r.s[nt] = __builtin_amdgcn_raw_buffer_load_b16(rs, kin ? sbase[nt] + grp * 16 : kOutOfRange, 0, 0);
      r.z[nt] = ZP ? __builtin_amdgcn_raw_buffer_load_b32(rz, kin ? zbase[nt] + grp * 4 : kOutOfRange, 0, 0) : 0u;
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      // token rows past M lie past the end of the X resource and read as 0
      const uint32_t xo = kin ? ((uint32_t)(16 * mt + li) * K + k0) * 2 : kOutOfRange;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        r.x[mt][e] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, xo, e * 16, 0));
    }
  };

  float4_t acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = float4_t{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const SkinnyStep<MT, NT>& r) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const uint32_t z = ZP ? ((r.z[nt] >> zshift) & 15u) : 8u;
      const ZeroBias zb = zero_bias(z);
      const half2_t s2 = splat2(__builtin_bit_cast(_Float16, (uint16_t)r.s[nt]));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const half8_t b = decode_word_scaled(r.w[nt][e], zb, kc, s2);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(r.x[mt][e]), b, acc[mt][nt], 0, 0, 0);
      }
    }
  };

  // rounds of SPW steps, double-buffered
  const int per_round = KS * SPW;
  const int rounds = (c_end - c_begin + per_round - 1) / per_round;
  const int c0 = c_begin + wave;
  SkinnyStep<MT, NT> ra[SPW], rb[SPW];
#pragma unroll
  for (int u = 0; u < SPW; ++u) fetch(ra[u], c0 + KS * u);
  int r = 0;
  for (; r + 1 < rounds; r += 2) {
#pragma unroll
    for (int u = 0; u < SPW; ++u) fetch(rb[u], c0 + KS * (SPW * (r + 1) + u));
#pragma unroll
    for (int u = 0; u < SPW; ++u) compute(ra[u]);
    if (r + 2 < rounds) {
#pragma unroll
      for (int u = 0; u < SPW; ++u) fetch(ra[u], c0 + KS * (SPW * (r + 2) + u));
    }
#pragma unroll
    for (int u = 0; u < SPW; ++u) compute(rb[u]);
  }
  if (r < rounds) {
#pragma unroll
    for (int u = 0; u < SPW; ++u) compute(ra[u]);
  }

  // 16x16 accumulator layout: lane (li, lh) holds column li, rows 4 lh + j.
  // Tile value o = 64 ((mt NT + nt) 4 + j) + lane.
  __shared__ float red[KS][MT * NT * 4][64];
  __shared__ int is_last;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int j = 0; j < 4; ++j) red[wave][(mt * NT + nt) * 4 + j][lane] = acc[mt][nt][j];
  __syncthreads();
  float sum[kPerThread];
#pragma unroll
  for (int q = 0; q < kPerThread; ++q) {
    const int o = t + q * KS * 64, idx = o >> 6, ln = o & 63;
    float v = 0.0f;
    if (o < kTileElems) {
      v = red[0][idx][ln];
#pragma unroll
      for (int w = 1; w < KS; ++w) v += red[w][idx][ln];
    }
    sum[q] = v;
  }

  if (splits > 1) {
    // Hand-off between the workgroups of a tile, which may run on different
    // XCDs (separate L2s).  Partials are written and read with device-scope
    // coherence (the SC1 cache-policy bit: the access is performed at the
    // agent's coherence point, as for agent-scope atomics), and each thread
    // waits for its partial stores to be acknowledged before the workgroup
    // barrier that precedes the counter increment; the reads are issued after
    // the increment has returned.  This orders the hand-off without
    // agent-scope fences, which would write back and invalidate whole L2s.
    constexpr int kDeviceScope = 1 << 4;  // SC1
    const __amdgpu_buffer_rsrc_t rp =
        make_rsrc(partials + (size_t)tile * splits * kTileElems, (uint32_t)splits * kTileElems * 4);
#pragma unroll
    for (int q = 0; q < kPerThread; ++q) {
      const int o = t + q * KS * 64;
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, sum[q]), rp,
                                            o < kTileElems ? (uint32_t)(split * kTileElems + o) * 4 : kOutOfRange, 0,
                                            kDeviceScope);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (t == 0) {
      const uint32_t prev = __hip_atomic_fetch_add(counters + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      is_last = prev == (uint32_t)(splits - 1);
      if (is_last) __hip_atomic_store(counters + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!is_last) return;
    // slices in order, four loads in flight per value; this workgroup's own
    // slice comes from its registers
    float tot[kPerThread];
    for (int s0 = 0; s0 < splits; s0 += 4) {
      float p[4][kPerThread];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int q = 0; q < kPerThread; ++q) {
          const int s = s0 + u, o = t + q * KS * 64;
          const uint32_t off =
              s < splits && s != split && o < kTileElems ? (uint32_t)(s * kTileElems + o) * 4 : kOutOfRange;
          p[u][q] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rp, off, 0, kDeviceScope));
        }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int q = 0; q < kPerThread; ++q) {
          const int s = s0 + u;
          const float v = s == split ? sum[q] : p[u][q];
          if (s == 0) tot[q] = v;
          else if (s < splits) tot[q] += v;
        }
    }
#pragma unroll
    for (int q = 0; q < kPerThread; ++q) sum[q] = tot[q];
  }

#pragma unroll
  for (int q = 0; q < kPerThread; ++q) {
    const int o = t + q * KS * 64, idx = o >> 6, ln = o & 63;
    const int mt = idx / (NT * 4), nt = (idx >> 2) % NT;
    const int m = 16 * mt + 4 * (ln >> 4) + (idx & 3), n = 16 * nt + (ln & 15);
    if (o < kTileElems && m < M && n < nrows) Y[(size_t)m * N + n0 + n] = (_Float16)sum[q];
  }
}

// Launch plan of the skinny kernel for an M x N x K product: token tiles,
// row tiles per workgroup, waves, steps per round and the K split.  The
// workspace size follows from it, so awq_gemm_workspace_bytes and the
// launcher share this one function.
struct SkinnyPlan {
  int mt, nt, ks, spw;
  int tiles_n, steps, splits, steps_per_split;
};

SkinnyPlan plan_skinny(int M, int N, int K) {
  SkinnyPlan p;
  p.mt = (M + 15) / 16;
  // Measured on the Llama-7B decode shapes (4096 x 4096, 4096 -> 11008,
  // 11008 -> 4096): from 9 tokens on (up to 8 go to the few-token kernel)
  // the activations dominate the load traffic and wide row tiles (each X
  // fragment reused by NT weight tiles) win, with K split to keep every
  // compute unit busy.
  int target_blocks;
  if (p.mt == 1) {
    p.nt = 2, p.ks = 4, p.spw = 2, target_blocks = 512;
  } else {
    p.nt = 4, p.ks = 4, p.spw = 1, target_blocks = 256;
  }
  p.tiles_n = (N + 16 * p.nt - 1) / (16 * p.nt);
  p.steps = (K + 127) / 128;
  int splits = (target_blocks + p.tiles_n - 1) / p.tiles_n;
  const int max_splits = (p.steps + p.ks - 1) / p.ks;  // each wave gets a step
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  p.steps_per_split = (p.steps + splits - 1) / splits;
  p.splits = (p.steps + p.steps_per_split - 1) / p.steps_per_split;  // no empty slice
  return p;
}

// The workspace starts with a counter region of fixed size, one 32-bit
// counter for every possible 16-row tile (N <= 2^21), so that calls of any
// shape sharing one workspace find their counters at zero: partial tiles
// always lie after it.
constexpr size_t kCounterBytes = ((size_t)1 << 21) / 16 * 4;

size_t skinny_workspace_bytes(const SkinnyPlan& p) {
  if (p.splits <= 1) return 0;
  return kCounterBytes + (size_t)p.tiles_n * p.splits * p.mt * p.nt * 256 * 4;
}

template <int MT, int NT, int KS, int SPW, bool ZP>
hipError_t launch_skinny(const SkinnyPlan& p, const void* x, const uint32_t* qw, const uint16_t* sc,
                         const uint32_t* qz, _Float16* Y, int M, int N, int K, int gs, void* workspace,
                         hipStream_t stream) {
  // the grid and the workspace follow the plan; the kernel's tile follows the
  // template arguments, so the two must agree
  if (p.mt != MT || p.nt != NT || p.ks != KS || p.spw != SPW) return hipErrorInvalidValue;
  uint32_t* counters = static_cast<uint32_t*>(workspace);
  float* partials = workspace ? reinterpret_cast<float*>(static_cast<char*>(workspace) + kCounterBytes) : nullptr;
  hipLaunchKernelGGL((gemm_skinny_kernel<MT, NT, KS, SPW, ZP>), dim3(p.tiles_n * p.splits), dim3(KS * 64), 0, stream,
                     static_cast<const _Float16*>(x), qw, sc, qz, Y, M, N, K, gs, p.splits, p.steps_per_split,
                     counters, partials);
  return hipGetLastError();
}
// --------------------------------------------------------------------------
// Large M: matrix-core bound.
// --------------------------------------------------------------------------
constexpr int BM = 256, BN = 256, BK = 64;  // the full tile; 128-row tiles where 256-row ones are too few

// LDS layout of a 256 x 64 fp16 tile: row r occupies bytes 128 r .. 128 r + 127,
// and its 16-byte chunk c (channels 8 c .. 8 c + 7) sits in slot
// c ^ ((r >> 1) & 7).  The LDS serves 16 lanes x 16 bytes (all 64 banks) per
// cycle; 16 consecutive rows read at the same logical chunk land in 16
// different bank groups (even and odd rows fill the two 128-byte halves), so
// the MFMA fragment reads are conflict-free without padding, and a 1 KiB run
// of slots is exactly what one buffer-to-LDS load of 64 lanes x 16 bytes writes.
__device__ __forceinline__ int swz_chunk(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

// One wave per SIMD: 4 waves of TBM x (32 NB) outputs (tile TBM x 128 NB, TBM
// = 256, or 128 where 256-row tiles are too few), every wave multiplying all
// TBM rows of the X tile, so each packed weight word is loaded and decoded
// once per workgroup (1.9 VALU instructions per MFMA at TBM = 256; with two
// M-halves decoding the same words it was 3.7, and at the power limit every
// VALU instruction per MFMA costs about 3% of throughput).  The TBM accumulators
// per lane sit in the AGPRs.
//
// Only X goes through LDS: tiles go from HBM straight into LDS by
// buffer-to-LDS loads, double-buffered.  The weights go to the matrix cores
// without LDS: with the channel-to-slot assignment below, the B fragment of a
// lane for one 16-channel slice is one packed word of one weight row, so lane
// (n, h) of a wave loads the 32 channels 64 s + 32 h .. +32 of its row as one
// 16-byte word (four slices) two steps ahead and decodes each word one slice
// before its MFMAs.  Software-pipelined by hand, as a single wave per SIMD
// has no other wave to hide latency behind: while the 16 MFMAs of one slice
// run, the wave reads the next slice's A fragments from LDS and decodes its B
// fragments (scheduling groups interleave one LDS read and four VALU
// instructions with every two MFMAs); the step's barrier sits before the last
// slice, whose MFMAs overlap the next step's first reads, its buffer-to-LDS
// loads and its first decode.  Every global access goes through a buffer
// resource based at the tile (rows past M or N read as zero), and the K loop
// has no branches: loads for steps past the end carry an out-of-range lane
// offset (they return zero) and land where no one reads again.
//   MFMA slice ks of step s, lane half h, element j  <->  channel 64 s + 32 h + 8 ks + j
// (A and B use the same assignment, so the product is unchanged.)
template <bool ZP, bool KTAIL, int NB, int TBM>
__global__ __launch_bounds__(256) void gemm_large_kernel(const _Float16* __restrict__ X,
                                                         const uint32_t* __restrict__ qweight,
                                                         const uint16_t* __restrict__ scales,
                                                         const uint32_t* __restrict__ qzeros,
                                                         _Float16* __restrict__ Y, int M, int N, int K, int gshift,
                                                         int tiles_m, int group_m, int ldy, int splits,
                                                         int steps_per_split, float* __restrict__ part) {
  constexpr int NW = 4, WMT = TBM / 32;       // waves; 32-row MFMA tiles per wave
  constexpr int WN = 32 * NB, TBN = NW * WN;  // wave and workgroup tile widths
  constexpr int XROWS = TBM / NW;             // X tile rows each wave loads, 8 per 1 KiB load
  constexpr int TILE_BYTES = TBM * BK * 2;    // one TBM x 64 fp16 tile in LDS
  // two arrays, so that the compiler's wait for buffer-to-LDS loads in flight
  // before an LDS read covers only the loads into the array being read
  __shared__ __attribute__((aligned(1024))) char lx0[TILE_BYTES], lx1[TILE_BYTES];

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  // with K split over `splits` workgroups per tile: the workgroups of one
  // slice are consecutive, so an XCD works on tiles of the same K slice
  const int id = xcd_contiguous_tile(blockIdx.x, gridDim.x);
  const int tiles = gridDim.x / splits;
  const int split = id / tiles, tile = id - split * tiles;
  const int tiles_n = tiles / tiles_m;
  const int per_group = group_m * tiles_n, grp0 = tile / per_group, first_m = grp0 * group_m;
  const int gm = min(tiles_m - first_m, group_m), r_in = tile - grp0 * per_group;
  const int tm = first_m + r_in % gm, tn = r_in / gm;
  const int m0 = tm * TBM, n0 = tn * TBN;
  const int rows_m = min(TBM, M - m0), rows_n = min(TBN, N - n0);
  const int wn = wave * WN;
  const int nsteps = (K + BK - 1) / BK;
  const int s0 = split * steps_per_split, s1 = min(nsteps, s0 + steps_per_split);  // this workgroup's K steps
  const int G = K >> gshift;
  const DecodeConsts kc;

  const __amdgpu_buffer_rsrc_t rx = make_rsrc(X + (size_t)m0 * K, (uint32_t)rows_m * K * 2);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(qweight + (size_t)n0 * (K >> 3), (uint32_t)rows_n * (K >> 1));
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(scales + scale_index(n0, 0, G), (uint32_t)(rows_n >> 3) * G * 16);
  const __amdgpu_buffer_rsrc_t rz = make_rsrc(ZP ? qzeros + zero_word_index(n0, 0, G) : qzeros,
                                              ZP ? (uint32_t)(rows_n >> 3) * G * 4 : 0u);

  // X: wave w fills tile rows XROWS w .. XROWS (w + 1) - 1
  int xchunk[XROWS / 8];
  uint32_t xoff[XROWS / 8];
#pragma unroll
  for (int j = 0; j < XROWS / 8; ++j) {
    const int row = XROWS * wave + 8 * j + (lane >> 3);
    xchunk[j] = swz_chunk(row, lane & 7);
    xoff[j] = (uint32_t)row * K * 2 + xchunk[j] * 16;
  }
  // `buf` is a constant at every call site (the K loop is unrolled by two)
  auto load_x = [&](int step, int buf) {
    char* dst = (buf ? lx1 : lx0) + wave * XROWS * 128;
#pragma unroll
    for (int j = 0; j < XROWS / 8; ++j) {
      // the step goes into the instruction's scalar offset, which the
      // hardware leaves out of the range check: a prefetch past the last
      // step must carry the out-of-range lane offset instead
      uint32_t off = step < nsteps ? xoff[j] : kOutOfRange;
      if constexpr (KTAIL) {
        if (step * BK + 8 * xchunk[j] >= K) off = kOutOfRange;
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (__attribute__((address_space(3))) void*)(dst + 1024 * j), 16, off,
                                               step * BK * 2, 0, 0);
    }
  };

  // W: lane (n = lane % 32, h = lane / 32) of this wave, rows wn + 32 b + n
  const int fi = lane & 31, fh = lane >> 5;
  uint32_t woff[NB], soff[NB], zoff[NB];
  int zshift[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int row = wn + 32 * b + fi;
    woff[b] = (uint32_t)row * (K >> 1) + fh * 16;
    soff[b] = (uint32_t)(((row >> 3) * G * 8 + (row & 7)) * 2);
    zoff[b] = (uint32_t)((row >> 3) * G * 4);
    zshift[b] = 4 * (row & 7);
  }
  struct WRegs {
    u32x4 w[NB];
    uint32_t s[NB], z[NB];
  };
  auto fetch_w = [&](WRegs& r, int step) {
    const int k0 = step * BK + 32 * fh;
    // past the last step the weight row offset would run off the buffer
    // through the scalar offset, which is not range-checked (see load_x)
    const bool kin = step < nsteps && (!KTAIL || k0 < K);
    const int grp = k0 >> gshift;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      r.w[b] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, kin ? woff[b] : kOutOfRange, step * (BK / 2), 0));
      // the group depends on the lane half: a per-lane offset, not a uniform one
      r.s[b] = __builtin_amdgcn_raw_buffer_load_b16(rs, soff[b] + grp * 16, 0, 0);
      r.z[b] = ZP ? __builtin_amdgcn_raw_buffer_load_b32(rz, zoff[b] + grp * 4, 0, 0) : 0u;
    }
  };

  float16_t acc[WMT][NB];
#pragma unroll
  for (int a = 0; a < WMT; ++a)
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

  const int fsw = (fi >> 1) & 7;  // swizzle of the fragment rows (tile row bases are multiples of 32)
  ZeroBias zb[NB];
  half2_t s2[NB];
  auto prep = [&](const WRegs& r) {  // the step's zero points and scales
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      zb[b] = zero_bias(ZP ? ((r.z[b] >> zshift[b]) & 15u) : 8u);
      s2[b] = splat2(__builtin_bit_cast(_Float16, (uint16_t)r.s[b]));
    }
  };
  half8_t af[2][WMT], bf[2][NB];
  // A fragments of slice ks of the tile in `buf` into af[d]; B fragments of
  // slice ks of the words in r into bf[d]; the MFMAs of af[d] x bf[d]
  auto read_a = [&](int buf, int ks, int d) {
    const char* xa = (buf ? lx1 : lx0) + fi * 128 + 16 * ((4 * fh + ks) ^ fsw);
#pragma unroll
    for (int a = 0; a < WMT; ++a) af[d][a] = *reinterpret_cast<const half8_t*>(xa + 32 * 128 * a);
  };
  auto decode_b = [&](const WRegs& r, int ks, int d) {
#pragma unroll
    for (int b = 0; b < NB; ++b) bf[d][b] = decode_word_scaled(r.w[b][ks], zb[b], kc, s2[b]);
  };
  auto mfmas = [&](int d) {
#pragma unroll
    for (int a = 0; a < WMT; ++a)
#pragma unroll
      for (int b = 0; b < NB; ++b)
        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[d][a], bf[d][b], acc[a][b], 0, 0, 0);
  };
  // the slice's scheduling groups: per 32-row tile, one LDS read, an MFMA,
  // three VALU instructions, the tile's other MFMAs, one VALU instruction
  auto interleave = [&]() {
#pragma unroll
    for (int i = 0; i < WMT; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // VALU
      __builtin_amdgcn_sched_group_barrier(0x008, NB - 1 > 0 ? NB - 1 : 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);
    }
  };
  // one K step with the tile in buffer c and its words in wc (wnx: the next
  // step's words).  On entry af[0] / bf[0] hold slice 0; with `handover`, on
  // exit they hold slice 0 of the next step.
  auto body = [&](int c, WRegs& wc, const WRegs& wnx, int step, bool handover) {
#pragma unroll
    for (int ks = 0; ks < 3; ++ks) {
      const int d = ks & 1;
      read_a(c, ks + 1, d ^ 1);
      decode_b(wc, ks + 1, d ^ 1);
      if (ks == 2) fetch_w(wc, step + 2);  // wc fully decoded
      mfmas(d);
      interleave();
      __builtin_amdgcn_sched_barrier(0);
    }
    if (handover) {
      // the next tile has landed everywhere and no wave still reads this one
      __syncthreads();
      asm volatile("" ::: "memory");
      load_x(step + 2, c);
      prep(wnx);
      read_a(c ^ 1, 0, 0);
      decode_b(wnx, 0, 0);
    }
    mfmas(1);
    interleave();
    __builtin_amdgcn_sched_barrier(0);
  };

  WRegs w0, w1;
  load_x(s0, 0);
  fetch_w(w0, s0);
  fetch_w(w1, s0 + 1);
  __syncthreads();
  load_x(s0 + 1, 1);
  prep(w0);
  read_a(0, 0, 0);
  decode_b(w0, 0, 0);
  int step = s0;
  for (; step + 1 < s1; step += 2) {
    body(0, w0, w1, step, true);
    body(1, w1, w0, step + 1, true);
  }
  if (step < s1) body(0, w0, w1, step, false);

  // 32x32 accumulator layout: lane l holds column l % 32 and, in register r,
  // row 8 (r / 4) + 4 (l / 32) + r % 4.  Rows past M fall outside the buffer
  // and are dropped; columns past N are skipped.  With K split, the fp32
  // partial tile goes to part[split][M][N] (rows of the tile at stride N).
  if (splits == 1) {
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(Y + (size_t)m0 * ldy, (uint32_t)rows_m * ldy * 2);
#pragma unroll
    for (int a = 0; a < WMT; ++a)
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int col = wn + 32 * b + fi;
        if (col >= rows_n) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = 32 * a + 8 * (r >> 2) + 4 * fh + (r & 3);
          __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (_Float16)acc[a][b][r]), ry,
                                                (uint32_t)(row * ldy + n0 + col) * 2, 0, 0);
        }
      }
  } else {
    const __amdgpu_buffer_rsrc_t rp =
        make_rsrc(part + ((size_t)split * M + m0) * N, (uint32_t)rows_m * N * 4);
#pragma unroll
    for (int a = 0; a < WMT; ++a)
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int col = wn + 32 * b + fi;
        if (col >= rows_n) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = 32 * a + 8 * (r >> 2) + 4 * fh + (r & 3);
          // through a named float: a bit cast applied to the vector element
          // itself was compiled into stores of one register for every r
          const float v = acc[a][b][r];
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rp,
                                                (uint32_t)(row * N + n0 + col) * 4, 0, 0);
        }
      }
  }
}

// Y[m][n] = fp16(sum over the K slices s = 0, 1, ... of part[s][m][n]), four
// outputs per thread, the slices added in order.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float4_t* __restrict__ part, int splits,
                                                            size_t quads, _Float16* __restrict__ Y) {
  typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < quads; i += (size_t)gridDim.x * 256) {
    float4_t v = part[i];
    for (int s = 1; s < splits; ++s) v += part[(size_t)s * quads + i];
    half4_t h;
    h[0] = (_Float16)v[0];
    h[1] = (_Float16)v[1];
    h[2] = (_Float16)v[2];
    h[3] = (_Float16)v[3];
    reinterpret_cast<half4_t*>(Y)[i] = h;
  }
}

struct LargePlan {
  int tbm, splits, steps_per_split;
};

// Tile height and K split of the matrix-core kernel, from a small time model:
// waves of workgroups over the compute units times the steps each takes (a
// 256 x 256 x 64 tile step ~1.2 us, a 128-row one ~0.70 us: half the matrix
// work, twice the weight decode per product; a last wave at most half full
// runs as half-width tiles without a K split and costs ~0.6 of a wave with
// 256-row tiles, ~0.85 with 128-row ones), plus, with K split, the fp32
// partials written and read at ~5 TB/s and the reduction launch.  128-row
// tiles win where 256-row ones are too few to fill the chip without a K split
// (4096-wide layers up to a few thousand tokens: 10-12% faster there).
LargePlan plan_large(int M, int N, int K) {
  const int steps = (K + BK - 1) / BK;
  constexpr int kUnits = 256;
  LargePlan best{BM, 1, steps};
  double best_t = 1e300;
  for (int tbm : {BM, BM / 2}) {
    const double step_us = tbm == BM ? 1.2 : 0.70, half_tail = tbm == BM ? 0.6 : 0.85;
    auto waves = [&](int wgs, bool split) {
      const int full = wgs / kUnits, rem = wgs % kUnits;
      if (rem == 0) return (double)full;
      return full + (!split && full > 0 && 2 * rem <= kUnits ? half_tail : 1.0);
    };
    const int tiles = ((M + tbm - 1) / tbm) * ((N + BN - 1) / BN);
    const double t1 = waves(tiles, false) * steps * step_us;
    if (t1 < best_t) {
      best_t = t1;
      best = {tbm, 1, steps};
    }
    // partial tiles are addressed with 32-bit offsets: tile rows x N fp32 < 2^31
    if ((size_t)tbm * N * 4 >= ((size_t)1 << 31)) continue;
    for (int s = 2; s <= 16 && steps / s >= 2; ++s) {
      const int spp = (steps + s - 1) / s;
      const int sp = (steps + spp - 1) / spp;
      const double t = waves(tiles * sp, true) * spp * step_us + (double)sp * M * N * 8 / 5e6 + 2.0;
      if (t < best_t) {
        best_t = t;
        best = {tbm, sp, spp};
      }
    }
  }
  return best;
}

int compute_units() {
  static int cus = [] {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    return n;
  }();
  return cus;
}

template <bool ZP, int NB, int TBM>
void launch_large_part(const _Float16* X, const uint32_t* qw, const uint16_t* sc, const uint32_t* qz, _Float16* Y, int M,
                       int N, int K, int gs, int n_base, int ldy, hipStream_t stream, LargePlan plan,
                       float* part = nullptr) {
  constexpr int TBN = 128 * NB;
  const int G = K >> gs;
  const int tiles_m = (M + TBM - 1) / TBM, tiles_n = (N + TBN - 1) / TBN;
  // tiles are ordered in groups of 4 tile rows (all tile columns of a group
  // before the next group), so the 32-tile band that one XCD works on spans
  // 4 row bands of X and 8 column bands of W instead of all row bands: about
  // 35% less traffic from HBM / Infinity Cache into the XCDs' L2s
  const int group_m = tiles_m < 4 ? tiles_m : 4;
  const uint32_t* qwp = qw + (size_t)n_base * (K >> 3);
  const uint16_t* scp = sc + scale_index(n_base, 0, G);
  const uint32_t* qzp = ZP ? qz + zero_word_index(n_base, 0, G) : qz;
  const int spp = plan.splits > 1 ? plan.steps_per_split : (K + BK - 1) / BK;
  const dim3 grid(tiles_m * tiles_n * plan.splits);
  if (K % BK == 0)
    hipLaunchKernelGGL((gemm_large_kernel<ZP, false, NB, TBM>), grid, dim3(256), 0, stream, X, qwp, scp, qzp,
                       Y + n_base, M, N, K, gs, tiles_m, group_m, ldy, plan.splits, spp, part);
  else
    hipLaunchKernelGGL((gemm_large_kernel<ZP, true, NB, TBM>), grid, dim3(256), 0, stream, X, qwp, scp, qzp,
                       Y + n_base, M, N, K, gs, tiles_m, group_m, ldy, plan.splits, spp, part);
}

// TBM x 256 tiles; when the last wave of tiles over the compute units would
// run at most half full, the N columns of that wave are computed instead as
// TBM x 128 tiles in a second launch, so the tail takes half a tile time.
template <bool ZP, int TBM>
hipError_t launch_large_tbm(const _Float16* X, const uint32_t* qw, const uint16_t* sc, const uint32_t* qz, _Float16* Y,
                            int M, int N, int K, int gs, void* workspace, const LargePlan& plan, hipStream_t stream) {
  if (plan.splits > 1) {
    // partials after the counter region of the skinny kernel, which stays zero
    float* part = reinterpret_cast<float*>(static_cast<char*>(workspace) + kCounterBytes);
    // the 64-row tiles (33-64 tokens) are 128 columns wide: twice the tiles
    // for the same K split, 3-5% faster than 256-column ones
    if constexpr (TBM == 64)
      launch_large_part<ZP, 1, TBM>(X, qw, sc, qz, Y, M, N, K, gs, 0, N, stream, plan, part);
    else
      launch_large_part<ZP, 2, TBM>(X, qw, sc, qz, Y, M, N, K, gs, 0, N, stream, plan, part);
    const size_t quads = (size_t)M * N / 4;
    size_t blocks = (quads + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       reinterpret_cast<const float4_t*>(part), plan.splits, quads, Y);
    return hipGetLastError();
  }
  const int cus = compute_units();
  const int tiles_m = (M + TBM - 1) / TBM, tiles_n = (N + BN - 1) / BN;
  const int tiles = tiles_m * tiles_n, rem = tiles % cus;
  int tail_n = 0;  // 256-wide N tiles moved to the half-width launch
  if (tiles > cus && rem > 0 && 2 * rem <= cus) {
    tail_n = (rem + tiles_m - 1) / tiles_m;
    if (tail_n >= tiles_n) tail_n = 0;
  }
  const int n_main = (tiles_n - tail_n) * BN;
  if (n_main > 0) launch_large_part<ZP, 2, TBM>(X, qw, sc, qz, Y, M, tail_n ? n_main : N, K, gs, 0, N, stream, plan);
  if (tail_n) launch_large_part<ZP, 1, TBM>(X, qw, sc, qz, Y, M, N - n_main, K, gs, n_main, N, stream, plan);
  return hipGetLastError();
}

// 33-64 tokens on wide layers (N >= 8192), and 49-64 tokens on layers with
// K >= 8192: the matrix-core kernel on 64 x 128 tiles, K split to about 128
// (wide layers) or 256 workgroups.  Its waves share each activation tile
// through LDS, where the skinny kernel's waves each load their own from L2
// (4096 -> 11008 at 64 tokens: 21.5 us against 31.9 us, at 48 tokens 20.9
// against 23.3; 11008 -> 4096 at 56 / 64 tokens: 19.4 / 19.5 us against 22.2 /
// 22.9, where the skinny kernel moves to four 16-token tiles).  On 4096 x 4096
// layers the skinny kernel stays faster (12.9 against 13.6 us at 64 tokens).
bool gemm_uses_mid(int M, int N, int K) {
  return M <= 64 && ((M > 32 && N >= 8192) || (M > 48 && K >= 8192));
}

LargePlan plan_mid(int M, int N, int K) {
  (void)M;
  const int steps = (K + BK - 1) / BK;
  const int tiles = (N + BN / 2 - 1) / (BN / 2);
  const int target = N >= 8192 ? 128 : 256;
  int s = (target + tiles - 1) / tiles;
  if (s > steps / 2) s = steps / 2;
  if (s < 1) s = 1;
  const int spp = (steps + s - 1) / s;
  return LargePlan{64, (steps + spp - 1) / spp, spp};
}

template <bool ZP>
hipError_t launch_large(const _Float16* X, const uint32_t* qw, const uint16_t* sc, const uint32_t* qz, _Float16* Y,
                        int M, int N, int K, int gs, void* workspace, hipStream_t stream) {
  if (gemm_uses_mid(M, N, K))
    return launch_large_tbm<ZP, 64>(X, qw, sc, qz, Y, M, N, K, gs, workspace, plan_mid(M, N, K), stream);
  const LargePlan plan = plan_large(M, N, K);
  return plan.tbm == BM ? launch_large_tbm<ZP, BM>(X, qw, sc, qz, Y, M, N, K, gs, workspace, plan, stream)
                        : launch_large_tbm<ZP, BM / 2>(X, qw, sc, qz, Y, M, N, K, gs, workspace, plan, stream);
}

template <bool ZP>
hipError_t launch_zp(const void* x, const uint32_t* qweight, const void* scales, const uint32_t* qzeros, void* y,
                     int M, int N, int K, int group_size, void* workspace, hipStream_t stream) {
  const uint16_t* sc = static_cast<const uint16_t*>(scales);
  _Float16* Y = static_cast<_Float16*>(y);
  const int gs = log2_group(group_size);
  if (M == 1) return launch_gemv(x, qweight, scales, qzeros, y, N, K, group_size, ZP, stream);
  if (M <= kMaxGemvTokens) return launch_gemv_small(x, qweight, scales, qzeros, y, M, N, K, group_size, ZP, stream);
  if (M <= 64 && !gemm_uses_mid(M, N, K)) {
    const SkinnyPlan p = plan_skinny(M, N, K);
    switch (p.mt) {
      case 1: return launch_skinny<1, 2, 4, 2, ZP>(p, x, qweight, sc, qzeros, Y, M, N, K, gs, workspace, stream);
      case 2: return launch_skinny<2, 4, 4, 1, ZP>(p, x, qweight, sc, qzeros, Y, M, N, K, gs, workspace, stream);
      case 3: return launch_skinny<3, 4, 4, 1, ZP>(p, x, qweight, sc, qzeros, Y, M, N, K, gs, workspace, stream);
      default: return launch_skinny<4, 4, 4, 1, ZP>(p, x, qweight, sc, qzeros, Y, M, N, K, gs, workspace, stream);
    }
  }
  return launch_large<ZP>(static_cast<const _Float16*>(x), qweight, sc, qzeros, Y, M, N, K, gs, workspace, stream);
}

}  // namespace

size_t gemm_counter_bytes() { return kCounterBytes; }

size_t gemm_workspace_bytes(int M, int N, int K) {
  if (M <= kMaxGemvTokens) return 0;
  if (M <= 64 && !gemm_uses_mid(M, N, K)) return skinny_workspace_bytes(plan_skinny(M, N, K));
  const LargePlan p = gemm_uses_mid(M, N, K) ? plan_mid(M, N, K) : plan_large(M, N, K);
  return p.splits > 1 ? kCounterBytes + (size_t)p.splits * M * N * 4 : 0;
}

hipError_t launch_gemm(const void* x, const uint32_t* qweight, const void* scales, const uint32_t* qzeros, void* y,
                       int M, int N, int K, int group_size, bool zero_point, void* workspace, hipStream_t stream) {
  return zero_point ? launch_zp<true>(x, qweight, scales, qzeros, y, M, N, K, group_size, workspace, stream)
                    : launch_zp<false>(x, qweight, scales, qzeros, y, M, N, K, group_size, workspace, stream);
}

}  // namespace awq
