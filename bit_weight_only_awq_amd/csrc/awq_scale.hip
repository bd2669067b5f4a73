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
// L(s) is evaluated as || X e^T ||_F with e = Q(W s) s^-1 - W (built by
// scale_error_kernel next to the quantizer): the same quantity, one dense
// product instead of two.  The product runs on the fp16 matrix cores with fp32
// accumulation; the squares are summed per tile and the tiles are added in a
// fixed order in fp64 (deterministic).
#include "awq_device.hpp"
#include "awq_launch.hpp"

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
      out[c] = (_Float16)(divide ? (float)h[c] / sc : (float)h[c] * sc);
    }
    dst[i] = __builtin_bit_cast(u32x4, out);
  }
}

// ---------------------------------------------------------------------------
// Sum of squares of X e_c^T.
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

// Workgroup of WM x WN waves; tile (32 WM WN) x (32 WM WN) with every wave
// loading 32 rows of each operand: 2 x 2 waves of 64 x 64 (128 x 128 tile) or
// 2 x 4 waves of 128 x 64 (256 x 256 tile), v_mfma_f32_32x32x16_f16; grid
// (tiles, candidates).  Both operands stream from HBM into LDS by
// buffer-to-LDS loads, double-buffered, one barrier per K step.  Rows past M
// or N read as zero and add nothing to the sum.  Output: the fp64 sum of the
// squares of the tile's outputs (each square and the per-lane sums in fp32,
// the wave and workgroup sums in a fixed order).
//
// GROUPED: the squares are taken per group of g input channels instead (the
// output error of each weight group, for the clipping search): at every group
// boundary each wave adds the squares of its accumulators over its rows, per
// column, writes them to gpart[c][tm][wave row half][group][n] and restarts
// its accumulators from zero.
template <int WM, int WN, bool KTAIL, bool GROUPED>
__global__ __launch_bounds__(WM * WN * 64) void sumsq_gemm_kernel(const _Float16* __restrict__ X,
                                                                  const _Float16* __restrict__ E_all, int M, int N,
                                                                  int K, int tiles_m, double* __restrict__ partial,
                                                                  int gshift, float* __restrict__ gpart) {
  constexpr int NW = WM * WN;
  constexpr int T = 32 * NW;             // tile rows of X and of E
  constexpr int AM = T / WM / 32;        // 32x32 MFMA tiles per wave along M
  constexpr int AN = T / WN / 32;        // ... along N
  constexpr int OP = T * TK * 2;         // bytes of one operand tile
  // the two buffers of each operand are separate arrays, so the compiler can
  // tell them apart and does not make reads of one wait for the loads into
  // the other
  __shared__ __attribute__((aligned(1024))) char lx0[OP], lx1[OP], le0[OP], le1[OP];
  __shared__ double wsum[NW];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  // (tile, candidate) from the workgroup's place in an XCD-contiguous order:
  // the row tiles of one column band of a candidate's E run on one XCD and
  // share its L2, so E is fetched once per XCD rather than once per row tile
  const int lin = xcd_contiguous_tile(blockIdx.x + blockIdx.y * gridDim.x, gridDim.x * gridDim.y);
  const int tile = lin % gridDim.x, cand = lin / gridDim.x;
  const int tm = tile % tiles_m, tn = tile / tiles_m;
  const int m0 = tm * T, n0 = tn * T;
  const _Float16* E = E_all + (size_t)cand * N * K;
  const int rows_m = min(T, M - m0), rows_n = min(T, N - n0);
  const int nsteps = (K + TK - 1) / TK;

  const __amdgpu_buffer_rsrc_t rx = rsrc(X + (size_t)m0 * K, (uint32_t)rows_m * K * 2);
  const __amdgpu_buffer_rsrc_t re = rsrc(E + (size_t)n0 * K, (uint32_t)rows_n * K * 2);

  // wave w fills rows 32 w .. 32 w + 31 of both tiles with 4 loads of 8 rows
  // x 128 B each; lane l of load j writes slot l of that 1 KiB run: row
  // 32 w + 8 j + l / 8, physical chunk l % 8, holding the logical chunk that
  // swizzles there (the swizzle is an involution)
  int chunk[4];
  uint32_t off[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = 32 * wave + 8 * j + (lane >> 3);
    chunk[j] = swz_chunk(row, lane & 7);
    off[j] = (uint32_t)row * K * 2 + chunk[j] * 16;
  }
  // `buf` is a constant at every call site (the K loop below is unrolled by two)
  auto load = [&](int step, int buf) {
    char* dx = (buf ? lx1 : lx0) + wave * 4096;
    char* de = (buf ? le1 : le0) + wave * 4096;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // the step sits in the scalar offset, outside the hardware's range
      // check: a prefetch past the last step takes the out-of-range lane offset
      uint32_t o = step < nsteps ? off[j] : kOutOfRange;
      if constexpr (KTAIL) {  // channels past K of the last step load as zero
        if (step * TK + 8 * chunk[j] >= K) o = kOutOfRange;
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (__attribute__((address_space(3))) void*)(dx + 1024 * j), 16, o,
                                               step * TK * 2, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(re, (__attribute__((address_space(3))) void*)(de + 1024 * j), 16, o,
                                               step * TK * 2, 0, 0);
    }
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

  // per-group flush (GROUPED): squares per column over this wave's rows
  const int G = K >> gshift;
  float* gout = GROUPED ? gpart + (((size_t)cand * tiles_m + tm) * WM + (wave % WM)) * G * N : nullptr;
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
      // lanes l and l + 32 hold the two row halves of column l % 32
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
      if constexpr (GROUPED) {
        const int kend = step * TK + (ks + 1) * 16;  // channels done after this slice
        if ((kend & ((1 << gshift) - 1)) == 0 && kend <= K) flush((kend >> gshift) - 1);
      }
    }
  };

  // Two steps per trip; the scheduling barriers keep each step's loads ahead
  // of the multiplies that hide their latency.  Loads of a step past the end
  // read zero (out-of-range lane offset) and land in a buffer no one reads
  // again.
  load(0, 0);
  __syncthreads();
  int step = 0;
  for (; step + 1 < nsteps; step += 2) {
    load(step + 1, 1);
    __builtin_amdgcn_sched_barrier(0);
    compute(0, step);
    __syncthreads();
    load(step + 2, 0);
    __builtin_amdgcn_sched_barrier(0);
    compute(1, step + 1);
    __syncthreads();
  }
  if (step < nsteps) compute(0, step);
  if constexpr (GROUPED) return;

  float ss = 0.0f;
#pragma unroll
  for (int a = 0; a < AM; ++a)
#pragma unroll
    for (int b = 0; b < AN; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) ss += acc[a][b][r] * acc[a][b][r];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
  if (lane == 0) wsum[wave] = (double)ss;
  __syncthreads();
  if (t == 0) {
    double v = wsum[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) v += wsum[w];
    partial[(size_t)cand * gridDim.x + tile] = v;
  }
}

// Tile edge of the loss product: 256 (8 waves) once M fills it, else 128.
int loss_tile(int M) { return M > 128 ? 256 : 128; }

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

// The loss product: whole-tile sums (scale search) or per-group sums (clip search).
static hipError_t launch_sumsq(const _Float16* x, const _Float16* e, int M, int N, int K, int T, int tiles_m,
                               dim3 grid, double* partial, int gshift, float* gpart, bool grouped,
                               hipStream_t stream) {
  const bool tail = K % TK != 0;
#define AWQ_SUMSQ(WM_, WN_, TAIL_, GR_)                                                                          \
  hipLaunchKernelGGL((sumsq_gemm_kernel<WM_, WN_, TAIL_, GR_>), grid, dim3(WM_ * WN_ * 64), 0, stream, x, e, M, N, \
                     K, tiles_m, partial, gshift, gpart)
  if (T == 256) {
    if (grouped) {
      if (tail) AWQ_SUMSQ(2, 4, true, true); else AWQ_SUMSQ(2, 4, false, true);
    } else {
      if (tail) AWQ_SUMSQ(2, 4, true, false); else AWQ_SUMSQ(2, 4, false, false);
    }
  } else {
    if (grouped) {
      if (tail) AWQ_SUMSQ(2, 2, true, true); else AWQ_SUMSQ(2, 2, false, true);
    } else {
      if (tail) AWQ_SUMSQ(2, 2, true, false); else AWQ_SUMSQ(2, 2, false, false);
    }
  }
#undef AWQ_SUMSQ
  return hipGetLastError();
}

size_t scale_loss_workspace_bytes(int count, int M, int N, int K) {
  const int T = loss_tile(M);
  const size_t tiles = (size_t)((M + T - 1) / T) * ((N + T - 1) / T);
  return align256((size_t)count * N * K * 2) + align256((size_t)count * tiles * 8);
}

hipError_t launch_scale_loss(const void* x, const void* w, const float* s, int count, int M, int N, int K,
                             int group_size, bool zero_point, void* workspace, double* loss, hipStream_t stream) {
  const int T = loss_tile(M);
  const int tiles_m = (M + T - 1) / T, tiles_n = (N + T - 1) / T;
  char* ws = static_cast<char*>(workspace);
  _Float16* e = reinterpret_cast<_Float16*>(ws);
  double* partial = reinterpret_cast<double*>(ws + align256((size_t)count * N * K * 2));
  hipError_t err = launch_scale_error(w, s, count, N, K, group_size, zero_point, e, stream);
  if (err != hipSuccess) return err;
  const dim3 grid(tiles_m * tiles_n, count);
  err = launch_sumsq(static_cast<const _Float16*>(x), e, M, N, K, T, tiles_m, grid, partial, 0, nullptr, false, stream);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(loss_finalize_kernel, dim3(count), dim3(256), 0, stream, partial, tiles_m * tiles_n, loss);
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

// Per-group partial errors: part[c][tm][h][j][n], h the two row halves of a tile.
size_t clip_search_workspace_bytes(int count, int M, int N, int K, int group_size) {
  const int T = loss_tile(M);
  const size_t tiles_m = (M + T - 1) / T;
  return align256((size_t)count * N * K * 2) + align256((size_t)count * tiles_m * 2 * (K / group_size) * N * 4);
}

hipError_t launch_clip_search(const void* x, const void* w, int M, int N, int K, int group_size, bool zero_point,
                              const float* ratios, int count, void* w_out, int32_t* choice, void* workspace,
                              hipStream_t stream) {
  const int T = loss_tile(M);
  const int tiles_m = (M + T - 1) / T, tiles_n = (N + T - 1) / T;
  char* ws = static_cast<char*>(workspace);
  _Float16* e = reinterpret_cast<_Float16*>(ws);
  float* gpart = reinterpret_cast<float*>(ws + align256((size_t)count * N * K * 2));
  ClipRatios r;
  for (int c = 0; c < kMaxClipCandidates; ++c) r.v[c] = c < count ? ratios[c] : 1.0f;
  hipError_t err = launch_clip_error(w, r, count, N, K, group_size, zero_point, e, stream);
  if (err != hipSuccess) return err;
  err = launch_sumsq(static_cast<const _Float16*>(x), e, M, N, K, T, tiles_m, dim3(tiles_m * tiles_n, count), nullptr,
                     log2_group(group_size), gpart, true, stream);
  if (err != hipSuccess) return err;
  // without a caller's choice buffer the choices go to the start of the
  // workspace: the weight errors there are dead once the product has run
  int32_t* ch = choice ? choice : reinterpret_cast<int32_t*>(ws);
  return launch_clip_apply(w, gpart, tiles_m * 2, r, count, N, K, group_size, zero_point, w_out, ch, stream);
}

}  // namespace awq
