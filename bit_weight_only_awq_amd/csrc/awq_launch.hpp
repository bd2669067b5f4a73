// Host-side launchers of the gfx950 kernels.  Arguments are validated by the
// C ABI layer before any of these is called; each returns hipGetLastError()
// after enqueueing its kernel(s) on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace awq {

hipError_t launch_pack(const void* w, int N, int K, int group_size, bool zero_point, uint32_t* qweight,
                       void* scales, uint32_t* qzeros, hipStream_t stream);

hipError_t launch_dequant(const uint32_t* qweight, const void* scales, const uint32_t* qzeros, void* w_out,
                          int N, int K, int group_size, bool zero_point, hipStream_t stream);

// One token (awq_gemv.hip).
hipError_t launch_gemv(const void* x, const uint32_t* qweight, const void* scales, const uint32_t* qzeros,
                       void* y, int N, int K, int group_size, bool zero_point, hipStream_t stream);

// 2 <= M <= kMaxGemvTokens tokens (awq_gemv_small.hip).
constexpr int kMaxGemvTokens = 8;
hipError_t launch_gemv_small(const void* x, const uint32_t* qweight, const void* scales, const uint32_t* qzeros,
                             void* y, int M, int N, int K, int group_size, bool zero_point, hipStream_t stream);

// Workspace bytes launch_gemm needs for an M x N x K product (0: none).
size_t gemm_workspace_bytes(int M, int N, int K);
// Bytes of the per-tile counter region at the start of every non-empty
// workspace (the part that must be zero when a workspace is first used).
size_t gemm_counter_bytes();

// `workspace` holds gemm_workspace_bytes(M, N, K) bytes whose leading
// per-tile counters are zero; the call leaves them zero again.
hipError_t launch_gemm(const void* x, const uint32_t* qweight, const void* scales, const uint32_t* qzeros,
                       void* y, int M, int N, int K, int group_size, bool zero_point, void* workspace,
                       hipStream_t stream);

// Candidate scales for the activation-aware scale search (at most
// kMaxScaleCandidates exponents per call; `alphas` is a host array).
constexpr int kMaxScaleCandidates = 64;
// With w != NULL (duo scaling) the candidates also divide by a weight
// statistic of w [N][K]; N is ignored otherwise.
size_t scale_candidates_workspace_bytes(int M, int N, int K);
hipError_t launch_scale_candidates(const void* x, int M, int K, const void* w, int N, const float* alphas, int count,
                                   float* s, void* workspace, hipStream_t stream);
// The whole search: candidates, losses, and the first candidate with the
// smallest loss (index to best[0], its scales to s_best).
size_t scale_search_workspace_bytes(int count, int M, int N, int K);
hipError_t launch_scale_search(const void* x, const void* w, int M, int N, int K, int group_size, bool zero_point,
                               const float* alphas, int count, bool duo, float* s_best, int32_t* best, double* losses,
                               void* workspace, hipStream_t stream);

// Group parameters of fp16(w[n][k] * s[c][k]) for each candidate c:
// gp[c][j][n] = fp16 scale bits | zero point << 16 (4 bytes each).
hipError_t launch_scale_group_params(const void* w, const float* s, int count, int N, int K, int group_size,
                                     bool zero_point, void* gp, hipStream_t stream);

// dst = fp16(src * s) or fp16(src / s), s per column (input channel).
hipError_t launch_scale_columns(const void* src, int rows, int K, const float* s, bool divide, void* dst,
                                hipStream_t stream);

// Candidate clipping ratios, passed by value to the kernels.
constexpr int kMaxClipCandidates = 64;
struct ClipRatios {
  float v[kMaxClipCandidates];
};

// Group parameters of the clipped weights for each ratio c:
// gp[c][j][n] = {fp16 scale bits | zero point << 16, fp16 lower bound bits |
// fp16 upper bound bits << 16} (8 bytes each).
hipError_t launch_clip_group_params(const void* w, const ClipRatios& ratios, int count, int N, int K, int group_size,
                                    bool zero_point, void* gp, hipStream_t stream);
// Per group: the ratio with the smallest summed partial error to choice[n][j]
// (device, [N][K / group_size], always written), then the clipped weights to w_out.
hipError_t launch_clip_apply(const void* w, const float* part, int parts, const ClipRatios& ratios, int count, int N,
                             int K, int group_size, bool zero_point, void* w_out, int32_t* choice, hipStream_t stream);
// Clip search: errors of every ratio, then choice and clipped weights.
size_t clip_search_workspace_bytes(int count, int M, int N, int K, int group_size);
hipError_t launch_clip_search(const void* x, const void* w, int M, int N, int K, int group_size, bool zero_point,
                              const float* ratios, int count, void* w_out, int32_t* choice, void* workspace,
                              hipStream_t stream);

// loss[c] = || X e_c^T ||_F for each candidate scale vector s[c].
size_t scale_loss_workspace_bytes(int count, int M, int N, int K);
hipError_t launch_scale_loss(const void* x, const void* w, const float* s, int count, int M, int N, int K,
                             int group_size, bool zero_point, void* workspace, double* loss, hipStream_t stream);

}  // namespace awq
