// C ABI of the W4A16 layer: argument validation, then one launch on the
// caller's stream.  Declarations and the contract of every entry point are in
// include/awq.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/awq.h"
#include "awq_launch.hpp"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_group(int32_t g) { return g == 32 || g == 64 || g == 128 || g == 256; }

// Largest N and K: keeps every per-tile buffer-resource extent and offset of
// the kernels below 2^31 bytes.
constexpr int32_t kMaxDim = 1 << 21;

// The loss product addresses one candidate's group parameters (K / 32 * N
// words at most) through a 32-bit buffer range, with offsets up to one group
// past its end.
bool loss_shape_ok(int32_t N, int32_t K) { return (int64_t)K * N < ((int64_t)1 << 34); }
// The clip search's parameters take 8 bytes per ratio, row and group.
bool clip_shape_ok(int32_t N, int32_t K) { return (int64_t)K * N < ((int64_t)1 << 33); }

// Checks shared by every entry point that reads or writes a packed weight.
int check_weight_shape(int32_t N, int32_t K, int32_t group_size) {
  if (!valid_group(group_size)) return AWQ_ERR_GROUP;
  if (N < 1 || K < 1 || (N & 7) != 0 || N > kMaxDim || K > kMaxDim) return AWQ_ERR_SHAPE;
  if (K % group_size != 0) return AWQ_ERR_GROUP;
  return AWQ_OK;
}

int check_packed(const uint32_t* qweight, const void* scales, const uint32_t* qzeros, int32_t zero_point) {
  if (!qweight || !scales || (zero_point && !qzeros)) return AWQ_ERR_NULL;
  if (!aligned16(qweight) || !aligned16(scales) || (zero_point && !aligned16(qzeros))) return AWQ_ERR_ALIGN;
  return AWQ_OK;
}

int from_hip(hipError_t e) { return e == hipSuccess ? AWQ_OK : AWQ_ERR_HIP; }

}  // namespace

extern "C" {

int awq_pack(const void* w, int32_t N, int32_t K, int32_t group_size, int32_t zero_point, uint32_t* qweight,
             void* scales, uint32_t* qzeros, void* stream) {
  int st = check_weight_shape(N, K, group_size);
  if (st != AWQ_OK) return st;
  if (!w) return AWQ_ERR_NULL;
  st = check_packed(qweight, scales, qzeros, zero_point);
  if (st != AWQ_OK) return st;
  if (!aligned16(w)) return AWQ_ERR_ALIGN;
  return from_hip(awq::launch_pack(w, N, K, group_size, zero_point != 0, qweight, scales, zero_point ? qzeros : nullptr,
                                   static_cast<hipStream_t>(stream)));
}

int awq_dequant(const uint32_t* qweight, const void* scales, const uint32_t* qzeros, void* w_out, int32_t N, int32_t K,
                int32_t group_size, int32_t zero_point, void* stream) {
  int st = check_weight_shape(N, K, group_size);
  if (st != AWQ_OK) return st;
  if (!w_out) return AWQ_ERR_NULL;
  st = check_packed(qweight, scales, qzeros, zero_point);
  if (st != AWQ_OK) return st;
  if (!aligned16(w_out)) return AWQ_ERR_ALIGN;
  return from_hip(awq::launch_dequant(qweight, scales, zero_point ? qzeros : nullptr, w_out, N, K, group_size,
                                      zero_point != 0, static_cast<hipStream_t>(stream)));
}

int awq_gemv(const void* x, const uint32_t* qweight, const void* scales, const uint32_t* qzeros, void* y, int32_t M,
             int32_t N, int32_t K, int32_t group_size, int32_t zero_point, void* stream) {
  int st = check_weight_shape(N, K, group_size);
  if (st != AWQ_OK) return st;
  if (M < 1) return AWQ_ERR_SHAPE;
  if (!x || !y) return AWQ_ERR_NULL;
  st = check_packed(qweight, scales, qzeros, zero_point);
  if (st != AWQ_OK) return st;
  if (!aligned16(x) || !aligned16(y)) return AWQ_ERR_ALIGN;
  if (M > awq::kMaxGemvTokens) return AWQ_ERR_UNSUPPORTED;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  if (M == 1)
    return from_hip(awq::launch_gemv(x, qweight, scales, zero_point ? qzeros : nullptr, y, N, K, group_size,
                                     zero_point != 0, hs));
  return from_hip(awq::launch_gemv_small(x, qweight, scales, zero_point ? qzeros : nullptr, y, M, N, K, group_size,
                                         zero_point != 0, hs));
}

size_t awq_gemm_workspace_bytes(int32_t M, int32_t N, int32_t K, int32_t group_size) {
  if (M < 1 || check_weight_shape(N, K, group_size) != AWQ_OK) return 0;
  return awq::gemm_workspace_bytes(M, N, K);
}

int awq_gemm(const void* x, const uint32_t* qweight, const void* scales, const uint32_t* qzeros, void* y, int32_t M,
             int32_t N, int32_t K, int32_t group_size, int32_t zero_point, void* workspace, size_t workspace_bytes,
             void* stream) {
  int st = check_weight_shape(N, K, group_size);
  if (st != AWQ_OK) return st;
  if (M < 1) return AWQ_ERR_SHAPE;
  if (!x || !y) return AWQ_ERR_NULL;
  st = check_packed(qweight, scales, qzeros, zero_point);
  if (st != AWQ_OK) return st;
  if (!aligned16(x) || !aligned16(y)) return AWQ_ERR_ALIGN;
  const size_t need = awq_gemm_workspace_bytes(M, N, K, group_size);
  if (workspace_bytes < need) return AWQ_ERR_WORKSPACE;
  if (need > 0 && !workspace) return AWQ_ERR_NULL;
  if (need > 0 && !aligned16(workspace)) return AWQ_ERR_ALIGN;
  return from_hip(awq::launch_gemm(x, qweight, scales, zero_point ? qzeros : nullptr, y, M, N, K, group_size,
                                   zero_point != 0, need > 0 ? workspace : nullptr,
                                   static_cast<hipStream_t>(stream)));
}

size_t awq_scale_candidates_workspace_bytes(int32_t M, int32_t N, int32_t K) {
  if (M < 1 || N < 0 || N > kMaxDim || K < 8 || K > kMaxDim || (K & 7) != 0) return 0;
  return awq::scale_candidates_workspace_bytes(M, N, K);
}

int awq_scale_candidates(const void* x, int32_t M, int32_t K, const void* w, int32_t N, int32_t duo,
                         const float* alphas, int32_t count, float* s, void* workspace, size_t workspace_bytes,
                         void* stream) {
  if (M < 1 || K < 8 || K > kMaxDim || (K & 7) != 0) return AWQ_ERR_SHAPE;
  if (count < 1 || count > awq::kMaxScaleCandidates) return AWQ_ERR_SHAPE;
  if (duo && (N < 1 || N > kMaxDim)) return AWQ_ERR_SHAPE;
  if (!x || !alphas || !s || !workspace || (duo && !w)) return AWQ_ERR_NULL;
  if (!aligned16(x) || !aligned16(s) || !aligned16(workspace) || (duo && !aligned16(w))) return AWQ_ERR_ALIGN;
  if (workspace_bytes < awq::scale_candidates_workspace_bytes(M, duo ? N : 0, K)) return AWQ_ERR_WORKSPACE;
  return from_hip(awq::launch_scale_candidates(x, M, K, duo ? w : nullptr, duo ? N : 0, alphas, count, s, workspace,
                                               static_cast<hipStream_t>(stream)));
}

size_t awq_scale_search_workspace_bytes(int32_t count, int32_t M, int32_t N, int32_t K) {
  if (count < 1 || count > awq::kMaxScaleCandidates || M < 1 || N < 8 || K < 8 || N > kMaxDim || K > kMaxDim)
    return 0;
  return awq::scale_search_workspace_bytes(count, M, N, K);
}

int awq_scale_search(const void* x, const void* w, int32_t M, int32_t N, int32_t K, int32_t group_size,
                     int32_t zero_point, const float* alphas, int32_t count, int32_t duo, float* s_best,
                     int32_t* best, double* losses, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_weight_shape(N, K, group_size);
  if (st != AWQ_OK) return st;
  if (M < 1 || count < 1 || count > awq::kMaxScaleCandidates || !loss_shape_ok(N, K)) return AWQ_ERR_SHAPE;
  if (!x || !w || !alphas || !s_best || !best || !workspace) return AWQ_ERR_NULL;
  if (!aligned16(x) || !aligned16(w) || !aligned16(s_best) || !aligned16(workspace) ||
      (reinterpret_cast<uintptr_t>(best) & 3u) != 0 || (reinterpret_cast<uintptr_t>(losses) & 7u) != 0)
    return AWQ_ERR_ALIGN;
  if (workspace_bytes < awq::scale_search_workspace_bytes(count, M, N, K)) return AWQ_ERR_WORKSPACE;
  return from_hip(awq::launch_scale_search(x, w, M, N, K, group_size, zero_point != 0, alphas, count, duo != 0,
                                           s_best, best, losses, workspace, static_cast<hipStream_t>(stream)));
}

size_t awq_scale_loss_workspace_bytes(int32_t count, int32_t M, int32_t N, int32_t K) {
  if (count < 1 || count > 65535 || M < 1 || N < 8 || K < 8 || N > kMaxDim || K > kMaxDim) return 0;
  return awq::scale_loss_workspace_bytes(count, M, N, K);
}

int awq_scale_loss(const void* x, const void* w, const float* s, int32_t count, int32_t M, int32_t N, int32_t K,
                   int32_t group_size, int32_t zero_point, void* workspace, size_t workspace_bytes, double* loss,
                   void* stream) {
  int st = check_weight_shape(N, K, group_size);
  if (st != AWQ_OK) return st;
  if (M < 1 || count < 1 || count > 65535 || !loss_shape_ok(N, K)) return AWQ_ERR_SHAPE;
  if (!x || !w || !s || !workspace || !loss) return AWQ_ERR_NULL;
  if (!aligned16(x) || !aligned16(w) || !aligned16(s) || !aligned16(workspace) ||
      (reinterpret_cast<uintptr_t>(loss) & 7u) != 0)
    return AWQ_ERR_ALIGN;
  if (workspace_bytes < awq::scale_loss_workspace_bytes(count, M, N, K)) return AWQ_ERR_WORKSPACE;
  return from_hip(awq::launch_scale_loss(x, w, s, count, M, N, K, group_size, zero_point != 0, workspace, loss,
                                         static_cast<hipStream_t>(stream)));
}

int awq_scale_columns(const void* src, int32_t rows, int32_t K, const float* s, int32_t divide, void* dst,
                      void* stream) {
  if (rows < 1 || K < 8 || K > kMaxDim || (K & 7) != 0) return AWQ_ERR_SHAPE;
  if (!src || !s || !dst) return AWQ_ERR_NULL;
  if (!aligned16(src) || !aligned16(s) || !aligned16(dst)) return AWQ_ERR_ALIGN;
  return from_hip(awq::launch_scale_columns(src, rows, K, s, divide != 0, dst, static_cast<hipStream_t>(stream)));
}

size_t awq_clip_search_workspace_bytes(int32_t count, int32_t M, int32_t N, int32_t K, int32_t group_size) {
  if (count < 1 || count > awq::kMaxClipCandidates || M < 1 || check_weight_shape(N, K, group_size) != AWQ_OK)
    return 0;
  return awq::clip_search_workspace_bytes(count, M, N, K, group_size);
}

int awq_clip_search(const void* x, const void* w, int32_t M, int32_t N, int32_t K, int32_t group_size,
                    int32_t zero_point, const float* ratios, int32_t count, void* w_clipped, int32_t* choice,
                    void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_weight_shape(N, K, group_size);
  if (st != AWQ_OK) return st;
  if (M < 1 || count < 1 || count > awq::kMaxClipCandidates || !clip_shape_ok(N, K)) return AWQ_ERR_SHAPE;
  if (!x || !w || !ratios || !w_clipped || !workspace) return AWQ_ERR_NULL;
  for (int c = 0; c < count; ++c)
    if (!(ratios[c] > 0.0f && ratios[c] <= 1.0f)) return AWQ_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(w) || !aligned16(w_clipped) || !aligned16(workspace) ||
      (reinterpret_cast<uintptr_t>(choice) & 3u) != 0)
    return AWQ_ERR_ALIGN;
  if (workspace_bytes < awq::clip_search_workspace_bytes(count, M, N, K, group_size)) return AWQ_ERR_WORKSPACE;
  return from_hip(awq::launch_clip_search(x, w, M, N, K, group_size, zero_point != 0, ratios, count, w_clipped, choice,
                                          workspace, static_cast<hipStream_t>(stream)));
}

const char* awq_strerror(int status) {
  switch (status) {
    case AWQ_OK: return "ok";
    case AWQ_ERR_NULL: return "a required pointer is NULL";
    case AWQ_ERR_SHAPE: return "invalid shape: need M >= 1, N >= 1 with N % 8 == 0, K >= 1";
    case AWQ_ERR_GROUP: return "invalid group size: need group_size in {32, 64, 128, 256} dividing K";
    case AWQ_ERR_ALIGN: return "a buffer pointer is not 16-byte aligned";
    case AWQ_ERR_UNSUPPORTED: return "unsupported argument combination for this entry point (awq_gemv takes M <= 8)";
    case AWQ_ERR_WORKSPACE: return "workspace smaller than awq_gemm_workspace_bytes()";
    case AWQ_ERR_HIP: return "the HIP runtime reported an error while launching";
    case AWQ_ERR_SCRATCH:
      return "the shape needs more split-K workspace than awq_gemm_noalloc's fixed scratch "
             "(awq_gemm_noalloc_max_workspace_bytes()); use awq_gemm with a workspace";
    default: return "unknown awq status";
  }
}

}  // extern "C"
