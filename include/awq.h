/*
 * awq.h - C ABI of the MI355X (gfx950) W4A16 group-wise quantized linear layer.
 *
 * The layer is AWQ's 4-bit weight-only linear layer: weights are stored as
 * 4-bit codes with one fp16 scale and one 4-bit zero point per group of
 * consecutive input channels, activations stay fp16, and the layer computes
 * Y = X . W'^T with W' = (q - z) * s.  Sources (web pages, by title and section):
 *   - "AI-Research-SKILLs AWQ 高级使用指南", section 分组大小与零点量化
 *     ("Group Size": a group shares one scale and zero point; 32/128/256,
 *     128 recommended; "Zero-Point": an offset for asymmetric ranges,
 *     zero_point False = symmetric), section WQLinear 内核全景 (GEMM kernel
 *     for batches, GEMV kernel for a single token).
 *   - "Optimization Awq", section "Quantizar seu próprio modelo" (quant_config
 *     = zero_point, q_group_size, w_bit = 4, version GEMM | GEMV) and section
 *     "Integração vLLM" (half-precision activations).
 *
 * Conventions for every entry point
 *   - All buffer pointers are DEVICE pointers on the current HIP device; the
 *     caller allocates and owns them.  The library never allocates, frees or
 *     keeps mutable state of its own between calls, and never synchronizes
 *     the device (awq_gemm's workspace, owned by the caller, is the one
 *     buffer a call hands on to the next; see there).
 *   - fp16 buffers are passed as void* and hold IEEE binary16 values.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued asynchronously; the return value reports argument
 *     validation and launch errors only.  On any error nothing is launched.
 *   - Every pointer must be 16-byte aligned.  Buffers must not overlap.
 *   - Shapes: N (output features) >= 1 and a multiple of 8; K (input
 *     features) >= 1 and a multiple of group_size; N, K <= 2^21;
 *     group_size in {32, 64, 128, 256}; M (tokens) >= 1.  G = K / group_size.
 *   - Weights must be finite; results for NaN/Inf weights are unspecified.
 *
 * Storage layout of a packed weight (the pages fix none; this one is ours):
 *   qweight  uint32 [N][K/8]  word (n, j) holds the 4-bit codes of channels
 *            k = 8j .. 8j+7 of row n: channel 8j+c sits at bit
 *            16*(c & 1) + 4*(c >> 1), i.e. the low halfword holds the even
 *            channels 0,2,4,6 and the high halfword the odd ones 1,3,5,7.
 *   scales   fp16   [N/8][G][8]  scale of row 8o+i, group j at (o, j, i):
 *            the scales of one octet of rows are contiguous, 8 per group.
 *   qzeros   uint32 [N/8][G]     zero point of row 8o+i, group j in bits
 *            4i..4i+3 of word (o, j).  Only with zero_point != 0; the
 *            symmetric format has the implicit zero point 8 and no qzeros.
 */
#ifndef AWQ_MI355X_AWQ_H
#define AWQ_MI355X_AWQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
enum awq_status {
  AWQ_OK = 0,
  AWQ_ERR_NULL = -1,        /* a required pointer is NULL                      */
  AWQ_ERR_SHAPE = -2,       /* M, N or K out of range / not a multiple         */
  AWQ_ERR_GROUP = -3,       /* group_size not in {32,64,128,256} or K % g != 0  */
  AWQ_ERR_ALIGN = -4,       /* a pointer is not 16-byte aligned                */
  AWQ_ERR_UNSUPPORTED = -5, /* valid arguments this entry point does not take  */
  AWQ_ERR_WORKSPACE = -6,   /* workspace smaller than awq_gemm_workspace_bytes */
  AWQ_ERR_HIP = -7,         /* the HIP runtime reported an error at launch     */
  AWQ_ERR_SCRATCH = -8      /* awq_gemm_noalloc: shape needs more than its scratch */
};

/*
 * awq_pack - quantize fp16 weights group-wise to 4 bits and store them.
 *
 * Defines the quantizer Q ("AI-Research-SKILLs AWQ 高级使用指南", section
 * 分组大小与零点量化; codes q = clamp(round(w/s) + z, 0, 15)).  For each row n
 * and group j (channels j*g .. j*g+g-1), all in IEEE fp32 with
 * round-half-to-even:
 *   zero_point != 0:  r = max(max - min, 1e-5);  s = fp16(r / 15);
 *                     z = clamp(rne(-min / s), 0, 15)
 *   zero_point == 0:  a = max(max |w|, 1e-5);    s = fp16(a / 7);  z = 8
 *   q = clamp(rne(w / s) + z, 0, 15)   (correctly rounded fp32 division by
 *                                       the fp16-rounded scale s)
 *
 * w        in   fp16  [N][K], row-major.
 * qweight  out  uint32 [N][K/8]; scales out fp16 [N/8][G][8];
 * qzeros   out  uint32 [N/8][G] when zero_point != 0 (may be NULL otherwise).
 * Deterministic: the output is bit-identical for identical input.
 */
int awq_pack(const void* w, int32_t N, int32_t K, int32_t group_size, int32_t zero_point,
             uint32_t* qweight, void* scales, uint32_t* qzeros, void* stream);

/*
 * awq_dequant - decode a packed weight to fp16: w_out[n][k] = fp16((q - z) * s),
 * rounded once to nearest-even.  A test and inspection aid; not on the hot path.
 * w_out out fp16 [N][K].
 */
int awq_dequant(const uint32_t* qweight, const void* scales, const uint32_t* qzeros, void* w_out,
                int32_t N, int32_t K, int32_t group_size, int32_t zero_point, void* stream);

/*
 * awq_gemv - single- and few-token quantized linear layer, Y = X . W'^T.
 *
 * The GEMV variants ("AI-Research-SKILLs AWQ 高级使用指南", section WQLinear 内核全景,
 * WQLinear_GEMV: single-token generation, batch size 1; WQLinear_GEMVFast:
 * the fastest few-token decoding; "Optimization Awq", section "Backends de
 * kernel": GEMV for batch size 1).  One token runs on the single-token
 * kernel (fp32 dot products); 2-8 tokens on the few-token kernel (the
 * products on the fp16 matrix cores from exact q - z, the group scale applied
 * to each 32-channel fp32 sum).
 * X in fp16 [M][K] with 1 <= M <= 8 (AWQ_ERR_UNSUPPORTED above; awq_gemm
 * takes any M); Y out fp16 [M][N].  Accumulation is fp32, the output rounded
 * once to fp16.  Each output meets |y - y_ref| <= 1e-3 * sum_k |x_k w'_k|
 * against the exact product, and is bit-reproducible run to run.
 */
int awq_gemv(const void* x, const uint32_t* qweight, const void* scales, const uint32_t* qzeros,
             void* y, int32_t M, int32_t N, int32_t K, int32_t group_size, int32_t zero_point,
             void* stream);

/*
 * awq_gemm - batched quantized linear layer, Y = X . W'^T, any M >= 1.
 *
 * The GEMM variant ("AI-Research-SKILLs AWQ 高级使用指南", section WQLinear 内核全景,
 * WQLinear_GEMM: general matrix multiplication for batches).  Weights are
 * decoded to fp16 in registers and multiplied on the fp16 matrix cores with
 * fp32 accumulation; the output is rounded once to fp16.
 * X in fp16 [M][K]; Y out fp16 [M][N].  Same accuracy contract as awq_gemv.
 * Deterministic run to run.  Up to 8 tokens it runs awq_gemv's kernels (the
 * same bits as awq_gemv) and needs no workspace.
 *
 * workspace: device scratch of at least awq_gemm_workspace_bytes(M, N, K,
 * group_size) bytes, 16-byte aligned, owned by the caller (may be NULL when
 * that size is 0).  For small M (9-64, except 33-64 tokens on layers with
 * N >= 8192 and 49-64 tokens on layers with K >= 8192, which take the
 * matrix-core path below) the K dimension is split across workgroups: the
 * workspace then starts with a 512 KiB region of 32-bit per-tile counters,
 * followed by fp32 partial tiles, and the last workgroup
 * of a tile to finish adds the partials in a fixed order (the result does not
 * depend on which one finishes last).  The counter region must be ZERO when
 * the buffer is first used (e.g. allocated zero-filled); every call returns
 * it to zero, so one buffer serves any number of calls of any shape in
 * stream order.  Calls that may run concurrently (different streams) need
 * separate workspaces.  For larger M with few output tiles (M up to about a
 * thousand on 4096-wide layers, and the 33-64 token cases above), K is
 * split as well: fp32 partial products [slices][M][N] follow the
 * counter region and a second kernel adds them in a fixed order.
 */
int awq_gemm(const void* x, const uint32_t* qweight, const void* scales, const uint32_t* qzeros,
             void* y, int32_t M, int32_t N, int32_t K, int32_t group_size, int32_t zero_point,
             void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace awq_gemm needs for this shape (0 when it needs none). */
size_t awq_gemm_workspace_bytes(int32_t M, int32_t N, int32_t K, int32_t group_size);

/*
 * awq_gemm_noalloc - awq_gemm for callers that cannot allocate: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * Same arguments, validation, kernels and results (bit for bit) as awq_gemm,
 * but the split-K workspace is a fixed array owned by the library: a
 * file-scope device array of awq_gemm_noalloc_max_workspace_bytes() bytes
 * (64 MiB) that each GPU the library runs on holds until the process ends.
 * The call allocates and frees nothing.  On the first call on a device the
 * array's address is looked up and its counter region is cleared by a
 * kernel on `stream`; every call leaves it zero again.
 * Shapes whose awq_gemm_workspace_bytes() exceeds the array return
 * AWQ_ERR_SCRATCH and launch nothing (e.g. 1536 tokens on a 28672 -> 8192
 * layer); every shape up to 128 tokens on the Llama-7B and 70B-shaped
 * layers fits.  All calls on one GPU share its array: calls that may
 * overlap on one GPU (different streams, or different host threads without
 * ordering) race and give wrong results; order them on one stream.
 */
int awq_gemm_noalloc(const void* x, const uint32_t* qweight, const void* scales, const uint32_t* qzeros, void* y,
                     int32_t M, int32_t N, int32_t K, int32_t group_size, int32_t zero_point, void* stream);
size_t awq_gemm_noalloc_max_workspace_bytes(void);

/*
 * awq_scale_candidates - candidate per-input-channel scales for the
 * activation-aware scale search.
 *
 * "AI-Research-SKILLs AWQ 高级使用指南", section 算法原理: salient channels are
 * found from the activation distribution and scaled up before quantization;
 * "AWQ Activation-aware Weight Quantization (Lin 2023年)": activation
 * statistics and per-channel scaling; section 自定义校准策略 (校准参数全景):
 * duo_scaling scales weights and activations.  The pages give no candidate
 * family; this one is
 *   a_k = max(mean_m |x[m][k]|, 1e-4),   s[c][k] = a_k ^ alphas[c]
 * (alphas[c] == 0 gives exactly 1), or with duo != 0
 *   b_k = max(mean_n |w[n][k]|, 1e-4),   s[c][k] = a_k ^ alphas[c] / b_k ^ (1 - alphas[c])
 * (fp32; each mean is an fp32 sum in row order divided by the row count).
 * x       in   fp16 [M][K] calibration activations (device).
 * w, N    in   fp16 [N][K] weights (device), read only with duo != 0 (may be
 *              NULL, and N is ignored, otherwise).
 * alphas  in   HOST array of `count` exponents, 1 <= count <= 64.
 * s       out  fp32 [count][K] (device).
 * workspace: device scratch of awq_scale_candidates_workspace_bytes(M,
 * duo ? N : 0, K) bytes, 16-byte aligned, contents not needed before or
 * after the call.  K must be a multiple of 8.  Deterministic.
 */
int awq_scale_candidates(const void* x, int32_t M, int32_t K, const void* w, int32_t N, int32_t duo,
                         const float* alphas, int32_t count, float* s, void* workspace, size_t workspace_bytes,
                         void* stream);
size_t awq_scale_candidates_workspace_bytes(int32_t M, int32_t N, int32_t K);

/*
 * awq_scale_search - the activation-aware scale search of one linear layer
 * ("AI-Research-SKILLs AWQ 高级使用指南", section 算法原理: choose the
 * per-channel scale s that makes L(s) = ||Q(W * s)(s^-1 * X) - W * X||
 * small): the candidates of awq_scale_candidates (duo scaling with duo != 0),
 * the loss of each as awq_scale_loss computes it, and the choice of the
 * first candidate with the smallest loss (a NaN loss is never chosen), all on
 * the device: nothing is copied to the host and the call does not wait.
 * x       in   fp16 [M][K] calibration activations.
 * w       in   fp16 [N][K] unquantized weights.
 * alphas  in   HOST array of `count` exponents, 1 <= count <= 64.
 * s_best  out  fp32 [K] (device): the chosen scale vector.
 * best    out  int32 [1] (device): the index of the chosen candidate.
 * losses  out  fp64 [count] (device, 8-byte aligned), or NULL.
 * workspace: device scratch of awq_scale_search_workspace_bytes(count, M, N,
 * K) bytes, 16-byte aligned; contents not needed before or after.
 * Same shape rules as awq_scale_loss; deterministic.
 */
int awq_scale_search(const void* x, const void* w, int32_t M, int32_t N, int32_t K, int32_t group_size,
                     int32_t zero_point, const float* alphas, int32_t count, int32_t duo, float* s_best,
                     int32_t* best, double* losses, void* workspace, size_t workspace_bytes, void* stream);
size_t awq_scale_search_workspace_bytes(int32_t count, int32_t M, int32_t N, int32_t K);

/*
 * awq_scale_loss - reconstruction error of the activation-aware scaling,
 *   loss[c] = L(s_c) = || (X diag(s_c)^-1) . Q(fp16(W diag(s_c)))'^T - X . W^T ||_F
 * ("AI-Research-SKILLs AWQ 高级使用指南", section 算法原理, the objective
 * L(s) = ||Q(W * s)(s^-1 * X) - W * X||), for `count` candidate scale vectors.
 * Q(.)' is the quantize-then-decode of awq_pack (same group size and zero
 * point mode; W * s is an fp32 product rounded to fp16).
 * x     in   fp16 [M][K] calibration activations.
 * w     in   fp16 [N][K] unquantized weights.
 * s     in   fp32 [count][K], every entry finite and > 0 (not checked).
 * loss  out  fp64 [count] (device, 8-byte aligned).
 * workspace: device scratch of awq_scale_loss_workspace_bytes(count, M, N, K)
 * bytes (count * N * K / 8 for the groups' scales and zero points of every
 * candidate, count * M * K * 2 for the activations scaled by each candidate,
 * plus per-wave sums), 16-byte aligned; contents not needed before or after.
 * Shapes: as awq_pack, and K * N < 2^34.
 * Computed as || (X diag(s)^-1) (Q(W s)' - W s)^T ||: the scaled weight error
 * is formed next to the matrix cores (never stored) in fp32 from the exact
 * code times scale, rounded once to fp16 (relative 2^-11), the scaled
 * activations are rounded to fp16 (relative 2^-11), the product accumulates
 * in fp32, its squares are summed in fp32 per wave (128 x 64 outputs) and the
 * waves' sums in fp64: |loss - L| <= 1e-3 * L.  The codes
 * are awq_pack's codes of fp16(W s) bit for bit.  Deterministic.
 */
int awq_scale_loss(const void* x, const void* w, const float* s, int32_t count, int32_t M, int32_t N, int32_t K,
                   int32_t group_size, int32_t zero_point, void* workspace, size_t workspace_bytes, double* loss,
                   void* stream);
size_t awq_scale_loss_workspace_bytes(int32_t count, int32_t M, int32_t N, int32_t K);

/*
 * awq_scale_columns - apply per-input-channel scales: dst[r][k] =
 * fp16(src[r][k] * s[k]) (divide == 0, the weights W * s) or
 * fp16(src[r][k] / s[k]) (divide != 0, the activations s^-1 * X); fp32
 * product or correctly rounded fp32 quotient, one rounding to fp16
 * ("AI-Research-SKILLs AWQ 高级使用指南", section 算法原理: the weights are
 * scaled by s and the activations by s^-1).
 * src, dst  fp16 [rows][K] (may be the same buffer); s fp32 [K] > 0.
 * K must be a multiple of 8.
 */
int awq_scale_columns(const void* src, int32_t rows, int32_t K, const float* s, int32_t divide, void* dst,
                      void* stream);

/*
 * awq_clip_search - weight clipping for the quantizer (apply_clip:
 * "AI-Research-SKILLs AWQ 高级使用指南", section 自定义校准策略 (校准参数全景), clip the
 * weights to reduce the effect of outliers on the quantization error).  The
 * pages give no rule; this one: for each ratio r in `ratios` every group's
 * range shrinks to [r*min, r*max] (zero_point != 0) or [-r*amax, r*amax]
 * (fp32 products) and its weights are clamped to it (fp32, then fp16); the
 * error of group (n, j) is
 *   err(n, j, r) = sum_m ( sum_{k in group j} x[m][k] (Dq(Q(clip_r(W)))[n][k] - w[n][k]) )^2
 * (Q and Dq as in awq_pack / awq_dequant).  Each group keeps the first ratio
 * with the smallest error, and w_clipped holds the weights clamped with it;
 * packing w_clipped with awq_pack gives the clipped quantization.
 * x          in   fp16 [M][K] calibration activations.
 * w          in   fp16 [N][K] weights.
 * ratios     in   HOST array of `count` ratios, each in (0, 1], 1 <= count <= 64.
 * w_clipped  out  fp16 [N][K].
 * choice     out  int32 [N][K/group_size]: index of the chosen ratio (may be NULL).
 * workspace: device scratch of awq_clip_search_workspace_bytes(count, M, N,
 * K, group_size) bytes (count * N * K / group_size * 8 for every ratio's
 * group scales, zero points and bounds, plus the per-group partial errors),
 * 16-byte aligned; contents not needed before or after.
 * Shapes: as awq_pack, and K * N < 2^33.
 * The weight errors are formed next to the matrix cores (never stored) and
 * rounded to fp16, the products accumulate in fp32 (relative error ~1e-3);
 * a ratio whose error is within that of the best may be chosen instead.
 * Deterministic.
 */
int awq_clip_search(const void* x, const void* w, int32_t M, int32_t N, int32_t K, int32_t group_size,
                    int32_t zero_point, const float* ratios, int32_t count, void* w_clipped, int32_t* choice,
                    void* workspace, size_t workspace_bytes, void* stream);
size_t awq_clip_search_workspace_bytes(int32_t count, int32_t M, int32_t N, int32_t K, int32_t group_size);

/* Static, NUL-terminated description of a status code. */
const char* awq_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* AWQ_MI355X_AWQ_H */
