"""CPU oracle for the W4A16 group-wise AWQ linear layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call this
module: only the test-suite, the smoke check in ``__graft_entry__`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table or
constant with the HIP library and imports nothing from it.

What it computes, and where that comes from
-------------------------------------------
Sources (web pages, cited by title and section):

* [P5] "AI-Research-SKILLs AWQ 高级使用指南" (lshu.cn): section "算法原理"
  (the reconstruction objective L(s)), section "分组大小与零点量化" with its
  two sub-parts "分组大小 Group Size" (weights share one scale/zero per group;
  sizes 32/128/256, 128 the default) and "零点量化 Zero-Point" (a zero point
  is an offset for asymmetric weight ranges; ``zero_point: False`` is the
  symmetric case), section "WQLinear 内核全景" (GEMM for batches, GEMV for a
  single token).
* [P2] "Optimization Awq" (skillsdirectory.com): section "Quantizar seu
  próprio modelo" (``quant_config`` = zero_point, q_group_size, w_bit=4,
  version) and section "Integração vLLM" (activations in half precision).
* [P4] "AWQ Activation-aware Weight Quantization (Lin 2023年)" (jisaku.com),
  section "主な特徴・仕組み": 4-bit weight-only, group-wise quantization.

The pages give neither a formula for the quantizer nor a storage layout.  The
readings taken here (every one is listed with its reason in the design notes
of the repository):

1. Groups are ``g`` consecutive input channels (K) of one output row of the
   ``nn.Linear`` weight W[N, K]; Y = X . W'^T.
2. zero_point=True (asymmetric, min-max):
   r = max(mx - mn, 1e-5); s = f16(r / 15); z = clamp(rne(-mn / s), 0, 15).
3. zero_point=False (symmetric):
   a = max(max|w|, 1e-5); s = f16(a / 7); z = 8 (implicit, not stored).
4. q = clamp(rne(w / s) + z, 0, 15); decoded weight w' = (q - z) * s.
   All of 2-4 is IEEE binary32 arithmetic with round-half-to-even, the scale
   rounded to binary16 before z and q are formed, every division a correctly
   rounded fp32 division.
5. Storage (our layout):
   qweight u32 [N][K/8]: bits 4i..4i+3 of word (n, j) hold the code of
   k = 8j + PACK_ORDER[i]; scales fp16 [N/8][G][8]: element (o, j, i) is the
   scale of row 8o + i, group j; qzeros u32 [N/8][G]: bits 4i..4i+3 of word
   (o, j) hold the zero point of row 8o + i, group j.
6. Y_ref = X . W'^T and D = |X| . |W'|^T in fp64.  Products of an fp16 x and
   an exact w' need at most 27 significant bits, so each product is exact in
   fp64; only the summation rounds.
7. L(s) = || (X diag(s)^-1) . Dq(f16(W diag(s)))^T - X . W^T ||_F in fp64.
8. Activation-aware scale search ([P5] "算法原理": salient channels are found
   from the activation distribution and scaled before quantization; [P4]
   "主な特徴・仕組み": activation statistics, per-channel scaling).  The pages
   give no candidate family; the reading taken is s = a^alpha with
   a_k = max(mean_m |x_mk|, 1e-4) and alpha on a grid in [0, 1); the search
   keeps the candidate with the smallest L(s) (the first one on ties).
   With ``duo_scaling`` ([P5] "自定义校准策略 (校准参数全景)": scale weights and
   activations) the candidate also divides by a weight statistic of the same
   channel: s = a^alpha / b^(1 - alpha), b_k = max(mean_n |w_nk|, 1e-4), the
   plainest reading that uses both (alpha = 1 is the activation-only a).
9. Weight clipping ([P5] "自定义校准策略" (校准参数全景), ``apply_clip``: clip the weights to
   further reduce the effect of outliers on the quantization error).  The pages
   give no rule; the reading taken: each group tries ratios r in (0, 1]; its
   range shrinks to [r*mn, r*mx] (symmetric: [-r*amax, r*amax], fp32 products)
   and its weights are clamped to it (fp32, then fp16).  The group keeps the r
   with the smallest output error over the calibration activations,
   err(n, j, r) = sum_m (sum_{k in group j} x_mk (Dq(Q(clip_r(W)))_nk - w_nk))^2
   (the first r on ties); the clipped weights are then packed as usual.

Parity pins: every function here is pinned by tests that do not re-type its
formula (hand-worked examples, brute force over every fp16 value of a range,
closed forms and invariants); none is "parity unpinned".
"""
from __future__ import annotations

import math

import numpy as np

F32 = np.float32

# Nibble slot i of a packed weight word holds the code of k = 8j + PACK_ORDER[i].
# With this order the low halfword of a word holds k = 0,2,4,6 and the high
# halfword k = 1,3,5,7 of its 8-channel block (storage reading 5 above).
PACK_ORDER = (0, 2, 4, 6, 1, 3, 5, 7)

SCALE_FLOOR = F32(1e-5)
QMAX = 15


def _check_shape(W16: np.ndarray, g: int) -> tuple[int, int, int]:
    if W16.dtype != np.float16 or W16.ndim != 2:
        raise TypeError("W must be a 2-D float16 array [N, K]")
    N, K = W16.shape
    if g <= 0 or K % g:
        raise ValueError(f"group size {g} must divide K={K}")
    return N, K, K // g


def group_params(W16: np.ndarray, g: int, zero_point: bool):
    """Per-(row, group) scale and zero point (readings 1-3).

    [P5] "分组大小 Group Size": all weights of a group share one scale and one
    zero point.  [P5] "零点量化 Zero-Point": with a zero point the grid is
    shifted to cover an asymmetric range; without one it is symmetric.

    Returns ``(s16, z)``: ``s16`` float16 [N, G], ``z`` int64 [N, G].
    """
    N, K, G = _check_shape(W16, g)
    a = W16.astype(F32).reshape(N, G, g)  # fp16 -> fp32 is exact
    if zero_point:
        mn = a.min(axis=2)
        mx = a.max(axis=2)
        r = (mx - mn).astype(F32)
        r = np.where(r < SCALE_FLOOR, SCALE_FLOOR, r).astype(F32)
        s16 = (r / F32(QMAX)).astype(F32).astype(np.float16)
        s = s16.astype(F32)
        zf = np.rint((-mn).astype(F32) / s).astype(F32)
        z = np.clip(zf, F32(0), F32(QMAX)).astype(np.int64)
    else:
        amax = np.abs(a).max(axis=2).astype(F32)
        amax = np.where(amax < SCALE_FLOOR, SCALE_FLOOR, amax).astype(F32)
        s16 = (amax / F32(7)).astype(F32).astype(np.float16)
        z = np.full((N, G), 8, dtype=np.int64)
    return s16, z


def codes(W16: np.ndarray, s16: np.ndarray, z: np.ndarray, g: int) -> np.ndarray:
    """q = clamp(rne(w / s) + z, 0, 15), one code per weight (reading 4).

    The division is a correctly rounded fp32 division and the sum is formed in
    fp32, exactly as written; the clamp keeps every code a 4-bit value.
    """
    N, K, G = _check_shape(W16, g)
    a = W16.astype(F32).reshape(N, G, g)
    s = s16.astype(F32)[:, :, None]
    v = (np.rint((a / s).astype(F32)) + z.astype(F32)[:, :, None]).astype(F32)
    q = np.clip(v, F32(0), F32(QMAX)).astype(np.uint8)
    return q.reshape(N, K)


def quantize(W16: np.ndarray, g: int, zero_point: bool):
    """Group-wise 4-bit quantization Q: returns ``(q uint8 [N,K], s16 [N,G], z [N,G])``."""
    s16, z = group_params(W16, g, zero_point)
    return codes(W16, s16, z, g), s16, z


def dequant(q: np.ndarray, s16: np.ndarray, z: np.ndarray, g: int) -> np.ndarray:
    """Decoded weight w' = (q - z) * s in fp64 (exact: a 5-bit by 11-bit product)."""
    N, K = q.shape
    G = K // g
    d = q.astype(np.float64).reshape(N, G, g) - z.astype(np.float64)[:, :, None]
    return (d * s16.astype(np.float64)[:, :, None]).reshape(N, K)


def fake_quant(W16: np.ndarray, g: int, zero_point: bool) -> np.ndarray:
    """Dq(Q(W)): quantize then decode, fp64 [N, K]."""
    q, s16, z = quantize(W16, g, zero_point)
    return dequant(q, s16, z, g)


# ---------------------------------------------------------------------------
# Storage layout (reading 5).  Written with explicit per-slot index formulas.
# ---------------------------------------------------------------------------

def pack_qweight(q: np.ndarray) -> np.ndarray:
    """qweight u32 [N][K/8]; nibble slot i of word (n, j) = q[n, 8j + PACK_ORDER[i]]."""
    N, K = q.shape
    if K % 8:
        raise ValueError("K must be a multiple of 8")
    words = np.zeros((N, K // 8), dtype=np.uint32)
    for i, kk in enumerate(PACK_ORDER):
        words |= q[:, kk::8].astype(np.uint32) << np.uint32(4 * i)
    return words


def unpack_qweight(qweight: np.ndarray, K: int) -> np.ndarray:
    N = qweight.shape[0]
    q = np.zeros((N, K), dtype=np.uint8)
    for i, kk in enumerate(PACK_ORDER):
        q[:, kk::8] = ((qweight >> np.uint32(4 * i)) & np.uint32(0xF)).astype(np.uint8)
    return q


def pack_scales(s16: np.ndarray) -> np.ndarray:
    """scales as raw fp16 bits, row-octet major: uint16 [N/8][G][8]; element
    (o, j, i) = scale of row 8o + i in group j."""
    N, G = s16.shape
    if N % 8:
        raise ValueError("N must be a multiple of 8")
    out = np.zeros((N // 8, G, 8), dtype=np.uint16)
    bits = s16.view(np.uint16)
    for i in range(8):
        out[:, :, i] = bits[i::8, :]
    return out


def unpack_scales(scales_u16: np.ndarray) -> np.ndarray:
    O8, G, _ = scales_u16.shape
    s = np.zeros((O8 * 8, G), dtype=np.uint16)
    for i in range(8):
        s[i::8, :] = scales_u16[:, :, i]
    return s.view(np.float16)


def pack_qzeros(z: np.ndarray) -> np.ndarray:
    """qzeros u32 [N/8][G]; nibble slot i of word (o, j) = zero point of row 8o + i, group j."""
    N, G = z.shape
    if N % 8:
        raise ValueError("N must be a multiple of 8")
    words = np.zeros((N // 8, G), dtype=np.uint32)
    for i in range(8):
        words |= z[i::8, :].astype(np.uint32) << np.uint32(4 * i)
    return words


def unpack_qzeros(qzeros: np.ndarray, N: int) -> np.ndarray:
    O8, G = qzeros.shape
    z = np.zeros((O8 * 8, G), dtype=np.int64)
    for i in range(8):
        z[i::8, :] = ((qzeros >> np.uint32(4 * i)) & np.uint32(0xF)).astype(np.int64)
    return z


def pack(W16: np.ndarray, g: int, zero_point: bool):
    """Quantize and store: ``(qweight u32 [N,K/8], scales u16 [N/8,G,8], qzeros u32 [N/8,G] | None)``."""
    q, s16, z = quantize(W16, g, zero_point)
    qz = pack_qzeros(z) if zero_point else None
    return pack_qweight(q), pack_scales(s16), qz


def unpack(qweight, scales_u16, qzeros, N: int, K: int, g: int, zero_point: bool):
    """Inverse of :func:`pack`: ``(q, s16, z)``; the symmetric zero is the implicit 8."""
    G = K // g
    q = unpack_qweight(qweight, K)
    s16 = unpack_scales(scales_u16)
    if zero_point:
        z = unpack_qzeros(qzeros, N)
    else:
        z = np.full((N, G), 8, dtype=np.int64)
    return q, s16, z


def dequant_packed(qweight, scales_u16, qzeros, N: int, K: int, g: int, zero_point: bool):
    q, s16, z = unpack(qweight, scales_u16, qzeros, N, K, g, zero_point)
    return dequant(q, s16, z, g)


# ---------------------------------------------------------------------------
# The linear layer and the acceptance test.
# ---------------------------------------------------------------------------

def matmul_ref(X16: np.ndarray, Wdq: np.ndarray):
    """Y_ref = X . W'^T and D = |X| . |W'|^T, both fp64 [M, N] (reading 6).

    [P5] "WQLinear 内核全景": the quantized layer is an ordinary linear map on
    the decoded weights; GEMM and GEMV differ only in how they are computed.
    """
    X = X16.astype(np.float64)
    W = np.asarray(Wdq, dtype=np.float64)
    return X @ W.T, np.abs(X) @ np.abs(W).T


def matmul_ref_fsum(X16: np.ndarray, Wdq: np.ndarray) -> np.ndarray:
    """The same Y with every dot product summed by ``math.fsum`` (small inputs only)."""
    X = X16.astype(np.float64)
    W = np.asarray(Wdq, dtype=np.float64)
    M, N = X.shape[0], W.shape[0]
    Y = np.empty((M, N))
    for m in range(M):
        for n in range(N):
            Y[m, n] = math.fsum((X[m] * W[n]).tolist())
    return Y


def tolerance_ratio(Y_dev: np.ndarray, Y_ref: np.ndarray, D: np.ndarray) -> np.ndarray:
    """|Y_dev - Y_ref| / D per element; 0 where both the error and D are 0, inf
    where D = 0 but the error is not."""
    err = np.abs(np.asarray(Y_dev, dtype=np.float64) - Y_ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(D > 0, err / np.where(D > 0, D, 1.0), np.where(err > 0, np.inf, 0.0))
    return r


def recon_loss(W16: np.ndarray, X: np.ndarray, s: np.ndarray, g: int, zero_point: bool) -> float:
    """L(s) = ||Q(W*s)(s^-1*X) - W*X|| (reading 7).

    [P5] "算法原理": the per-input-channel scale s multiplies the weight before
    quantization and its inverse multiplies the activation; AWQ picks s to make
    this reconstruction error small.  ``s`` is a positive fp32 vector of length
    K; ``W*s`` is formed in fp32 and rounded to fp16 (Q takes fp16 weights);
    ``s^-1 * X`` and the norm are fp64.
    """
    N, K, _ = _check_shape(W16, g)
    s = np.asarray(s, dtype=F32)
    if s.shape != (K,) or not np.all(s > 0):
        raise ValueError("s must be a positive vector of length K")
    Wq = fake_quant(scale_weights(W16, s), g, zero_point)
    Xs = np.asarray(X, dtype=np.float64) / s.astype(np.float64)[None, :]
    ref = np.asarray(X, dtype=np.float64) @ W16.astype(np.float64).T
    return float(np.linalg.norm(Xs @ Wq.T - ref))


def scale_weights(W16: np.ndarray, s: np.ndarray) -> np.ndarray:
    """fp16(W * s): each weight times its input channel's scale, an fp32
    product rounded once to fp16 (reading 7: Q takes fp16 weights)."""
    s = np.asarray(s, dtype=F32)
    return (W16.astype(F32) * s[None, :]).astype(F32).astype(np.float16)


ACT_FLOOR = 1e-4
WEIGHT_FLOOR = 1e-4


def activation_scale(X16: np.ndarray) -> np.ndarray:
    """Per-input-channel activation statistic a_k = max(mean_m |x_mk|, 1e-4)
    (reading 8), fp64."""
    X = np.asarray(X16, dtype=np.float64)
    if X.ndim != 2 or X.shape[0] < 1:
        raise ValueError("X must be [M, K] with M >= 1")
    return np.maximum(np.abs(X).mean(axis=0), ACT_FLOOR)


def weight_scale(W16: np.ndarray) -> np.ndarray:
    """Per-input-channel weight statistic of duo scaling (reading 8),
    b_k = max(mean_n |w_nk|, 1e-4), fp64."""
    W = np.asarray(W16, dtype=np.float64)
    if W.ndim != 2 or W.shape[0] < 1:
        raise ValueError("W must be [N, K] with N >= 1")
    return np.maximum(np.abs(W).mean(axis=0), WEIGHT_FLOOR)


def scale_candidates(X16: np.ndarray, alphas, W16: np.ndarray | None = None) -> np.ndarray:
    """Candidate scales (reading 8) as fp32 [len(alphas), K]: s_c = a^alpha_c
    (alpha = 0 gives exactly 1), or with ``W16`` (duo scaling)
    s_c = a^alpha_c / b^(1 - alpha_c), computed in fp64 and rounded to fp32."""
    a = activation_scale(X16)
    if W16 is None:
        return np.stack([np.power(a, float(al)).astype(F32) for al in alphas])
    b = weight_scale(W16)
    return np.stack([(np.power(a, float(al)) / np.power(b, 1.0 - float(al))).astype(F32) for al in alphas])


def search_scale(W16: np.ndarray, X16: np.ndarray, g: int, zero_point: bool, alphas, duo: bool = False):
    """Evaluate L(s_c) (reading 7) for every candidate of reading 8 (duo
    scaling with ``duo``) and return (index of the smallest loss, the
    candidates, the losses)."""
    S = scale_candidates(X16, alphas, W16 if duo else None)
    losses = [recon_loss(W16, X16, s, g, zero_point) for s in S]
    return int(np.argmin(losses)), S, losses


def clip_weight(W16: np.ndarray, g: int, zero_point: bool, ratio) -> np.ndarray:
    """Clamp every group of W to its range shrunk by ``ratio`` (reading 9);
    ``ratio`` is one value or an [N, G] array.  Returns fp16 [N, K]."""
    N, K, G = _check_shape(W16, g)
    a = W16.astype(F32).reshape(N, G, g)
    r = np.broadcast_to(np.asarray(ratio, dtype=F32), (N, G))[:, :, None]
    if zero_point:
        lo = (r * a.min(axis=2)[:, :, None]).astype(F32)
        hi = (r * a.max(axis=2)[:, :, None]).astype(F32)
    else:
        hi = (r * np.abs(a).max(axis=2)[:, :, None]).astype(F32)
        lo = -hi
    return np.minimum(np.maximum(a, lo), hi).astype(F32).astype(np.float16).reshape(N, K)


def clip_errors(W16: np.ndarray, X16: np.ndarray, g: int, zero_point: bool, ratios) -> np.ndarray:
    """err[i, n, j]: the output error of group (n, j) over the calibration
    activations when every group is clipped by ratios[i] (reading 9), fp64."""
    N, K, G = _check_shape(W16, g)
    X = np.asarray(X16, dtype=np.float64)
    W = W16.astype(np.float64)
    out = np.empty((len(ratios), N, G))
    for i, r in enumerate(ratios):
        E = fake_quant(clip_weight(W16, g, zero_point, r), g, zero_point) - W
        for j in range(G):
            Y = X[:, j * g:(j + 1) * g] @ E[:, j * g:(j + 1) * g].T
            out[i, :, j] = (Y * Y).sum(axis=0)
    return out


def search_clip(W16: np.ndarray, X16: np.ndarray, g: int, zero_point: bool, ratios):
    """Per group, the ratio with the smallest output error (reading 9).
    Returns (choice int [N, G], clipped weights fp16 [N, K], err)."""
    err = clip_errors(W16, X16, g, zero_point, ratios)
    best = np.argmin(err, axis=0)
    Wc = clip_weight(W16, g, zero_point, np.asarray(ratios, dtype=F32)[best])
    return best, Wc, err
