"""Pins for the CPU oracle, checked against what the definitions fix.

Nothing here re-types the oracle's formulas.  The checks are:
hand-worked examples (tests/golden), brute-force searches over candidate codes,
zero points and every finite fp16 value of a range, exact rational arithmetic
for the scale, closed forms (a weight already on a 4-bit grid must come back
unchanged), and invariants (sign symmetry, power-of-two equivariance, the
ordering of scales under group size and zero point, L(s) invariance).

The last test plants plausible mistakes in the oracle (on the CPU) and checks
that at least one pin catches each of them.
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import awq_oracle as O
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

ALL_FP16 = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16).view(np.float16)
FINITE_FP16 = ALL_FP16[np.isfinite(ALL_FP16)]


def read_golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = line.split(":", 1)
            out[key.strip()] = val.split()
    return out


def _num(xs):
    return np.array([float(Fraction(v)) for v in xs])


def _hex(v):
    return int(v[0], 16)


# ---------------------------------------------------------------------------
# Individual checks, written as functions so the mutation test can rerun them.
# Each returns None on success and raises AssertionError on failure.
# ---------------------------------------------------------------------------

def check_hand_example(name, zero_point):
    gold = read_golden(name)
    w = _num(gold["w"]).astype(np.float16)[None, :]
    q, s16, z = O.quantize(w, 8, zero_point)
    assert int(s16.view(np.uint16)[0, 0]) == _hex(gold["scale_bits"])
    assert int(z[0, 0]) == int(gold["zero"][0])
    assert q[0].tolist() == [int(v) for v in gold["q"]]
    wdq = O.dequant(q, s16, z, 8)
    assert np.array_equal(wdq[0], _num(gold["w_dq"]))
    # the natural-order word in the fixture is consistent with its codes
    nat = sum(int(c) << (4 * i) for i, c in enumerate(gold["q"]))
    assert nat == _hex(gold["word_natural"])
    assert int(O.pack_qweight(q)[0, 0]) == _hex(gold["word_packed"])
    if zero_point:
        qz = O.pack_qzeros(np.repeat(z, 8, axis=0))  # 8 rows of the same group
        assert int(qz[0, 0]) == int("0x" + gold["zero"][0] * 8, 16)
    for xs, ys in (("x1", "y1"), ("x2", "y2")):
        if xs not in gold:
            continue
        x = _num(gold[xs]).astype(np.float16)[None, :]
        y, d = O.matmul_ref(x, wdq)
        assert y[0, 0] == float(Fraction(gold[ys][0]))
        assert O.matmul_ref_fsum(x, wdq)[0, 0] == y[0, 0]
        if "d2" in gold and xs == "x2":
            assert d[0, 0] == float(Fraction(gold["d2"][0]))


def _argmin_code(w, s, z):
    """Nearest grid point by exhaustive search over the 16 codes; a tie goes to
    the even value of (code - zero).  Exact fp64 arithmetic."""
    w = np.asarray(w, dtype=np.float64)[:, None]
    c = np.arange(16, dtype=np.float64)[None, :]
    err = np.abs(w - (c - z) * s)
    best = err.min(axis=1, keepdims=True)
    cand = err == best
    even = ((np.arange(16) - z) % 2 == 0)[None, :]
    pick_even = cand & even
    use = np.where(pick_even.any(axis=1, keepdims=True), pick_even, cand)
    return np.argmax(use, axis=1)


def check_brute_force_codes(scales_bits=(0x2C00, 0x1E66, 0x3555, 0x2001, 0x0400, 0x0013), zeros=(0, 3, 8, 15)):
    for sb in scales_bits:
        s16 = np.array([sb], dtype=np.uint16).view(np.float16)[0]
        s = float(s16)
        for z in zeros:
            lo, hi = -z * s, (15 - z) * s
            w = FINITE_FP16[(FINITE_FP16.astype(np.float64) >= lo) & (FINITE_FP16.astype(np.float64) <= hi)]
            if w.size == 0:
                continue
            W = w[None, :]
            gs = W.shape[1]
            q = O.codes(W, np.full((1, 1), s16, np.float16), np.full((1, 1), z, np.int64), gs)[0]
            ref = _argmin_code(w, s, z)
            assert np.array_equal(q.astype(np.int64), ref), (hex(sb), z)
            err = np.abs(w.astype(np.float64) - (q.astype(np.float64) - z) * s)
            assert err.max() <= s / 2


def _brute_zero(mn, s):
    """z minimising |mn - (0 - z) s| over z in 0..15; ties to even z."""
    zs = np.arange(16, dtype=np.float64)
    err = np.abs(mn + zs * s)
    best = err.min()
    cand = np.flatnonzero(err == best)
    ev = [c for c in cand if c % 2 == 0]
    return int(ev[0] if ev else cand[0])


def _fp16_neighbours(t: Fraction):
    x = np.float16(float(t))
    lo = x if Fraction(float(x)) <= t else np.nextafter(x, np.float16(-np.inf))
    hi = np.nextafter(lo, np.float16(np.inf))
    return lo, hi


def check_scale_and_zero(W16, g, zero_point):
    """The scale is the fp16 value nearest the exact range/15 (max|w|/7), with a
    2^-22 relative allowance for the fp32 intermediate; the zero point is the
    nearest-to-min grid offset (brute force)."""
    s16, z = O.group_params(W16, g, zero_point)
    N, K = W16.shape
    G = K // g
    a = W16.astype(np.float64).reshape(N, G, g)
    for n in range(N):
        for j in range(G):
            grp = a[n, j]
            if zero_point:
                r = Fraction(float(grp.max())) - Fraction(float(grp.min()))
                floor = Fraction(float(np.float32(1e-5)))
                t = max(r, floor) / 15
            else:
                t = max(Fraction(float(np.abs(grp).max())), Fraction(float(np.float32(1e-5)))) / 7
            lo, hi = _fp16_neighbours(t)
            got = s16[n, j]
            mid = (Fraction(float(lo)) + Fraction(float(hi))) / 2
            if abs(t - mid) <= t * Fraction(1, 1 << 22):
                assert got in (lo, hi)
            else:
                want = lo if t < mid else hi
                assert got == want, (n, j, float(t), float(got), float(want))
            if zero_point:
                assert int(z[n, j]) == _brute_zero(float(grp.min()), float(got))
            else:
                assert int(z[n, j]) == 8


def _grid_weight(rng, N, K, g, zero_point):
    """fp16 weights that already lie on a 4-bit grid spanning the full code
    range of each group, with scales of at most 7 mantissa bits so every grid
    value is an exact fp16 number.  Returns (W16, q, s16, z)."""
    G = K // g
    mant = rng.integers(64, 128, size=(N, G))
    expo = rng.integers(-12, -2, size=(N, G))
    s = (mant.astype(np.float64) / 64.0) * np.exp2(expo.astype(np.float64))
    s16 = s.astype(np.float16)
    assert np.array_equal(s16.astype(np.float64), s)
    if zero_point:
        z = rng.integers(0, 16, size=(N, G))
        q = rng.integers(0, 16, size=(N, G, g))
        q[:, :, 0] = 0
        q[:, :, 1] = 15
    else:
        z = np.full((N, G), 8)
        q = rng.integers(1, 16, size=(N, G, g))
        q[:, :, 0] = np.where(rng.integers(0, 2, size=(N, G)) == 1, 1, 15)
    perm = rng.permuted(np.tile(np.arange(g), (N, G, 1)), axis=2)
    q = np.take_along_axis(q, perm, axis=2)
    w = (q - z[:, :, None]) * s[:, :, None]
    W16 = w.reshape(N, K).astype(np.float16)
    assert np.array_equal(W16.astype(np.float64), w.reshape(N, K))
    return W16, q.reshape(N, K).astype(np.uint8), s16, z


def check_grid_recovery(seed=1):
    rng = np.random.default_rng(seed)
    for zp in (True, False):
        for g in (8, 32, 128):
            W16, q, s16, z = _grid_weight(rng, 16, 4 * g, g, zp)
            q2, s2, z2 = O.quantize(W16, g, zp)
            assert np.array_equal(s2.view(np.uint16), s16.view(np.uint16))
            assert np.array_equal(z2, z)
            assert np.array_equal(q2, q)
            assert np.array_equal(O.dequant(q2, s2, z2, g), W16.astype(np.float64))


def check_symmetric_negation(seed=2):
    W = workloads.weight(64, 512, cfg=99, layer=seed)
    q, s, z = O.quantize(W, 128, False)
    qn, sn, zn = O.quantize(-W, 128, False)
    assert np.array_equal(s.view(np.uint16), sn.view(np.uint16))
    assert np.array_equal(qn.astype(np.int64), 16 - q.astype(np.int64))
    assert np.array_equal(O.dequant(qn, sn, zn, 128), -O.dequant(q, s, z, 128))


def check_equivariance(seed=3):
    W = workloads.weight(32, 512, cfg=98, layer=seed)
    W = np.where(np.abs(W.astype(np.float32)) < 2.0 ** -10, np.float16(0.01), W).astype(np.float16)
    for zp in (True, False):
        q, s, z = O.quantize(W, 64, zp)
        for e in (-2, -1, 1, 3):
            We = (W.astype(np.float64) * 2.0 ** e).astype(np.float16)
            assert np.array_equal(We.astype(np.float64), W.astype(np.float64) * 2.0 ** e)
            qe, se, ze = O.quantize(We, 64, zp)
            assert np.array_equal(qe, q) and np.array_equal(ze, z)
            assert np.array_equal(se.astype(np.float64), s.astype(np.float64) * 2.0 ** e)


def check_code_range_and_error_bound(seed=4):
    for kind in ("gauss", "offset", "adversarial"):
        if kind == "adversarial":
            W = workloads.adversarial_weight(24, 256, 32, seed=seed)
        else:
            W = workloads.weight(48, 1024, cfg=97, layer=seed, row_offset=(kind == "offset"))
        for zp in (True, False):
            for g in (32, 128):
                if W.shape[1] % g:
                    continue
                q, s16, z = O.quantize(W, g, zp)
                assert q.min() >= (0 if zp else 1) and q.max() <= 15
                s = np.repeat(s16.astype(np.float64), g, axis=1)
                zz = np.repeat(z.astype(np.float64), g, axis=1)
                w = W.astype(np.float64)
                inr = (w >= -zz * s) & (w <= (15 - zz) * s)
                err = np.abs(w - O.dequant(q, s16, z, g))
                assert np.all(err[inr] <= s[inr] / 2)


def check_orderings(seed=5):
    W = workloads.weight(64, 1024, cfg=96, layer=seed, row_offset=True)
    s1, _ = O.group_params(W, 128, True)
    s0, _ = O.group_params(W, 128, False)
    assert np.all(s1.astype(np.float64) <= s0.astype(np.float64))
    for zp in (True, False):
        parent, _ = O.group_params(W, 256, zp)
        child, _ = O.group_params(W, 32, zp)
        child = child.astype(np.float64).reshape(64, 1024 // 256, 8)
        assert np.all(child <= parent.astype(np.float64)[:, :, None])


def check_special_groups():
    g = 32
    # all zeros: floor on the range, subnormal fp16 scale, codes equal the zero
    Z = np.zeros((8, g), np.float16)
    q, s, z = O.quantize(Z, g, True)
    assert int(s.view(np.uint16)[0, 0]) == 0x000B and np.all(z == 0) and np.all(q == 0)
    q, s, z = O.quantize(Z, g, False)
    assert int(s.view(np.uint16)[0, 0]) == 0x0018 and np.all(q == 8)
    # a range that excludes 0 saturates: z = 0 and every code is 15
    P = np.linspace(0.4, 0.5, g).astype(np.float16)[None, :].repeat(8, 0)
    q, s, z = O.quantize(P, g, True)
    assert np.all(z == 0) and np.all(q == 15)
    # the mirrored all-negative group: z = 15, every code 0
    q, s, z = O.quantize(-P, g, True)
    assert np.all(z == 15) and np.all(q == 0)


def check_layout(seed=6):
    rng = np.random.default_rng(seed)
    N, K, g = 16, 64, 32
    q = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    words = O.pack_qweight(q)
    for n in range(N):
        for k in range(K):
            j, r = divmod(k, 8)
            slot = [0, 4, 1, 5, 2, 6, 3, 7][r]  # slot of channel r within its word
            assert (int(words[n, j]) >> (4 * slot)) & 0xF == q[n, k]
    # the 0x000F000F mask at shift 4t picks channels (2t, 2t+1)
    for t in range(4):
        lo = (words >> np.uint32(4 * t)) & np.uint32(0xF)
        hi = (words >> np.uint32(16 + 4 * t)) & np.uint32(0xF)
        assert np.array_equal(lo, q[:, 2 * t::8]) and np.array_equal(hi, q[:, 2 * t + 1::8])
    z = rng.integers(0, 16, size=(N, K // g))
    qz = O.pack_qzeros(z)
    assert qz.shape == (N // 8, K // g)
    for n in range(N):
        for j in range(K // g):
            assert (int(qz[n // 8, j]) >> (4 * (n % 8))) & 0xF == z[n, j]
    s = rng.standard_normal((N, K // g)).astype(np.float16)
    sc = O.pack_scales(s)
    assert sc.shape == (N // 8, K // g, 8) and sc.dtype == np.uint16
    flat = sc.reshape(-1)
    G = K // g
    for n in range(N):
        for j in range(G):
            assert flat[((n // 8) * G + j) * 8 + n % 8] == s.view(np.uint16)[n, j]
    q2, s2, z2 = O.unpack(words, sc, qz, N, K, g, True)
    assert np.array_equal(q2, q) and np.array_equal(z2, z)
    assert np.array_equal(s2.view(np.uint16), s.view(np.uint16))


def check_recon_loss(seed=7):
    gold = read_golden("hand_asym_g8.txt")
    w = _num(gold["w"]).astype(np.float16)[None, :]
    x = _num(gold["x2"])[None, :]
    assert O.recon_loss(w, x, np.ones(8, np.float32), 8, True) == float(Fraction(gold["loss_x2_s1"][0]))
    rng = np.random.default_rng(seed)
    for zp in (True, False):
        W = workloads.weight(16, 256, cfg=95, layer=seed)
        X = workloads.activations(4, 256, cfg=95, layer=seed).astype(np.float64)
        L1 = O.recon_loss(W, X, np.ones(256, np.float32), 64, zp)
        assert L1 > 0
        e = rng.integers(-2, 3, size=256 // 64)
        s = np.repeat(np.exp2(e.astype(np.float64)), 64).astype(np.float32)
        assert O.recon_loss(W, X, s, 64, zp) == L1
        Wg, _, _, _ = _grid_weight(rng, 16, 256, 64, zp)
        assert O.recon_loss(Wg, X, np.ones(256, np.float32), 64, zp) == 0.0
        s_rand = rng.uniform(0.5, 2.0, size=256).astype(np.float32)
        assert O.recon_loss(W, X, s_rand, 64, zp) >= 0.0


def check_scale_candidates():
    # a = mean |x| per channel with the 1e-4 floor: [2, 1, 1e-4, 0.5]
    X = np.array([[1, -2, 0, 0.5], [3, 0, 0, -0.5]], np.float16)
    a = O.activation_scale(X)
    assert np.array_equal(a, np.array([2.0, 1.0, 1e-4, 0.5]))
    S = O.scale_candidates(X, [0.0, 0.5, 1.0])
    assert S.dtype == np.float32 and S.shape == (3, 4)
    assert np.array_equal(S[0], np.ones(4, np.float32))
    assert np.array_equal(S[2], np.array([2.0, 1.0, 1e-4, 0.5], np.float32))
    assert np.array_equal(S[1], np.sqrt(np.array([2.0, 1.0, 1e-4, 0.5])).astype(np.float32))


def check_duo_candidates():
    # a = [2, 1, 1e-4 (floor), 0.5] as above; b = mean |w| per channel = [0.5, 1, 2, 1e-4 (floor)]
    X = np.array([[1, -2, 0, 0.5], [3, 0, 0, -0.5]], np.float16)
    W = np.array([[0.5, 1, 2, 0], [0.5, -1, -2, 0]], np.float16)
    assert np.array_equal(O.weight_scale(W), np.array([0.5, 1.0, 2.0, 1e-4]))
    S = O.scale_candidates(X, [0.0, 0.5, 1.0], W)
    assert S.dtype == np.float32 and S.shape == (3, 4)
    # alpha = 0: 1 / b; alpha = 1: a (the activation-only candidate); alpha = 1/2: sqrt(a / b)
    assert np.array_equal(S[0], np.array([2.0, 1.0, 0.5, 1e4], np.float32))
    assert np.array_equal(S[2], np.array([2.0, 1.0, 1e-4, 0.5], np.float32))
    np.testing.assert_allclose(S[1], [2.0, 1.0, math.sqrt(5e-5), math.sqrt(5e3)], rtol=2.4e-7)
    # weights twice as large halve the alpha = 0 candidate exactly (the floored
    # all-zero channel keeps its floor)
    S2 = O.scale_candidates(X, [0.0], (W.astype(np.float32) * 2).astype(np.float16))[0]
    assert np.array_equal(S2[:3], S[0][:3] / 2) and S2[3] == S[0][3]


def check_weight_scale_brute_force():
    W = workloads.weight(37, 24, cfg=96, layer=3, row_offset=True)
    W[:, 5] = 0  # an all-zero channel takes the floor
    b = O.weight_scale(W)
    for k in range(24):
        want = max(math.fsum(abs(float(v)) for v in W[:, k]) / 37, 1e-4)
        assert abs(b[k] - want) <= 1e-15 * want, k
    assert b[5] == 1e-4


def check_scale_weights():
    W = np.array([[0.5, 3, -1.5, 1.0], [0.25, -2, 0, 1.0]], np.float16)
    s = np.array([2.0, 0.5, 3.0, 1.0 / 3.0], np.float32)
    got = O.scale_weights(W, s)
    assert got.dtype == np.float16
    # products exact in fp16, except 1 * fp32(1/3) = 0.33333334 whose nearest fp16 is 0x3555 (0.333251953125)
    want = np.array([[1.0, 1.5, -4.5, 0.333251953125], [0.5, -1.0, 0.0, 0.333251953125]], np.float16)
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16))
    assert got.view(np.uint16)[0, 3] == 0x3555
    # a power-of-two scale >= 1 per channel scales exactly
    Wr = workloads.weight(8, 64, cfg=96, layer=4)
    e = np.random.default_rng(3).integers(0, 4, size=64)  # no scale into the fp16 subnormals
    assert np.array_equal(O.scale_weights(Wr, np.exp2(e).astype(np.float32)).astype(np.float64),
                          Wr.astype(np.float64) * np.exp2(e)[None, :])


def check_duo_search():
    W = workloads.weight(64, 256, cfg=96, layer=1)
    X = workloads.activations(64, 256, cfg=96, layer=1)
    alphas = [i / 10 for i in range(10)]
    best, S, losses = O.search_scale(W, X, 64, True, alphas, duo=True)
    assert np.array_equal(S, O.scale_candidates(X, alphas, W))
    for i in (0, 3, 9):
        assert losses[i] == O.recon_loss(W, X, S[i], 64, True)
    assert losses[best] == min(losses) and all(losses[best] < losses[i] for i in range(best))
    rtn = O.recon_loss(W, X, np.ones(256, np.float32), 64, True)
    assert losses[best] < 0.8 * rtn, "duo scaling must beat plain rounding on 1%-outlier data"


def check_search_scale():
    W = workloads.weight(64, 256, cfg=96, layer=1)
    X = workloads.activations(64, 256, cfg=96, layer=1)
    alphas = [i / 10 for i in range(10)]
    best, S, losses = O.search_scale(W, X, 64, True, alphas)
    assert len(losses) == 10 and S.shape == (10, 256)
    # alpha = 0 is plain round-to-nearest: s = 1
    assert losses[0] == O.recon_loss(W, X, np.ones(256, np.float32), 64, True)
    assert losses[best] == min(losses) and all(losses[best] < losses[i] for i in range(best))
    # the outlier channels (x20) get the largest scales for alpha > 0
    out = np.argsort(O.activation_scale(X))[-3:]
    assert np.all(S[5][out] > np.median(S[5]))
    # with 1% outlier channels, scaling them protects the weights that meet them
    assert best > 0 and losses[best] < 0.8 * losses[0]


def check_clip_weight():
    gold = read_golden("hand_asym_g8.txt")
    w = _num(gold["w"]).astype(np.float16)[None, :]
    for zp in (True, False):
        assert np.array_equal(O.clip_weight(w, 8, zp, 1.0).view(np.uint16), w.view(np.uint16))
    # r = 1/2: asymmetric range [-0.125, 0.34375]; symmetric [-0.34375, 0.34375]
    half = [-0.125, 0.34375, 0, 0.125, -0.0625, 0.3125, 0.34375, 0.03125]
    assert np.array_equal(O.clip_weight(w, 8, True, 0.5)[0].astype(np.float64), half)
    sym = [-0.25, 0.34375, 0, 0.125, -0.0625, 0.3125, 0.34375, 0.03125]
    assert np.array_equal(O.clip_weight(w, 8, False, 0.5)[0].astype(np.float64), sym)
    # per-group ratios: each group uses its own
    W = workloads.weight(8, 64, cfg=97, layer=3)
    r = np.linspace(0.5, 1.0, 16, dtype=np.float32).reshape(8, 2)
    Wc = O.clip_weight(W, 32, True, r)
    for n in range(8):
        for j in range(2):
            assert np.array_equal(Wc[n, 32 * j:32 * j + 32], O.clip_weight(W[n:n + 1, 32 * j:32 * j + 32], 32, True,
                                                                              r[n, j])[0])


def check_clip_errors():
    # brute force on a tiny layer, straight from the definition
    W = workloads.weight(8, 16, cfg=97, layer=4)
    X = workloads.activations(3, 16, cfg=97, layer=4)
    ratios = [1.0, 0.75, 0.5]
    for zp in (True, False):
        err = O.clip_errors(W, X, 8, zp, ratios)
        for i, r in enumerate(ratios):
            Wq = O.fake_quant(O.clip_weight(W, 8, zp, r), 8, zp)
            for n in range(8):
                for j in range(2):
                    tot = 0.0
                    for m in range(3):
                        y = math.fsum(float(X[m, k]) * (Wq[n, k] - float(W[n, k])) for k in range(8 * j, 8 * j + 8))
                        tot += y * y
                    assert abs(err[i, n, j] - tot) <= 1e-12 * max(tot, 1e-30)
    # one group per row: the unclipped errors add up to L(1)^2
    W = workloads.weight(16, 128, cfg=97, layer=5)
    X = workloads.activations(8, 128, cfg=97, layer=5)
    e1 = O.clip_errors(W, X, 128, True, [1.0])
    L = O.recon_loss(W, X, np.ones(128, np.float32), 128, True)
    assert abs(e1.sum() - L * L) <= 1e-12 * L * L


def check_search_clip():
    W = workloads.weight(64, 256, cfg=97, layer=1)
    X = workloads.activations(64, 256, cfg=97, layer=1)
    ratios = [1 - 0.025 * i for i in range(20)]
    best, Wc, err = O.search_clip(W, X, 64, True, ratios)
    assert best.shape == (64, 4) and Wc.dtype == np.float16
    n, j = np.meshgrid(np.arange(64), np.arange(4), indexing="ij")
    assert np.all(err[best, n, j] == err.min(axis=0))
    assert np.all(err[best, n, j] <= err[0])
    # clipping pays off on these weights, and the clipped layer has a lower L(1)
    assert np.count_nonzero(best) > 64
    Xd = X.astype(np.float64)
    ref = Xd @ W.astype(np.float64).T
    assert np.linalg.norm(Xd @ O.fake_quant(Wc, 64, True).T - ref) < 0.8 * O.recon_loss(
        W, X, np.ones(256, np.float32), 64, True)


def check_matmul_exact(seed=8):
    W = workloads.weight(512, 512, cfg=0, layer=0, seed=0)
    X = workloads.activations(1, 512, cfg=0, layer=0, seed=0)
    Wdq = O.fake_quant(W, 128, True)
    y, d = O.matmul_ref(X, Wdq)
    yf = O.matmul_ref_fsum(X, Wdq)
    # fsum is exactly rounded; the BLAS sum stays within K * 2^-53 * D of it
    assert np.all(np.abs(y - yf) <= 512 * 2.0 ** -53 * d)
    df = np.array([[math.fsum(np.abs(X[0].astype(np.float64) * Wdq[n]).tolist()) for n in range(512)]])
    assert np.all(np.abs(d - df) <= 512 * 2.0 ** -53 * d)


# ---------------------------------------------------------------------------
# The tests.
# ---------------------------------------------------------------------------

def test_hand_example_asymmetric():
    check_hand_example("hand_asym_g8.txt", True)


def test_hand_example_symmetric():
    check_hand_example("hand_sym_g8.txt", False)


def test_codes_match_brute_force_over_every_fp16_in_range():
    check_brute_force_codes()


@pytest.mark.parametrize("zp", [True, False])
@pytest.mark.parametrize("g", [8, 32])
def test_scale_and_zero_match_exact_arithmetic(zp, g):
    W = workloads.weight(8, 4 * g, cfg=94, layer=g, row_offset=True)
    check_scale_and_zero(W, g, zp)
    check_scale_and_zero(workloads.adversarial_weight(8, 4 * g, g, seed=g), g, zp)


def test_grid_weights_come_back_unchanged():
    check_grid_recovery()


def test_symmetric_negation():
    check_symmetric_negation()


def test_power_of_two_equivariance():
    check_equivariance()


def test_code_range_and_half_step_error_bound():
    check_code_range_and_error_bound()


def test_scale_orderings_zero_point_and_group_size():
    check_orderings()


def test_special_groups():
    check_special_groups()


def test_packed_layout_index_formulas():
    check_layout()


def test_recon_loss():
    check_recon_loss()


def test_scale_candidates():
    check_scale_candidates()


def test_search_scale():
    check_search_scale()


def test_duo_scaling_candidates():
    check_duo_candidates()
    check_weight_scale_brute_force()


def test_scale_weights():
    check_scale_weights()


def test_duo_search():
    check_duo_search()


def test_clip_weight():
    check_clip_weight()


def test_clip_errors():
    check_clip_errors()


def test_search_clip():
    check_search_clip()


def test_matmul_ref_against_fsum():
    check_matmul_exact()


def test_tolerance_ratio_edge_cases():
    y_ref = np.array([[0.0, 1.0, 0.0]])
    d = np.array([[0.0, 2.0, 1.0]])
    r = O.tolerance_ratio(np.array([[0.0, 1.002, 0.0]]), y_ref, d)
    assert r[0, 0] == 0 and abs(r[0, 1] - 1e-3) < 1e-12 and r[0, 2] == 0
    assert np.isinf(O.tolerance_ratio(np.array([[1e-9, 1.0, 0.0]]), y_ref, d)[0, 0])


def test_packed_compare_detects_a_flipped_bit():
    W = workloads.weight(64, 256, cfg=93, layer=0)
    qw, sc, qz = O.pack(W, 64, True)
    for arr in (qw, sc, qz):
        bad = arr.copy()
        flat = bad.reshape(-1)
        flat[flat.size // 3] ^= type(flat[0])(1 << 3)
        assert not np.array_equal(bad, arr)


# ---------------------------------------------------------------------------
# Planted mistakes: each must be caught by at least one pin.
# ---------------------------------------------------------------------------

ALL_CHECKS = (
    lambda: check_hand_example("hand_asym_g8.txt", True),
    lambda: check_hand_example("hand_sym_g8.txt", False),
    lambda: check_brute_force_codes(scales_bits=(0x2C00, 0x1E66), zeros=(0, 8)),
    lambda: check_scale_and_zero(workloads.weight(4, 64, cfg=94, layer=1, row_offset=True), 32, True),
    lambda: check_scale_and_zero(workloads.weight(4, 64, cfg=94, layer=1), 32, False),
    check_grid_recovery,
    check_symmetric_negation,
    check_equivariance,
    check_code_range_and_error_bound,
    check_orderings,
    check_special_groups,
    check_layout,
    check_recon_loss,
    check_matmul_exact,
    check_scale_candidates,
    check_search_scale,
    check_duo_candidates,
    check_weight_scale_brute_force,
    check_scale_weights,
    check_duo_search,
    check_clip_weight,
    check_clip_errors,
    check_search_clip,
)


def _round_half_away(x):
    return np.sign(x) * np.floor(np.abs(x) + 0.5)


def _some_check_fails():
    for chk in ALL_CHECKS:
        try:
            chk()
        except AssertionError:
            return True
    return False


MUTATIONS = {
    "round_half_away": lambda mp: mp.setattr(O.np, "rint", _round_half_away),
    "qmax_16": lambda mp: mp.setattr(O, "QMAX", 16),
    "pack_order_natural": lambda mp: mp.setattr(O, "PACK_ORDER", (0, 1, 2, 3, 4, 5, 6, 7)),
    "floor_1e-4": lambda mp: mp.setattr(O, "SCALE_FLOOR", np.float32(1e-4)),
    "scale_not_rounded_to_fp16": None,
    "zero_sign_flipped": None,
    "dequant_drops_zero": None,
    "matmul_wrong_operand_index": None,
    "recon_loss_scales_x_by_s": None,
    "act_stat_max_not_mean": None,
    "candidate_inverse_power": None,
    "search_keeps_largest_loss": None,
    "clip_low_bound_unscaled": None,
    "duo_weight_power_flipped": None,
    "weight_stat_max_not_mean": None,
    "scale_weights_divides": None,
    "clip_error_against_clipped_weight": None,
}


def _patch_function(mp, name):
    if name == "scale_not_rounded_to_fp16":
        orig_gp = O.group_params

        def quantize(W16, g, zero_point):
            # z and q formed with the fp32 scale instead of the stored fp16 one
            s16, _ = orig_gp(W16, g, zero_point)
            N, K = W16.shape
            a = W16.astype(np.float32).reshape(N, K // g, g)
            if zero_point:
                mn = a.min(2)
                s = np.maximum(a.max(2) - mn, np.float32(1e-5)) / np.float32(15)
                z = np.clip(np.rint(-mn / s), 0, 15).astype(np.int64)
            else:
                s = np.maximum(np.abs(a).max(2), np.float32(1e-5)) / np.float32(7)
                z = np.full((N, K // g), 8, np.int64)
            q = np.clip(np.rint(a / s[:, :, None]) + z[:, :, None], 0, 15).astype(np.uint8)
            return q.reshape(N, K), s16, z

        mp.setattr(O, "quantize", quantize)
    elif name == "zero_sign_flipped":
        orig = O.group_params

        def gp(W16, g, zero_point):
            s16, z = orig(W16, g, zero_point)
            return s16, (15 - z) if zero_point else z

        mp.setattr(O, "group_params", gp)
    elif name == "dequant_drops_zero":
        def dq(q, s16, z, g):
            N, K = q.shape
            return (q.astype(np.float64).reshape(N, K // g, g) * s16.astype(np.float64)[:, :, None]).reshape(N, K)

        mp.setattr(O, "dequant", dq)
    elif name == "matmul_wrong_operand_index":
        def mm(X16, Wdq):
            X = X16.astype(np.float64)
            W = np.asarray(Wdq, dtype=np.float64)
            Wt = W.T.reshape(W.shape) if W.shape[0] == W.shape[1] else W[::-1]
            return X @ Wt.T, np.abs(X) @ np.abs(Wt).T

        mp.setattr(O, "matmul_ref", mm)
    elif name == "recon_loss_scales_x_by_s":
        orig_fq = O.fake_quant

        def rl(W16, X, s, g, zero_point):
            s = np.asarray(s, dtype=np.float32)
            Ws16 = (W16.astype(np.float32) * s[None, :]).astype(np.float16)
            Wq = orig_fq(Ws16, g, zero_point)
            Xs = np.asarray(X, dtype=np.float64) * s.astype(np.float64)[None, :]
            ref = np.asarray(X, dtype=np.float64) @ W16.astype(np.float64).T
            return float(np.linalg.norm(Xs @ Wq.T - ref))

        mp.setattr(O, "recon_loss", rl)
    elif name == "act_stat_max_not_mean":
        mp.setattr(O, "activation_scale",
                   lambda X16: np.maximum(np.abs(np.asarray(X16, np.float64)).max(axis=0), O.ACT_FLOOR))
    elif name == "candidate_inverse_power":
        mp.setattr(O, "scale_candidates", lambda X16, alphas: np.stack(
            [np.power(O.activation_scale(X16), -float(al)).astype(np.float32) for al in alphas]))
    elif name == "search_keeps_largest_loss":
        orig_search = O.search_scale

        def search(W16, X16, g, zero_point, alphas):
            _, S, losses = orig_search(W16, X16, g, zero_point, alphas)
            return int(np.argmax(losses)), S, losses

        mp.setattr(O, "search_scale", search)
    elif name == "duo_weight_power_flipped":
        orig_sc = O.scale_candidates

        def sc(X16, alphas, W16=None):
            if W16 is None:
                return orig_sc(X16, alphas)
            a, b = O.activation_scale(X16), O.weight_scale(W16)
            return np.stack([(np.power(a, al) * np.power(b, 1.0 - al)).astype(np.float32) for al in alphas])

        mp.setattr(O, "scale_candidates", sc)
    elif name == "weight_stat_max_not_mean":
        mp.setattr(O, "weight_scale",
                   lambda W16: np.maximum(np.abs(np.asarray(W16, np.float64)).max(axis=0), O.WEIGHT_FLOOR))
    elif name == "scale_weights_divides":
        mp.setattr(O, "scale_weights", lambda W16, s: (W16.astype(np.float32) / np.asarray(s, np.float32)[None, :])
                   .astype(np.float32).astype(np.float16))
    elif name == "clip_low_bound_unscaled":
        def cw(W16, g, zero_point, ratio):
            N, K = W16.shape
            a = W16.astype(np.float32).reshape(N, K // g, g)
            r = np.broadcast_to(np.asarray(ratio, dtype=np.float32), (N, K // g))[:, :, None]
            hi = (r * (a.max(axis=2) if zero_point else np.abs(a).max(axis=2))[:, :, None]).astype(np.float32)
            lo = a.min(axis=2)[:, :, None] if zero_point else -hi
            return np.minimum(np.maximum(a, lo), hi).astype(np.float16).reshape(N, K)

        mp.setattr(O, "clip_weight", cw)
    elif name == "clip_error_against_clipped_weight":
        def ce(W16, X16, g, zero_point, ratios):
            N, K = W16.shape
            X = np.asarray(X16, dtype=np.float64)
            out = np.empty((len(ratios), N, K // g))
            for i, r in enumerate(ratios):
                Wc = O.clip_weight(W16, g, zero_point, r)
                E = O.fake_quant(Wc, g, zero_point) - Wc.astype(np.float64)
                for j in range(K // g):
                    Y = X[:, j * g:(j + 1) * g] @ E[:, j * g:(j + 1) * g].T
                    out[i, :, j] = (Y * Y).sum(axis=0)
            return out

        mp.setattr(O, "clip_errors", ce)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    assert not _some_check_fails(), "pins must pass on the unmodified oracle"
    if MUTATIONS[name] is not None:
        MUTATIONS[name](monkeypatch)
    else:
        _patch_function(monkeypatch, name)
    assert _some_check_fails(), f"planted mistake {name!r} went undetected"
