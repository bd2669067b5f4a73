"""The largest shapes the library takes (N, K up to 2^21): pack, the single-
and few-token GEMV and both GEMM kernels at K = 2^21 and at N = 2^21, where
the 32-bit buffer offsets of the kernels come closest to their limit.  Checked against the oracle (packing
bit-exact, products within tolerance on sampled rows)."""
from __future__ import annotations

import numpy as np
import pytest

import workloads
from oracle import awq_oracle as O
from tests import _gpu as G

pytestmark = [pytest.mark.gpu, pytest.mark.slow]
torch = pytest.importorskip("torch")

KMAX = 1 << 21


def _weights(N, K, seed):
    # row by row from the seeded generator would be slow at these sizes; one draw
    rng = np.random.default_rng([seed, N, K])
    return (rng.standard_normal((N, K), dtype=np.float32) / np.sqrt(K)).astype(np.float16)


def test_max_k_pack_gemv_gemm():
    awq = G.lib()
    N, K, g = 16, KMAX, 128
    W = _weights(N, K, 1)
    w = G.dev_f16(W)
    qw, sc, qz = awq.awq_pack(w, g, True)
    oq, os_, oz = O.pack(W, g, True)
    assert np.array_equal(G.host_u32(qw), oq)
    assert np.array_equal(G.host_f16_bits(sc), os_)
    assert np.array_equal(G.host_u32(qz), oz)
    del w
    wdq = O.dequant_packed(oq, os_, oz, N, K, g, True)
    # 2, 3 and 8 tokens: the few-token kernel, 171 rounds of sub-chunks at 8 tokens
    for M, fn in ((1, "gemv"), (2, "gemv"), (3, "gemm"), (8, "gemv"), (257, "gemm")):
        X = workloads.activations(M, K, cfg=8, layer=M)
        x = G.dev_f16(X)
        f = awq.awq_gemv if fn == "gemv" else awq.awq_gemm
        y = G.host_f16(f(x, qw, sc, qz, N, K, g, True))
        rows = np.arange(M) if M < 8 else np.sort(np.random.default_rng(M).choice(M, 8, replace=False))
        y_ref, d = O.matmul_ref(X[rows], wdq)
        G.assert_within_tolerance(y[rows], y_ref, d, f"{fn} M={M} K=2^21")
        del x


def test_max_n_pack_gemv_gemm():
    awq = G.lib()
    N, K, g = KMAX, 64, 32
    W = _weights(N, K, 2)
    w = G.dev_f16(W)
    qw, sc, qz = awq.awq_pack(w, g, True)
    del w
    oq, os_, oz = O.pack(W, g, True)
    assert np.array_equal(G.host_u32(qw), oq)
    assert np.array_equal(G.host_f16_bits(sc), os_)
    assert np.array_equal(G.host_u32(qz), oz)
    cols = np.sort(np.random.default_rng(3).choice(N // 8, 64, replace=False))
    cols = (cols[:, None] * 8 + np.arange(8)[None, :]).reshape(-1)
    cols = np.concatenate([cols, np.arange(N - 8, N)])  # the last octet
    wdq = O.dequant_packed(oq[cols], os_[cols[::8] // 8], oz[cols[::8] // 8], len(cols), K, g, True)
    for M, fn in ((1, "gemv"), (5, "gemm"), (8, "gemv"), (48, "gemm"), (300, "gemm")):
        X = workloads.activations(M, K, cfg=8, layer=M + 1)
        y = G.host_f16((awq.awq_gemv if fn == "gemv" else awq.awq_gemm)(G.dev_f16(X), qw, sc, qz, N, K, g, True))
        rows = np.arange(M) if M < 8 else np.sort(np.random.default_rng(M).choice(M, 8, replace=False))
        y_ref, d = O.matmul_ref(X[rows], wdq)
        G.assert_within_tolerance(y[np.ix_(rows, cols)], y_ref, d, f"{fn} M={M} N=2^21")
