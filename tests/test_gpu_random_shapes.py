"""Seeded random shapes through every launch path: awq_pack on the GPU against
the oracle (bit-exact), then awq_gemm (and awq_gemv up to 8 tokens) on the packed
weights against the oracle's fp64 product (per-element tolerance).  The token
counts are drawn per kernel regime: 1, 2-8, 9-16, 17-32, 33-64 on narrow and on
wide (N >= 8192) layers, 65-300 and 301-1100; N, K and the group size are
drawn at random (N a multiple of 8, K a multiple of the group size), so ragged
tiles, ragged K steps and K splits all occur."""
from __future__ import annotations

import numpy as np
import pytest

import workloads
from oracle import awq_oracle as O
from tests import _gpu as G

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

REGIMES = [(1, 1), (2, 8), (9, 16), (17, 32), (33, 64), (65, 300), (301, 1100)]


def _cases(n_per_regime=4, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for lo, hi in REGIMES:
        for i in range(n_per_regime):
            M = int(rng.integers(lo, hi + 1))
            g = int(rng.choice([32, 64, 128, 256]))
            zp = bool(rng.integers(0, 2))
            if lo == 33 and i % 2 == 1:  # 33-64 tokens on a wide layer: the 64-row matrix-core tiles
                N = 8 * int(rng.integers(1024, 1101))
                K = g * int(rng.integers(1, max(2, 640 // g) + 1))
            else:
                N = 8 * int(rng.integers(1, 201))
                K = g * int(rng.integers(1, 3072 // g + 1))
            out.append((M, N, K, g, zp, int(rng.integers(0, 1 << 30))))
    return out


@pytest.mark.parametrize("M,N,K,g,zp,seed", _cases())
def test_random_shape_pack_and_products(M, N, K, g, zp, seed):
    awq = G.lib()
    W = workloads.weight(N, K, cfg=9, layer=seed % 1000, row_offset=bool(seed & 1))
    X = workloads.activations(M, K, cfg=9, layer=seed % 1000)
    what = f"M={M} N={N} K={K} g={g} zp={zp}"
    qw, sc, qz = awq.awq_pack(G.dev_f16(W), g, zp)
    oq, os_, oz = O.pack(W, g, zp)
    assert np.array_equal(G.host_u32(qw), oq), what
    assert np.array_equal(G.host_f16_bits(sc), os_), what
    if zp:
        assert np.array_equal(G.host_u32(qz), oz), what
    y_ref, d = O.matmul_ref(X, O.dequant_packed(oq, os_, oz, N, K, g, zp))
    x = G.dev_f16(X)
    y = G.host_f16(awq.awq_gemm(x, qw, sc, qz, N, K, g, zp))
    G.assert_within_tolerance(y, y_ref, d, "gemm " + what)
    if M <= 8:
        y = G.host_f16(awq.awq_gemv(x, qw, sc, qz, N, K, g, zp))
        G.assert_within_tolerance(y, y_ref, d, "gemv " + what)
