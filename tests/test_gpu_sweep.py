"""Group-size / symmetry sweep at full size: the seven linears of one
Llama-7B-shaped block (weights with per-row mean offsets, so that zero points
matter) for g = 32 / 128 / 256 with and without zero points.  On sampled row
octets, the packed words, scales and zero points are bit-identical to the
oracle's, and the one-token GEMV and eight-token GEMM outputs are within
tolerance of the exact product with the oracle's decoded weights."""
from __future__ import annotations

import numpy as np
import pytest

import workloads
from oracle import awq_oracle as O
from tests import _gpu as G

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def block_weights():
    return [workloads.weight(N, K, cfg=5, layer=li, row_offset=True)
            for li, (_, K, N) in enumerate(workloads.LLAMA7B_BLOCK)]


@pytest.mark.parametrize("zp", [True, False])
@pytest.mark.parametrize("g", [32, 128, 256])
def test_sweep_block_sampled_rows(block_weights, g, zp):
    awq = G.lib()
    rng = np.random.default_rng([g, int(zp)])
    for li, (name, K, N) in enumerate(workloads.LLAMA7B_BLOCK):
        W = block_weights[li]
        qw, sc, qz = awq.awq_pack(G.dev_f16(W), g, zp)
        # quantization is independent per row: the oracle packs only the sampled octets
        octets = np.sort(rng.choice(N // 8, size=8, replace=False))
        rows = (octets[:, None] * 8 + np.arange(8)[None, :]).reshape(-1)
        oq, os_, oz = O.pack(W[rows], g, zp)
        what = f"{name} g={g} zp={zp}"
        assert np.array_equal(G.host_u32(qw)[rows], oq), f"{what}: packed words differ"
        assert np.array_equal(G.host_f16_bits(sc)[octets], os_), f"{what}: scales differ"
        if zp:
            assert np.array_equal(G.host_u32(qz)[octets], oz), f"{what}: zero points differ"
        wdq = O.dequant_packed(oq, os_, oz, len(rows), K, g, zp)
        for M in (1, 8):
            X = workloads.activations(M, K, cfg=5, layer=li)
            x = G.dev_f16(X)
            y = (awq.awq_gemv if M == 1 else awq.awq_gemm)(x, qw, sc, qz, N, K, g, zp)
            torch.cuda.synchronize()
            y_ref, d = O.matmul_ref(X, wdq)
            G.assert_within_tolerance(G.host_f16(y)[:, rows], y_ref, d, f"{what} M={M}")
