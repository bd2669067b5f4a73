"""Fused projections: several weights that read the same input packed as one
weight (q/k/v, gate/up) give bit-identical packed data to the separate layers,
outputs bit-identical to theirs for a few tokens (same kernels and plans) and
within tolerance of the oracle for any number of tokens."""
from __future__ import annotations

import numpy as np
import pytest

import workloads
from oracle import awq_oracle as O
from tests import _gpu as G

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _parts(shapes, K, cfg):
    return [workloads.weight(N, K, cfg=cfg, layer=i) for i, N in enumerate(shapes)]


@pytest.mark.parametrize("zp", [True, False])
@pytest.mark.parametrize("shapes,K,g", [((4096, 4096, 4096), 4096, 128), ((11008, 11008), 4096, 128),
                                        ((24, 40, 8), 512, 32)])
def test_fused_pack_and_layers_match_separate(shapes, K, g, zp):
    awq = G.lib()
    Ws = _parts(shapes, K, cfg=6)
    dev = [G.dev_f16(W) for W in Ws]
    fused = awq.pack_fused(dev, g, zp)
    sep = [awq.pack(w, g, zp) for w in dev]
    torch.cuda.synchronize()
    assert np.array_equal(G.host_u32(fused.qweight), np.concatenate([G.host_u32(p.qweight) for p in sep]))
    assert np.array_equal(G.host_f16_bits(fused.scales), np.concatenate([G.host_f16_bits(p.scales) for p in sep]))
    if zp:
        assert np.array_equal(G.host_u32(fused.qzeros), np.concatenate([G.host_u32(p.qzeros) for p in sep]))
    oq, os_, oz = O.pack(np.concatenate(Ws), g, zp)
    wdq = O.dequant_packed(oq, os_, oz, sum(shapes), K, g, zp)
    for M in (1, 4, 300):
        X = workloads.activations(M, K, cfg=6, layer=M)
        x = G.dev_f16(X)
        yf = G.host_f16(awq.linear(x, fused))
        ys = np.concatenate([G.host_f16(awq.linear(x, p)) for p in sep], axis=1)
        torch.cuda.synchronize()
        if M <= 4:
            # same kernels and launch plans per row: bit-identical
            assert np.array_equal(yf.view(np.uint16), ys.view(np.uint16)), M
        # larger M may split K differently for the fused and the separate N:
        # both within tolerance of the exact product
        rows = np.arange(M) if M <= 4 else np.sort(np.random.default_rng(M).choice(M, 12, replace=False))
        y_ref, d = O.matmul_ref(X[rows], wdq)
        G.assert_within_tolerance(yf[rows], y_ref, d, f"fused M={M}")
        G.assert_within_tolerance(ys[rows], y_ref, d, f"separate M={M}")


@pytest.mark.parametrize("zp", [True, False])
def test_fused_octets_match_separate_quads(zp):
    """A fused layer wide enough for the GEMV's row octets (4096 -> 2 x 16384:
    4096 octets x 2 waves) against its two parts, which run on row quads: the
    octet and quad reductions add every row in the same order, so the outputs
    are bit-identical; sampled octets are checked against the oracle."""
    awq = G.lib()
    K, g, shapes = 4096, 128, (16384, 16384)
    Ws = _parts(shapes, K, cfg=7)
    dev = [G.dev_f16(W) for W in Ws]
    fused = awq.pack_fused(dev, g, zp)
    sep = [awq.pack(w, g, zp) for w in dev]
    X = workloads.activations(1, K, cfg=7, layer=1)
    x = G.dev_f16(X)
    yf = G.host_f16(awq.linear(x, fused))
    ys = np.concatenate([G.host_f16(awq.linear(x, p)) for p in sep], axis=1)
    torch.cuda.synchronize()
    assert np.array_equal(yf.view(np.uint16), ys.view(np.uint16))
    N = sum(shapes)
    octets = np.sort(np.random.default_rng(7).choice(N // 8, size=16, replace=False))
    rows = (octets[:, None] * 8 + np.arange(8)[None, :]).reshape(-1)
    W = np.concatenate(Ws)[rows]
    wdq = O.dequant_packed(*O.pack(W, g, zp), len(rows), K, g, zp)
    y_ref, d = O.matmul_ref(X, wdq)
    G.assert_within_tolerance(yf[:, rows], y_ref, d, f"fused octets zp={zp}")
