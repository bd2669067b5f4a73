"""Activation-aware scale search on the GPU against the oracle: candidate
scales (awq_scale_candidates) and the reconstruction error L(s)
(awq_scale_loss) for ragged and full-size shapes, exact special cases, and
the search end to end."""
from __future__ import annotations

import numpy as np
import pytest

import workloads
from oracle import awq_oracle as O
from tests import _gpu as G

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

LOSS_TOL = 1e-3  # |L_gpu - L_ref| <= 1e-3 * L_ref (fp16 weight error, fp32 accumulation)


def gpu_losses(X16, W16, S, g, zp):
    awq = G.lib()
    loss = awq.awq_scale_loss(G.dev_f16(X16), G.dev_f16(W16), torch.from_numpy(np.ascontiguousarray(S)).cuda(), g, zp)
    torch.cuda.synchronize()
    return loss.cpu().numpy()


@pytest.mark.parametrize("M,K", [(1, 8), (64, 512), (300, 4096), (129, 11008)])
def test_scale_candidates_match_oracle(M, K):
    awq = G.lib()
    X = workloads.activations(M, K, cfg=6, layer=K)
    alphas = [0.0, 0.05, 0.25, 0.5, 0.95, 1.0]
    s = awq.awq_scale_candidates(G.dev_f16(X), alphas).cpu().numpy()
    ref = O.scale_candidates(X, alphas)
    assert s.shape == ref.shape and s.dtype == np.float32
    assert np.array_equal(s[0], np.ones(K, np.float32))
    # fp32 sum in row order and powf against fp64 mean and power
    assert np.max(np.abs(s.astype(np.float64) / ref.astype(np.float64) - 1)) <= 1e-5


@pytest.mark.parametrize("zp", [True, False])
@pytest.mark.parametrize("M,N,K,g", [(64, 256, 512, 64), (37, 264, 2080, 32), (1, 8, 256, 256),
                                     (130, 1032, 1024, 128), (256, 512, 4096, 128)])
def test_scale_loss_matches_oracle(M, N, K, g, zp):
    W = workloads.weight(N, K, cfg=6, layer=N, row_offset=True)
    X = workloads.activations(M, K, cfg=6, layer=N)
    rng = np.random.default_rng(N + K)
    S = np.stack([np.ones(K, np.float32), rng.uniform(0.5, 2.0, K).astype(np.float32),
                  O.scale_candidates(X, [0.5])[0]])
    got = gpu_losses(X, W, S, g, zp)
    for c in range(len(S)):
        ref = O.recon_loss(W, X, S[c], g, zp)
        assert ref > 0
        assert abs(got[c] - ref) <= LOSS_TOL * ref, (c, got[c], ref)


def test_scale_loss_exact_cases():
    """Weights on a full-span 4-bit grid with s = 1 give L = 0 exactly; scales
    that are a power of two per group give exactly L(1)."""
    N, K, g = 64, 512, 64
    rng = np.random.default_rng(5)
    q = rng.integers(0, 16, size=(N, K))
    q[:, ::g] = 0
    q[:, 1::g] = 15
    sc = (2.0 ** rng.integers(-8, -3, size=(N, K // g))).astype(np.float16)
    z = rng.integers(0, 16, size=(N, K // g))
    Wg = ((q.reshape(N, K // g, g) - z[:, :, None]) * sc.astype(np.float64)[:, :, None]).reshape(N, K)
    Wg = Wg.astype(np.float16)
    X = workloads.activations(32, K, cfg=6, layer=1)
    e = rng.integers(-2, 3, size=K // g)
    S = np.stack([np.ones(K, np.float32), np.repeat(np.exp2(e.astype(np.float64)), g).astype(np.float32)])
    got = gpu_losses(X, Wg, S, g, True)
    assert got[0] == 0.0 and got[1] == 0.0
    W = workloads.weight(N, K, cfg=6, layer=2)
    got = gpu_losses(X, W, S, g, True)
    assert got[0] > 0 and got[1] == got[0]


@pytest.mark.parametrize("zp", [True, False])
def test_search_scale_end_to_end(zp):
    """The GPU search (candidates, losses, smallest loss) against the oracle's:
    same losses within tolerance and the same choice unless the two best
    candidates are within tolerance of each other."""
    awq = G.lib()
    N, K, M, g = 512, 1024, 64, 128
    W = workloads.weight(N, K, cfg=6, layer=3)
    X = workloads.activations(M, K, cfg=6, layer=3)
    alphas = [i / 20 for i in range(20)]
    res = awq.search_scale(G.dev_f16(X), G.dev_f16(W), g, zp, alphas)
    best, S, losses = O.search_scale(W, X, g, zp, alphas)
    got = np.array(res.losses)
    assert np.all(np.abs(got - np.array(losses)) <= LOSS_TOL * np.array(losses))
    i = alphas.index(res.alpha)
    order = np.argsort(losses)
    if losses[order[1]] - losses[order[0]] > 2 * LOSS_TOL * losses[order[0]]:
        assert i == best
    else:
        assert losses[i] <= losses[order[0]] * (1 + 2 * LOSS_TOL)
    assert losses[best] < losses[0], "scaling the outlier channels must beat plain rounding here"
    assert np.max(np.abs(res.scale.cpu().numpy() / S[i] - 1)) <= 1e-5


def test_scale_loss_full_size_llama7b():
    """A Llama-7B q_proj (4096 x 4096) with 256 calibration tokens, two candidates."""
    N = K = 4096
    M, g = 256, 128
    W = workloads.weight(N, K, cfg=6, layer=7)
    X = workloads.activations(M, K, cfg=6, layer=7)
    S = O.scale_candidates(X, [0.0, 0.5])
    got = gpu_losses(X, W, S, g, True)
    for c in range(2):
        ref = O.recon_loss(W, X, S[c], g, True)
        assert abs(got[c] - ref) <= LOSS_TOL * ref, (c, got[c], ref)


def test_scale_loss_deterministic():
    N, K, M, g = 520, 2048, 200, 128
    W = workloads.weight(N, K, cfg=6, layer=9)
    X = workloads.activations(M, K, cfg=6, layer=9)
    S = O.scale_candidates(X, [0.0, 0.3, 0.6])
    a = gpu_losses(X, W, S, g, True)
    b = gpu_losses(X, W, S, g, True)
    assert np.array_equal(a, b)
