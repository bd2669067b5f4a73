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


@pytest.mark.parametrize("duo", [False, True])
@pytest.mark.parametrize("M,K", [(1, 8), (64, 512), (300, 4096), (129, 11008)])
def test_scale_candidates_match_oracle(M, K, duo):
    awq = G.lib()
    X = workloads.activations(M, K, cfg=6, layer=K)
    W = workloads.weight(72, K, cfg=6, layer=K, row_offset=True)
    W[:, 3] = 0  # an all-zero weight channel takes the floor
    alphas = [0.0, 0.05, 0.25, 0.5, 0.95, 1.0]
    s = awq.awq_scale_candidates(G.dev_f16(X), alphas, G.dev_f16(W) if duo else None).cpu().numpy()
    ref = O.scale_candidates(X, alphas, W if duo else None)
    assert s.shape == ref.shape and s.dtype == np.float32
    if not duo:
        assert np.array_equal(s[0], np.ones(K, np.float32))
    # fp32 sums in row order and powf against fp64 means and powers
    assert np.max(np.abs(s.astype(np.float64) / ref.astype(np.float64) - 1)) <= 1e-5


@pytest.mark.parametrize("zp", [True, False])
@pytest.mark.parametrize("M,N,K,g", [(64, 256, 512, 64), (37, 264, 2080, 32), (1, 8, 256, 256),
                                     (130, 1032, 1024, 128), (256, 512, 4096, 128),
                                     (600, 256, 512, 64), (1100, 136, 1056, 32)])
def test_scale_loss_matches_oracle(M, N, K, g, zp):
    """(600 and 1100 tokens: two and three 512-token tiles, the last ragged.)"""
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


def check_choice(got_losses, got_best, losses, best, what):
    """The device's losses within tolerance of the oracle's, and its choice the
    oracle's unless the two best candidates are within twice the tolerance
    (then any candidate that close to the best is a correct choice)."""
    losses = np.array(losses)
    assert np.all(np.abs(got_losses - losses) <= LOSS_TOL * losses), what
    order = np.argsort(losses, kind="stable")
    if losses[order[1]] - losses[order[0]] > 2 * LOSS_TOL * losses[order[0]]:
        assert got_best == best, (what, got_best, best)
    else:
        assert losses[got_best] <= losses[order[0]] * (1 + 2 * LOSS_TOL), what


@pytest.mark.parametrize("duo", [False, True])
@pytest.mark.parametrize("zp", [True, False])
def test_search_scale_end_to_end(zp, duo):
    """awq_scale_search (candidates, losses and the choice, all on the device)
    against the oracle's search; the chosen scale vector is the chosen
    candidate's, bit for bit."""
    awq = G.lib()
    N, K, M, g = 512, 1024, 64, 128
    W = workloads.weight(N, K, cfg=6, layer=3)
    X = workloads.activations(M, K, cfg=6, layer=3)
    alphas = [i / 20 for i in range(20)]
    x, w = G.dev_f16(X), G.dev_f16(W)
    res = awq.search_scale(x, w, g, zp, alphas, duo=duo)
    cands = awq.awq_scale_candidates(x, alphas, w if duo else None)
    torch.cuda.synchronize()
    best, S, losses = O.search_scale(W, X, g, zp, alphas, duo=duo)
    i = int(res.best.cpu().item())
    check_choice(res.losses.cpu().numpy(), i, losses, best, f"zp={zp} duo={duo}")
    assert res.alpha == alphas[i]
    assert torch.equal(res.scale, cands[i])
    assert np.max(np.abs(res.scale.cpu().numpy() / S[i] - 1)) <= 1e-5
    assert losses[best] < losses[0] * (0.8 if not duo else 1.0), "scaling must beat plain rounding here"


@pytest.mark.parametrize("zp", [True, False])
@pytest.mark.parametrize("N,K,g", [(264, 1024, 32), (264, 4096, 128), (40, 11008, 64), (8, 512, 256)])
def test_scale_loss_group_params_bit_exact(N, K, g, zp):
    """The group scales and zero points the loss product quantizes with, read
    from the first region of the caller's workspace ([count][K/g][N] words of
    fp16 scale bits | zero point << 16), against the oracle's group_params of
    scale_weights(W, s_c) for every candidate, bit for bit.  N = 264 and 40 end
    in a partial band of rows, K = 4096 and 11008 span several K slices."""
    awq = G.lib()
    lib = awq.load_library()
    M = 24
    W = workloads.weight(N, K, cfg=6, layer=N + g, row_offset=True)
    X = workloads.activations(M, K, cfg=6, layer=N + g)
    S = np.stack([np.ones(K, np.float32)] + list(O.scale_candidates(X, [0.25, 0.5, 0.75])) +
                 list(O.scale_candidates(X, [0.4], W)))
    count = len(S)
    x, w, s = G.dev_f16(X), G.dev_f16(W), torch.from_numpy(np.ascontiguousarray(S)).cuda()
    ws = torch.zeros(int(lib.awq_scale_loss_workspace_bytes(count, M, N, K)), dtype=torch.uint8, device="cuda")
    loss = torch.empty(count, dtype=torch.float64, device="cuda")
    st = lib.awq_scale_loss(awq._ptr(x), awq._ptr(w), awq._ptr(s), count, M, N, K, g, int(zp), awq._ptr(ws),
                            ws.numel(), awq._ptr(loss), awq._stream(x))
    assert st == 0, awq.awq_strerror(st)
    torch.cuda.synchronize()
    G_ = K // g
    gp = ws[: count * G_ * N * 4].cpu().numpy().view(np.uint32).reshape(count, G_, N)
    for c in range(count):
        s16, z = O.group_params(O.scale_weights(W, S[c]), g, zp)
        want = s16.view(np.uint16).astype(np.uint32) | (z.astype(np.uint32) << 16)
        assert np.array_equal(gp[c].T, want), (c, int(np.count_nonzero(gp[c].T != want)))


@pytest.mark.parametrize("zp", [True, False])
@pytest.mark.parametrize("g", [32, 128])
def test_scaled_weight_codes_bit_exact(g, zp):
    """The quantizer on scaled weights: awq_scale_columns (fp16 of the fp32
    product W * s) then awq_pack, against the oracle's pack of
    scale_weights(W, s), bit for bit, for an activation-only and a duo
    candidate."""
    awq = G.lib()
    N, K, M = 264, 1024, 48
    W = workloads.weight(N, K, cfg=6, layer=11, row_offset=True)
    X = workloads.activations(M, K, cfg=6, layer=11)
    for s in (O.scale_candidates(X, [0.5])[0], O.scale_candidates(X, [0.3], W)[0]):
        ws = awq.awq_scale_columns(G.dev_f16(W), torch.from_numpy(s).cuda())
        assert np.array_equal(G.host_f16_bits(ws), O.scale_weights(W, s).view(np.uint16))
        qw, sc, qz = awq.awq_pack(ws, g, zp)
        oq, os_, oz = O.pack(O.scale_weights(W, s), g, zp)
        assert np.array_equal(G.host_u32(qw), oq)
        assert np.array_equal(G.host_f16_bits(sc), os_)
        if zp:
            assert np.array_equal(G.host_u32(qz), oz)


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


def test_scale_search_full_size_llama7b_duo():
    """awq_scale_search with duo scaling on a Llama-7B q_proj, 256 tokens,
    four candidates: losses and choice against the oracle."""
    awq = G.lib()
    N = K = 4096
    M, g = 256, 128
    W = workloads.weight(N, K, cfg=6, layer=8)
    X = workloads.activations(M, K, cfg=6, layer=8)
    alphas = [0.2, 0.4, 0.6, 0.8]
    res = awq.awq_scale_search(G.dev_f16(X), G.dev_f16(W), g, True, alphas, duo=True)
    best, S, losses = O.search_scale(W, X, g, True, alphas, duo=True)
    check_choice(res.losses.cpu().numpy(), int(res.best.cpu().item()), losses, best, "7B duo")


def test_scale_loss_deterministic():
    N, K, M, g = 520, 2048, 200, 128
    W = workloads.weight(N, K, cfg=6, layer=9)
    X = workloads.activations(M, K, cfg=6, layer=9)
    S = O.scale_candidates(X, [0.0, 0.3, 0.6])
    a = gpu_losses(X, W, S, g, True)
    b = gpu_losses(X, W, S, g, True)
    assert np.array_equal(a, b)
