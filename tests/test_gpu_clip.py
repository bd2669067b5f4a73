"""Weight clipping (awq_clip_search), per-channel scaling (awq_scale_columns)
and the whole activation-aware quantization of a layer (scale search, scaling,
clipping, packing) on the GPU against the oracle."""
from __future__ import annotations

import numpy as np
import pytest

import workloads
from oracle import awq_oracle as O
from tests import _gpu as G

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

ERR_TOL = 2e-3  # relative error of the GPU's group errors (fp16 weight error, fp32 sums)
RATIOS = [1.0 - 0.025 * i for i in range(20)]


def check_choices(gpu_choice, gpu_wc, W, X, g, zp, ratios):
    best, Wc, err = O.search_clip(W, X, g, zp, ratios)
    N, Gn = best.shape
    n, j = np.meshgrid(np.arange(N), np.arange(Gn), indexing="ij")
    e_best = err[best, n, j]
    e_gpu = err[gpu_choice, n, j]
    # the GPU's choice is the oracle's, or within the GPU's error of the best
    assert np.all(e_gpu <= e_best * (1 + 2 * ERR_TOL) + 1e-30), np.max(e_gpu / np.maximum(e_best, 1e-30))
    same = gpu_choice == best
    assert same.mean() > 0.9, same.mean()
    # where the choices agree, the clipped weights are bit-identical
    rows_same = np.repeat(same, g, axis=1)
    assert np.array_equal(gpu_wc.view(np.uint16)[rows_same], Wc.view(np.uint16)[rows_same])
    # elsewhere they are the oracle's clipping with the GPU's ratio
    Wg = O.clip_weight(W, g, zp, np.asarray(ratios, np.float32)[gpu_choice])
    assert np.array_equal(gpu_wc.view(np.uint16), Wg.view(np.uint16))


@pytest.mark.parametrize("zp", [True, False])
@pytest.mark.parametrize("N,K,g", [(264, 1024, 32), (40, 4096, 128), (8, 512, 256)])
def test_clip_group_params_bit_exact(N, K, g, zp):
    """Every ratio's group parameters as the loss product uses them, read from
    the first region of the caller's workspace ([count][K/g][N] pairs of words
    {fp16 scale bits | zero point << 16, fp16(lo) bits | fp16(hi) bits << 16}):
    the scale and zero point are the oracle's group_params of clip_weight(W,
    r) bit for bit, and clamping each fp16 weight of the group to [lo, hi]
    reproduces clip_weight(W, r) bit for bit."""
    awq = G.lib()
    lib = awq.load_library()
    M = 16
    W = workloads.weight(N, K, cfg=7, layer=N + g, row_offset=True)
    X = workloads.activations(M, K, cfg=7, layer=N + g)
    ratios = [1.0, 0.9, 0.725, 0.525]
    count, Gn = len(ratios), K // g
    x, w = G.dev_f16(X), G.dev_f16(W)
    out = torch.empty_like(w)
    # (a caller's choice buffer: without one the choices overwrite the start of the workspace)
    choice = torch.empty((N, Gn), dtype=torch.int32, device="cuda")
    ws = torch.zeros(int(lib.awq_clip_search_workspace_bytes(count, M, N, K, g)), dtype=torch.uint8, device="cuda")
    import ctypes
    arr = (ctypes.c_float * count)(*ratios)
    st = lib.awq_clip_search(awq._ptr(x), awq._ptr(w), M, N, K, g, int(zp), ctypes.cast(arr, ctypes.c_void_p), count,
                             awq._ptr(out), awq._ptr(choice), awq._ptr(ws), ws.numel(), awq._stream(x))
    assert st == 0, awq.awq_strerror(st)
    torch.cuda.synchronize()
    gp = ws[: count * Gn * N * 8].cpu().numpy().view(np.uint32).reshape(count, Gn, N, 2)
    for c, r in enumerate(ratios):
        Wc = O.clip_weight(W, g, zp, r)
        s16, z = O.group_params(Wc, g, zp)
        want = s16.view(np.uint16).astype(np.uint32) | (z.astype(np.uint32) << 16)
        assert np.array_equal(gp[c, :, :, 0].T, want), (r, int(np.count_nonzero(gp[c, :, :, 0].T != want)))
        lo = (gp[c, :, :, 1].T & 0xFFFF).astype(np.uint16).view(np.float16)
        hi = (gp[c, :, :, 1].T >> 16).astype(np.uint16).view(np.float16)
        a = W.reshape(N, Gn, g)
        clamped = np.minimum(np.maximum(a, lo[:, :, None]), hi[:, :, None]).reshape(N, K)
        assert np.array_equal(clamped.view(np.uint16), Wc.view(np.uint16)), r


@pytest.mark.parametrize("zp", [True, False])
@pytest.mark.parametrize("M,N,K,g", [(64, 256, 512, 64), (37, 264, 2080, 32), (130, 520, 1024, 128),
                                     (300, 256, 2048, 256), (1, 8, 128, 128), (700, 264, 1024, 128),
                                     (1030, 136, 544, 32)])
def test_clip_search_matches_oracle(M, N, K, g, zp):
    """(700 and 1030 tokens: two and three 512-token tiles, the last ragged;
    their per-group partial errors are added by the choice kernel.)"""
    awq = G.lib()
    W = workloads.weight(N, K, cfg=7, layer=N, row_offset=True)
    X = workloads.activations(M, K, cfg=7, layer=N)
    wc, choice = awq.awq_clip_search(G.dev_f16(X), G.dev_f16(W), g, zp, RATIOS)
    torch.cuda.synchronize()
    check_choices(choice.cpu().numpy(), G.host_f16(wc), W, X, g, zp, RATIOS)


def test_clip_ratio_one_is_identity():
    awq = G.lib()
    W = workloads.adversarial_weight(64, 512, 64, seed=3)
    X = workloads.activations(16, 512, cfg=7, layer=1)
    wc, choice = awq.awq_clip_search(G.dev_f16(X), G.dev_f16(W), 64, True, [1.0])
    assert np.array_equal(G.host_f16(wc).view(np.uint16), W.view(np.uint16))
    assert not choice.cpu().numpy().any()


def test_clip_search_full_size_llama7b_gate():
    """A Llama-7B gate_proj (4096 -> 11008) with 128 calibration tokens."""
    awq = G.lib()
    N, K, M, g = 11008, 4096, 128, 128
    W = workloads.weight(N, K, cfg=7, layer=4)
    X = workloads.activations(M, K, cfg=7, layer=4)
    ratios = [1.0, 0.9, 0.8, 0.7]
    wc, choice = awq.awq_clip_search(G.dev_f16(X), G.dev_f16(W), g, True, ratios)
    torch.cuda.synchronize()
    # the oracle on a sample of rows (errors of a group depend only on its row)
    rows = np.sort(np.random.default_rng(1).choice(N, size=64, replace=False))
    check_choices(choice.cpu().numpy()[rows], G.host_f16(wc)[rows], W[rows], X, g, True, ratios)


@pytest.mark.parametrize("divide", [False, True])
def test_scale_columns_exact(divide):
    awq = G.lib()
    X = workloads.activations(33, 1032, cfg=7, layer=5)
    s = np.random.default_rng(2).uniform(0.25, 4.0, 1032).astype(np.float32)
    out = G.host_f16(awq.awq_scale_columns(G.dev_f16(X), torch.from_numpy(s).cuda(), divide))
    x32 = X.astype(np.float32)
    ref = ((x32 / s) if divide else (x32 * s)).astype(np.float32).astype(np.float16)
    assert np.array_equal(out.view(np.uint16), ref.view(np.uint16))


@pytest.mark.parametrize("zp", [True, False])
def test_quantize_awq_end_to_end(zp):
    """Scale search, scaling, clipping and packing on the GPU.  The result is
    checked through the oracle: its packed weights decode to a layer whose
    reconstruction error on the calibration set is close to the oracle's own
    pipeline and well below plain rounding."""
    awq = G.lib()
    N, K, M, g = 512, 1024, 128, 128
    W = workloads.weight(N, K, cfg=7, layer=6)
    X = workloads.activations(M, K, cfg=7, layer=6)
    alphas = [i / 20 for i in range(20)]
    q = awq.quantize_awq(G.dev_f16(W), G.dev_f16(X), g, zp, alphas, RATIOS)
    torch.cuda.synchronize()
    s = q.input_scale.cpu().numpy()
    wq = O.dequant_packed(G.host_u32(q.packed.qweight), G.host_f16_bits(q.packed.scales),
                          G.host_u32(q.packed.qzeros) if zp else None, N, K, g, zp)
    Xd = X.astype(np.float64)
    ref = Xd @ W.astype(np.float64).T
    L_gpu = np.linalg.norm((Xd / s.astype(np.float64)) @ wq.T - ref)
    # the oracle's pipeline: same steps, its own candidates
    best, S, losses = O.search_scale(W, X, g, zp, alphas)
    s_o = S[best]
    Ws = (W.astype(np.float32) * s_o).astype(np.float32).astype(np.float16)
    Xs = (X.astype(np.float32) / s_o).astype(np.float32).astype(np.float16)
    _, Wc, _ = O.search_clip(Ws, Xs, g, zp, RATIOS)
    L_o = np.linalg.norm((Xd / s_o.astype(np.float64)) @ O.fake_quant(Wc, g, zp).T - ref)
    L_rtn = O.recon_loss(W, X, np.ones(K, np.float32), g, zp)
    assert L_gpu <= L_o * 1.01, (L_gpu, L_o)
    assert L_gpu < 0.7 * L_rtn, (L_gpu, L_rtn)
