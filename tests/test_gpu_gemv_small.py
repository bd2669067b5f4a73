"""The few-token kernel (2-8 tokens, through awq_gemv and awq_gemm) against the
oracle's fp64 product of the decoded weights: |y - y_ref| <= 1e-3 * sum_k
|x_k w'_k| for every output, at every token count, group size and zero-point
mode, on ragged row tiles (N % 16 == 8), ragged K (sub-chunks of 512 channels
cut short), K long enough to take several rounds, the full-size Llama-7B
shapes at every M from 1 to 8, and sampled 70B-shaped layers; one-hot inputs
reproduce fp16(w') bit-exactly; both entry points give the same bits."""
from __future__ import annotations

import numpy as np
import pytest

import workloads
from oracle import awq_oracle as O
from tests import _gpu as G

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def both_entry_points(X16, dev_packed, N, K, g, zp):
    """awq_gemv and awq_gemm on the same inputs: the same kernel, so the same bits."""
    awq = G.lib()
    x = G.dev_f16(X16)
    a = awq.awq_gemv(x, *dev_packed, N, K, g, zp)
    b = awq.awq_gemm(x, *dev_packed, N, K, g, zp)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)), "awq_gemv and awq_gemm differ"
    return G.host_f16(a)


def check(M, N, K, g, zp, W=None, X=None, what=""):
    if W is None:
        W = workloads.weight(N, K, cfg=8, layer=N + K, row_offset=True)
    if X is None:
        X = workloads.activations(M, K, cfg=8, layer=N + K)
    packed = O.pack(W, g, zp)
    y = both_entry_points(X, G.upload_packed(*packed), N, K, g, zp)
    y_ref, d = O.matmul_ref(X, O.dequant_packed(*packed, N, K, g, zp))
    return G.assert_within_tolerance(y, y_ref, d, what or f"small M={M} N={N} K={K} g={g} zp={zp}")


@pytest.mark.parametrize("zp", [True, False])
@pytest.mark.parametrize("g", [32, 64, 128, 256])
@pytest.mark.parametrize("M", [2, 3, 4, 5, 6, 7, 8])
def test_small_m_group_sizes_ragged(M, g, zp):
    """N = 264 ends in a half tile (8 of 16 rows); K = 2304 is 4.5 sub-chunks."""
    check(M, 264, 2304, g, zp)


@pytest.mark.parametrize("M", [2, 5, 8])
@pytest.mark.parametrize("N,K,g", [(8, 32, 32), (8, 96, 32), (16, 512, 64), (24, 544, 32), (8, 256, 256)])
def test_small_m_minimal_shapes(M, N, K, g):
    check(M, N, K, g, True)
    check(M, N, K, g, False)


@pytest.mark.parametrize("M", [3, 7])
@pytest.mark.parametrize("N,K,g", [(40, 30720, 256), (264, 12800, 128), (16, 28672, 128)])
def test_small_m_several_rounds(M, N, K, g):
    """K past one round of sub-chunks (24 per round: 12 waves x 2 up to 4
    tokens, 8 waves x 3 above): 2-3 rounds, the last one partial."""
    check(M, N, K, g, True)


@pytest.mark.parametrize("name,K,N", [workloads.LLAMA7B_BLOCK[0], workloads.LLAMA7B_BLOCK[4],
                                      workloads.LLAMA7B_BLOCK[6]])
def test_small_m_llama7b_full_size_every_m(name, K, N):
    """The Llama-7B decode shapes at full size, every token count from 1 to 8
    (M = 1: the single-token kernel; 2-8: the few-token kernel), every output."""
    layer = [n for n, _, _ in workloads.LLAMA7B_BLOCK].index(name)
    W = workloads.weight(N, K, cfg=3, layer=layer)
    packed = O.pack(W, 128, True)
    dev = G.upload_packed(*packed)
    wdq = O.dequant_packed(*packed, N, K, 128, True)
    for M in range(1, 9):
        X = workloads.activations(M, K, cfg=3, layer=layer)
        y = both_entry_points(X, dev, N, K, 128, True)
        y_ref, d = O.matmul_ref(X, wdq)
        G.assert_within_tolerance(y, y_ref, d, f"{name} M={M}")


@pytest.mark.parametrize("M", [4, 8])
@pytest.mark.parametrize("name,K,N", workloads.LLAMA70B_MLP)
def test_small_m_70b_sampled(M, name, K, N):
    """The 70B MLP shapes (K = 28672: three rounds at 8 tokens), GPU-packed;
    the oracle checks sampled row octets of the packing and of the output."""
    awq = G.lib()
    g = 128
    layer = 0 if K == 8192 else 1
    W = workloads.weight(N, K, cfg=4, layer=layer)
    X = workloads.activations(M, K, cfg=4, layer=layer)
    w = G.dev_f16(W)
    qw, sc, qz = awq.awq_pack(w, g, True)
    del w
    y = G.host_f16(awq.awq_gemv(G.dev_f16(X), qw, sc, qz, N, K, g, True))
    rng = np.random.default_rng(M)
    octets = np.sort(rng.choice(N // 8, size=12, replace=False))
    rows = (octets[:, None] * 8 + np.arange(8)[None, :]).reshape(-1)
    oq, os_, oz = O.pack(W[rows], g, True)
    assert np.array_equal(G.host_u32(qw)[rows], oq)
    assert np.array_equal(G.host_f16_bits(sc)[octets], os_)
    assert np.array_equal(G.host_u32(qz)[octets], oz)
    y_ref, d = O.matmul_ref(X, O.dequant_packed(oq, os_, oz, len(rows), K, g, True))
    G.assert_within_tolerance(y[:, rows], y_ref, d, f"small {name} M={M}")


@pytest.mark.parametrize("zp", [True, False])
@pytest.mark.parametrize("M", [2, 4, 5, 8])
def test_small_m_one_hot_reproduces_decoded_weights(M, zp):
    """Token m is one-hot at channel k_m: y[m] = fp16(w'[:, k_m]) bit for bit
    (the slice sum is the exact q - z, times the scale, rounded once)."""
    N, K, g = 136, 1024, 32
    W = workloads.adversarial_weight(N, K, g, seed=13)
    packed = O.pack(W, g, zp)
    wdq = O.dequant_packed(*packed, N, K, g, zp).astype(np.float16)
    ks = np.random.default_rng(M).choice(K, size=M, replace=False)
    X = np.zeros((M, K), np.float16)
    X[np.arange(M), ks] = 1
    y = both_entry_points(X, G.upload_packed(*packed), N, K, g, zp)
    assert np.array_equal(y.astype(np.float64), wdq[:, ks].T.astype(np.float64))


def test_small_m_zero_tokens_and_adversarial_weights():
    """Zero token rows give exact zeros next to non-zero ones; adversarial
    groups (ties, subnormals, saturating ranges, |w| up to 6e4) stay within
    tolerance."""
    N, K, g = 72, 1024, 32
    W = workloads.adversarial_weight(N, K, g, seed=5)
    X = (workloads.activations(6, K, cfg=9, layer=0).astype(np.float32) / 64).astype(np.float16)
    X[1] = 0
    X[4] = 0
    for zp in (True, False):
        packed = O.pack(W, g, zp)
        y = both_entry_points(X, G.upload_packed(*packed), N, K, g, zp)
        assert np.all(y[1] == 0) and np.all(y[4] == 0)
        y_ref, d = O.matmul_ref(X, O.dequant_packed(*packed, N, K, g, zp))
        G.assert_within_tolerance(y, y_ref, d, f"adversarial zp={zp}")


def test_small_m_deterministic_and_stream():
    awq = G.lib()
    N, K, g = 4096, 4096, 128
    W = workloads.weight(N, K, cfg=2, layer=0)
    X = workloads.activations(6, K, cfg=2, layer=0)
    dev = G.upload_packed(*O.pack(W, g, True))
    x = G.dev_f16(X)
    a = awq.awq_gemv(x, *dev, N, K, g, True)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        b = awq.awq_gemv(x, *dev, N, K, g, True)
    s.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
