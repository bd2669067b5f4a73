"""awq_gemv (batch 1) on the GPU against the oracle's fp64 product of the
decoded weights: |y - y_ref| <= 1e-3 * sum_k |x_k w'_k| for every output,
one-hot inputs reproduce fp16(w') bit-exactly, results are deterministic."""
from __future__ import annotations

import numpy as np
import pytest

import workloads
from oracle import awq_oracle as O
from tests import _gpu as G

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def run_gemv(X16, packed, N, K, g, zp, stream=None):
    awq = G.lib()
    dqw, dsc, dqz = G.upload_packed(*packed)
    x = G.dev_f16(X16)
    if stream is None:
        y = awq.awq_gemv(x, dqw, dsc, dqz, N, K, g, zp)
    else:
        with torch.cuda.stream(stream):
            y = awq.awq_gemv(x, dqw, dsc, dqz, N, K, g, zp)
        stream.synchronize()
    torch.cuda.synchronize()
    return G.host_f16(y)


def check_layer(N, K, g, zp, W=None, X=None, what=""):
    if W is None:
        W = workloads.weight(N, K, cfg=1, layer=N + K)
    if X is None:
        X = workloads.activations(1, K, cfg=1, layer=N + K)
    packed = O.pack(W, g, zp)
    y = run_gemv(X, packed, N, K, g, zp)
    y_ref, d = O.matmul_ref(X, O.dequant_packed(*packed, N, K, g, zp))
    return G.assert_within_tolerance(y, y_ref, d, what or f"gemv N={N} K={K} g={g} zp={zp}")


def test_gemv_tiny_layer():
    W = workloads.weight(512, 512, cfg=0, layer=0)
    X = workloads.activations(1, 512, cfg=0, layer=0)
    check_layer(512, 512, 128, True, W, X)


@pytest.mark.parametrize("zp", [True, False])
@pytest.mark.parametrize("g", [32, 64, 128, 256])
def test_gemv_group_sizes_and_symmetry(g, zp):
    W = workloads.weight(1024, 2048, cfg=5, layer=g, row_offset=True)
    check_layer(1024, 2048, g, zp, W=W)


@pytest.mark.parametrize("N,K,g", [(8, 32, 32), (8, 96, 32), (16, 160, 32), (8, 2304, 256), (40, 11008, 128),
                                   (24, 4128, 32), (8, 32768, 256), (16, 16416, 32), (24, 24608, 32)])
def test_gemv_ragged_and_minimal_shapes(N, K, g):
    """Minimal and ragged shapes; K = 16416 and 24608 are just past 512 and 768
    32-channel chunks, so the 12-wave workgroups run with most lanes idle, or
    with one chunk for most lanes and a second for a few."""
    check_layer(N, K, g, True)
    check_layer(N, K, g, False)


@pytest.mark.parametrize("N,K,g,zp", [(65536, 2048, 128, True), (32768, 2080, 32, False), (65536, 2048, 64, True),
                                      (65536, 2048, 256, False)])
def test_gemv_row_octets_full(N, K, g, zp):
    """Layers wide enough that the GEMV works on row octets instead of quads
    (8 rows per workgroup, the octet's scales in one 16-byte load, the
    eight-row register reduction), one with a ragged chunk count; every
    output is checked."""
    W = workloads.weight(N, K, cfg=5, layer=N + K, row_offset=True)
    check_layer(N, K, g, zp, W=W)


@pytest.mark.parametrize("name,K,N", workloads.LLAMA7B_BLOCK)
def test_gemv_llama7b_block_full_size(name, K, N):
    layer = [n for n, _, _ in workloads.LLAMA7B_BLOCK].index(name)
    W = workloads.weight(N, K, cfg=2, layer=layer)
    X = workloads.activations(1, K, cfg=2, layer=layer)
    check_layer(N, K, 128, True, W, X, f"gemv {name}")


@pytest.mark.parametrize("name,K,N", workloads.LLAMA70B_MLP)
def test_gemv_70b_sampled(name, K, N):
    """Single-token GEMV on the 70B MLP shapes (K = 28672 loops over chunks:
    8 waves of 64 lanes cover 512 of its 896 chunks per pass); the oracle
    checks sampled row octets of the GPU packing and of the output."""
    awq = G.lib()
    g = 128
    layer = 0 if K == 8192 else 1
    W = workloads.weight(N, K, cfg=4, layer=layer)
    X = workloads.activations(1, K, cfg=4, layer=layer)
    w = G.dev_f16(W)
    qw, sc, qz = awq.awq_pack(w, g, True)
    del w
    y = G.host_f16(awq.awq_gemv(G.dev_f16(X), qw, sc, qz, N, K, g, True))
    rng = np.random.default_rng(5)
    octets = np.sort(rng.choice(N // 8, size=16, replace=False))
    rows = (octets[:, None] * 8 + np.arange(8)[None, :]).reshape(-1)
    oq, os_, oz = O.pack(W[rows], g, True)
    assert np.array_equal(G.host_u32(qw)[rows], oq)
    assert np.array_equal(G.host_f16_bits(sc)[octets], os_)
    assert np.array_equal(G.host_u32(qz)[octets], oz)
    y_ref, d = O.matmul_ref(X, O.dequant_packed(oq, os_, oz, len(rows), K, g, True))
    G.assert_within_tolerance(y[:, rows], y_ref, d, f"gemv {name}")


def test_gemv_adversarial_weights():
    W = workloads.adversarial_weight(64, 1024, 32, seed=5)
    # keep the outputs inside fp16 range: the adversarial groups hold |w| up to 6e4
    X = (workloads.activations(1, 1024, cfg=9, layer=0).astype(np.float32) / 64).astype(np.float16)
    check_layer(64, 1024, 32, True, W, X)
    check_layer(64, 1024, 32, False, W, X)


@pytest.mark.parametrize("zp", [True, False])
def test_gemv_one_hot_reproduces_decoded_weights(zp):
    N, K, g = 64, 512, 32
    W = workloads.adversarial_weight(N, K, g, seed=7)
    packed = O.pack(W, g, zp)
    wdq = O.dequant_packed(*packed, N, K, g, zp).astype(np.float16)
    for k in (0, 1, 7, 31, 32, 255, 256, 511):
        X = np.zeros((1, K), np.float16)
        X[0, k] = 1
        y = run_gemv(X, packed, N, K, g, zp)
        assert np.array_equal(y[0].astype(np.float64), wdq[:, k].astype(np.float64)), k


def test_gemv_zero_input_gives_exact_zero():
    N, K, g = 64, 512, 128
    packed = O.pack(workloads.weight(N, K, cfg=9, layer=1), g, True)
    y = run_gemv(np.zeros((1, K), np.float16), packed, N, K, g, True)
    assert np.all(y == 0)


def test_gemv_deterministic_and_stream():
    N, K, g = 4096, 4096, 128
    W = workloads.weight(N, K, cfg=2, layer=0)
    X = workloads.activations(1, K, cfg=2, layer=0)
    packed = O.pack(W, g, True)
    a = run_gemv(X, packed, N, K, g, True)
    b = run_gemv(X, packed, N, K, g, True, stream=torch.cuda.Stream())
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
