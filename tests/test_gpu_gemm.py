"""awq_gemm (any M) on the GPU against the oracle: per-element tolerance
1e-3 * sum_k |x_k w'_k| on the skinny (M <= 64) and the matrix-core (M > 64)
kernels, ragged tiles, one-hot bit-exactness, the batched-decode and prefill
shapes at full size (prefill on sampled outputs), determinism."""
from __future__ import annotations

import numpy as np
import pytest

import workloads
from oracle import awq_oracle as O
from tests import _gpu as G

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def run_gemm(X16, packed, N, K, g, zp, stream=None):
    awq = G.lib()
    dqw, dsc, dqz = G.upload_packed(*packed)
    x = G.dev_f16(X16)
    if stream is None:
        y = awq.awq_gemm(x, dqw, dsc, dqz, N, K, g, zp)
    else:
        with torch.cuda.stream(stream):
            y = awq.awq_gemm(x, dqw, dsc, dqz, N, K, g, zp)
        stream.synchronize()
    torch.cuda.synchronize()
    return G.host_f16(y)


def check(M, N, K, g, zp, W=None, X=None, what=""):
    if W is None:
        W = workloads.weight(N, K, cfg=3, layer=N + K)
    if X is None:
        X = workloads.activations(M, K, cfg=3, layer=N + K)
    packed = O.pack(W, g, zp)
    y = run_gemm(X, packed, N, K, g, zp)
    y_ref, d = O.matmul_ref(X, O.dequant_packed(*packed, N, K, g, zp))
    return G.assert_within_tolerance(y, y_ref, d, what or f"gemm M={M} N={N} K={K} g={g} zp={zp}")


@pytest.mark.parametrize("M", [1, 2, 3, 4, 8, 15, 16, 17, 31, 33, 48, 64])
def test_gemm_skinny_m(M):
    check(M, 512, 512, 128, True)


@pytest.mark.parametrize("M", [65, 128, 256, 300, 512])
def test_gemm_large_m(M):
    check(M, 512, 1024, 128, True)


@pytest.mark.parametrize("zp", [True, False])
@pytest.mark.parametrize("g", [32, 64, 128, 256])
@pytest.mark.parametrize("M", [8, 96])
def test_gemm_group_sizes_and_symmetry(M, g, zp):
    W = workloads.weight(512, 2048, cfg=5, layer=g, row_offset=True)
    check(M, 512, 2048, g, zp, W=W)


@pytest.mark.parametrize("M,N,K,g", [(1, 8, 32, 32), (5, 8, 96, 32), (70, 8, 96, 32), (3, 24, 160, 32),
                                     (200, 264, 2080, 32), (64, 40, 4128, 32), (257, 520, 544, 32),
                                     (33, 4104, 256, 256)])
def test_gemm_ragged_tiles(M, N, K, g):
    check(M, N, K, g, True)
    check(M, N, K, g, False)


@pytest.mark.parametrize("M,N,K,g", [(9, 264, 2080, 32), (40, 8, 4096, 128), (64, 4104, 11008, 128),
                                     (12, 40, 1664, 64), (17, 136, 8192, 256)])
def test_gemm_split_k(M, N, K, g):
    """Shapes whose K is split across workgroups (partials in the workspace,
    reduced by the last workgroup of each tile), with ragged row tiles and
    a short last slice."""
    assert G.lib().awq_gemm_workspace_bytes(M, N, K, g) > 0
    check(M, N, K, g, True)
    check(M, N, K, g, False)


def test_gemm_split_k_workspace_reuse():
    """One workspace serves consecutive calls of different shapes: every call
    leaves the per-tile counters at zero, and the result is bit-identical
    whichever workgroup of a tile finishes last."""
    awq = G.lib()
    g = 128
    shapes = [(16, 4096, 4096), (64, 4104, 11008), (4, 11008, 4096), (300, 1024, 8192), (64, 1024, 8192),
              (3, 4096, 4096), (9, 264, 4096)]
    need = max(awq.awq_gemm_workspace_bytes(M, N, K, g) for M, N, K in shapes)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for M, N, K in shapes:
        W = workloads.weight(N, K, cfg=3, layer=M)
        X = workloads.activations(M, K, cfg=3, layer=M)
        qw, sc, qz = G.upload_packed(*O.pack(W, g, True))
        x = G.dev_f16(X)
        ys = [awq.awq_gemm(x, qw, sc, qz, N, K, g, True, workspace=ws) for _ in range(4)]
        torch.cuda.synchronize()
        # a counter left non-zero would make the next call skip (or repeat) the reduction of its tile
        for y in ys[1:]:
            assert torch.equal(y.view(torch.int16), ys[0].view(torch.int16))
    y_ref, d = O.matmul_ref(X, O.dequant_packed(*O.pack(W, g, True), N, K, g, True))
    G.assert_within_tolerance(G.host_f16(ys[-1]), y_ref, d, "reused workspace")


def test_gemm_split_k_back_to_back_new_data():
    """Split-K calls of one shape in a row on one workspace, each with new
    activations (the k_proj / v_proj case of batched decode): a last
    workgroup that read a stale partial or a stale counter would give the
    previous call's bytes.  Each output must equal the same call on a freshly
    zeroed workspace and meet the oracle's tolerance."""
    awq = G.lib()
    g = 128
    for M, N, K in [(16, 4096, 4096), (56, 1032, 8192), (9, 264, 4096)]:
        need = awq.awq_gemm_workspace_bytes(M, N, K, g)
        assert need > 0
        ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
        W = workloads.weight(N, K, cfg=3, layer=7 * M)
        packed = O.pack(W, g, True)
        qw, sc, qz = G.upload_packed(*packed)
        wdq = O.dequant_packed(*packed, N, K, g, True)
        for call in range(4):
            X = workloads.activations(M, K, cfg=3, layer=100 * M + call)
            x = G.dev_f16(X)
            y = awq.awq_gemm(x, qw, sc, qz, N, K, g, True, workspace=ws)
            fresh = awq.awq_gemm(x, qw, sc, qz, N, K, g, True,
                                 workspace=torch.zeros(need, dtype=torch.uint8, device="cuda"))
            torch.cuda.synchronize()
            assert torch.equal(y.view(torch.int16), fresh.view(torch.int16)), f"M={M} N={N} K={K} call {call}"
            y_ref, d = O.matmul_ref(X, wdq)
            G.assert_within_tolerance(G.host_f16(y), y_ref, d, f"back-to-back M={M} N={N} K={K} call {call}")


@pytest.mark.parametrize("M", [4, 200])
@pytest.mark.parametrize("zp", [True, False])
def test_gemm_one_hot_reproduces_decoded_weights(M, zp):
    N, K, g = 264, 512, 32
    W = workloads.adversarial_weight(N, K, g, seed=11)
    packed = O.pack(W, g, zp)
    wdq = O.dequant_packed(*packed, N, K, g, zp).astype(np.float16)
    ks = np.random.default_rng(M).integers(0, K, size=M)
    X = np.zeros((M, K), np.float16)
    X[np.arange(M), ks] = 1
    y = run_gemm(X, packed, N, K, g, zp)
    assert np.array_equal(y.astype(np.float64), wdq[:, ks].T.astype(np.float64))


@pytest.mark.parametrize("M", [4, 16, 64])
@pytest.mark.parametrize("name,K,N", [workloads.LLAMA7B_BLOCK[0], workloads.LLAMA7B_BLOCK[4],
                                      workloads.LLAMA7B_BLOCK[6]])
def test_gemm_batched_decode_full_size(M, name, K, N):
    layer = [n for n, _, _ in workloads.LLAMA7B_BLOCK].index(name)
    W = workloads.weight(N, K, cfg=3, layer=layer)
    X = workloads.activations(M, K, cfg=3, layer=layer)
    check(M, N, K, 128, True, W, X, f"gemm {name} M={M}")


# Launch paths of the matrix-core kernel, one shape each (all outputs
# checked; N ragged by 8 rows): 256- or 128-row tiles as the launch plan
# picks them, with the last wave of tiles run by the second, half-width
# launch or not, with K split or not, with a ragged last K step or not.
@pytest.mark.parametrize("M,N,K,g,split,what", [
    (261, 44280, 128, 128, False, "256-row tiles, half-width tail"),
    (261, 44280, 96, 32, False, "256-row tiles, half-width tail, ragged K"),
    (135, 33528, 96, 32, False, "256-row tiles, one wave, ragged K"),
    (513, 44280, 128, 128, False, "128-row tiles, half-width tail"),
    (513, 44280, 96, 32, False, "128-row tiles, half-width tail, ragged K"),
    (65, 512, 544, 32, True, "128-row tiles, K split, ragged K"),
])
def test_gemm_large_launch_paths(M, N, K, g, split, what):
    assert (G.lib().awq_gemm_workspace_bytes(M, N, K, g) > 0) == split, what
    check(M, N, K, g, True, what=f"{what}: M={M} N={N} K={K} g={g}")


@pytest.mark.parametrize("M,N,K,g,split", [(48, 8200, 544, 32, True), (64, 8192, 1024, 128, True),
                                           (33, 16384, 256, 64, False), (56, 1032, 8224, 32, True),
                                           (64, 4096, 11008, 128, True)])
def test_gemm_mid_tokens_wide_layers(M, N, K, g, split):
    """33-64 tokens on layers with N >= 8192, and 49-64 tokens on layers with
    K >= 8192, run on the matrix-core kernel's 64-row tiles: 64 x 128 with K
    split, or 64 x 256 without where the tiles alone fill the chip (the third
    case); ragged last tile and K step in the first and fourth cases; every
    output is checked."""
    need = G.lib().awq_gemm_workspace_bytes(M, N, K, g)
    # each case pins whether K is split; a split needs whole fp32 [M][N]
    # partial slices past the 512 KiB of tile counters
    if split:
        assert need > 512 * 1024 and (need - 512 * 1024) % (M * N * 4) == 0
    else:
        assert need == 0
    check(M, N, K, g, True)
    check(M, N, K, g, False)


@pytest.mark.parametrize("M", [96, 256, 512, 1000, 2048])
@pytest.mark.parametrize("name,K,N", [workloads.LLAMA7B_BLOCK[0], workloads.LLAMA7B_BLOCK[4],
                                      workloads.LLAMA7B_BLOCK[6]])
def test_gemm_medium_m_full_size(M, name, K, N):
    """Token counts between the skinny and the full-GPU regimes on the 7B
    shapes: the matrix-core kernel on 128- or 256-row tiles, splitting K over
    workgroups (fp32 partials added by a second kernel) while the tiles are
    too few, with a ragged last row tile at M = 1000; the oracle checks a
    sample of rows."""
    awq = G.lib()
    g = 128
    layer = [n for n, _, _ in workloads.LLAMA7B_BLOCK].index(name)
    W = workloads.weight(N, K, cfg=3, layer=layer)
    X = workloads.activations(M, K, cfg=3, layer=layer)
    packed = O.pack(W, g, True)
    y = run_gemm(X, packed, N, K, g, True)
    rows = np.sort(np.random.default_rng(M).choice(M, 16, replace=False))
    y_ref, d = O.matmul_ref(X[rows], O.dequant_packed(*packed, N, K, g, True))
    G.assert_within_tolerance(y[rows], y_ref, d, f"gemm {name} M={M}")
    if M <= 256:
        assert awq.awq_gemm_workspace_bytes(M, N, K, g) > 0, "expected a K split at this size"


@pytest.mark.parametrize("name,K,N", workloads.LLAMA70B_MLP)
def test_gemm_prefill_70b_sampled(name, K, N):
    """Full-size prefill GEMM (M=2048) launched as in the benchmark; the oracle
    checks a random sample of output rows and columns."""
    awq = G.lib()
    M, g = 2048, 128
    layer = 0 if K == 8192 else 1
    W = workloads.weight(N, K, cfg=4, layer=layer)
    X = workloads.activations(M, K, cfg=4, layer=layer)
    w = G.dev_f16(W)
    qw, sc, qz = awq.awq_pack(w, g, True)
    del w
    y = G.host_f16(awq.awq_gemm(G.dev_f16(X), qw, sc, qz, N, K, g, True))
    rng = np.random.default_rng(4)
    octets = rng.choice(N // 8, size=8, replace=False)
    cols = (octets[:, None] * 8 + np.arange(8)[None, :]).reshape(-1)
    rows = np.sort(rng.choice(M, size=64, replace=False))
    # the GPU-packed sample must equal the oracle's packing of the same rows
    oq, os_, oz = O.pack(W[cols], g, True)
    assert np.array_equal(G.host_u32(qw)[cols], oq)
    assert np.array_equal(G.host_f16_bits(sc)[octets], os_)
    assert np.array_equal(G.host_u32(qz)[octets], oz)
    y_ref, d = O.matmul_ref(X[rows], O.dequant_packed(oq, os_, oz, len(cols), K, g, True))
    G.assert_within_tolerance(y[np.ix_(rows, cols)], y_ref, d, f"prefill {name}")


def test_gemm_deterministic_and_stream():
    M, N, K, g = 300, 1024, 2048, 128
    W = workloads.weight(N, K, cfg=3, layer=99)
    X = workloads.activations(M, K, cfg=3, layer=99)
    packed = O.pack(W, g, True)
    a = run_gemm(X, packed, N, K, g, True)
    b = run_gemm(X, packed, N, K, g, True, stream=torch.cuda.Stream())
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    a = run_gemm(X[:16], packed, N, K, g, True)
    b = run_gemm(X[:16], packed, N, K, g, True, stream=torch.cuda.Stream())
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


def test_gemm_repeat_bit_identical_many_tiles():
    """Four waves of 256 x 256 tiles over the compute units (2048 x 28672 x
    1024: 768 tiles and a half-width tail launch), so that most workgroups
    start on a compute unit another one has just left: four calls give the
    same bits in every output, and the oracle checks whole rows at the end of
    a tile's last X load (rows 56-63 of the tile) and elsewhere.  (A build
    whose register spill landed between that load and its barrier varied in
    exactly those rows.)"""
    awq = G.lib()
    M, N, K, g = 2048, 28672, 1024, 128
    W = workloads.weight(N, K, cfg=4, layer=7)
    X = workloads.activations(M, K, cfg=4, layer=7)
    w = G.dev_f16(W)
    qw, sc, qz = awq.awq_pack(w, g, True)
    del w
    x = G.dev_f16(X)
    y0 = awq.awq_gemm(x, qw, sc, qz, N, K, g, True)
    for _ in range(3):
        y = awq.awq_gemm(x, qw, sc, qz, N, K, g, True)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y0.view(torch.int16))
    rows = np.array([56, 63, 256 + 57, 1024 + 60, 2047 - 192, 1500])
    yh = G.host_f16(y0)[rows]
    # the oracle on all columns of these rows, from its own packing of W
    packed = O.pack(W, g, True)
    y_ref, d = O.matmul_ref(X[rows], O.dequant_packed(*packed, N, K, g, True))
    G.assert_within_tolerance(yh, y_ref, d, "repeat many tiles")
