"""awq_pack and awq_dequant on the GPU against the oracle: packed words,
scales and zero points bit-identical; decoded weights equal fp16((q-z)*s)."""
from __future__ import annotations

import numpy as np
import pytest

import workloads
from oracle import awq_oracle as O
from tests import _gpu as G

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def gpu_pack(W16, g, zp, stream=None):
    awq = G.lib()
    w = G.dev_f16(W16)
    if stream is None:
        qw, sc, qz = awq.awq_pack(w, g, zp)
    else:
        with torch.cuda.stream(stream):
            qw, sc, qz = awq.awq_pack(w, g, zp)
        stream.synchronize()
    torch.cuda.synchronize()
    return G.host_u32(qw), G.host_f16_bits(sc), (G.host_u32(qz) if zp else None)


def assert_pack_equal(W16, g, zp, rows=None):
    qw, sc, qz = gpu_pack(W16, g, zp)
    if rows is not None:
        # quantization is independent per row: the oracle packs only the sampled rows
        rows = np.asarray(rows)
        octets = rows[::8] // 8  # sampled rows come in whole octets
        oq, os_, oz = O.pack(W16[rows], g, zp)
        assert np.array_equal(qw[rows], oq)
        assert np.array_equal(sc[octets], os_)
        if zp:
            assert np.array_equal(qz[octets], oz)
        return
    oq, os_, oz = O.pack(W16, g, zp)
    assert np.array_equal(qw, oq), f"qweight differs at {np.argwhere(qw != oq)[:5].tolist()}"
    assert np.array_equal(sc, os_), f"scales differ at {np.argwhere(sc != os_)[:5].tolist()}"
    if zp:
        assert np.array_equal(qz, oz), f"qzeros differ at {np.argwhere(qz != oz)[:5].tolist()}"


def test_pack_tiny_layer_bit_exact():
    W = workloads.weight(512, 512, cfg=0, layer=0)
    assert_pack_equal(W, 128, True)


@pytest.mark.parametrize("zp", [True, False])
@pytest.mark.parametrize("g", [32, 64, 128, 256])
def test_pack_adversarial_groups_bit_exact(g, zp):
    assert_pack_equal(workloads.adversarial_weight(64, 1024, g, seed=g), g, zp)


@pytest.mark.parametrize("zp", [True, False])
@pytest.mark.parametrize("g", [32, 64, 128, 256])
def test_pack_row_offset_weights_bit_exact(g, zp):
    assert_pack_equal(workloads.weight(128, 2048, cfg=5, layer=g, row_offset=True), g, zp)


@pytest.mark.parametrize("N,K,g", [(8, 32, 32), (8, 96, 32), (16, 11008, 128), (24, 11008, 64), (8, 2304, 256),
                                   (40, 4128, 32)])
def test_pack_ragged_and_minimal_shapes(N, K, g):
    W = workloads.weight(N, K, cfg=7, layer=K)
    assert_pack_equal(W, g, True)
    assert_pack_equal(W, g, False)


@pytest.mark.parametrize("name,K,N", workloads.LLAMA7B_BLOCK[3:])
def test_pack_llama7b_shapes_bit_exact(name, K, N):
    assert_pack_equal(workloads.weight(N, K, cfg=2, layer=K + N), 128, True)


@pytest.mark.parametrize("name,K,N", workloads.LLAMA70B_MLP)
def test_pack_70b_shapes_sampled_rows(name, K, N):
    W = workloads.weight(N, K, cfg=4, layer=0 if K == 8192 else 1)
    rng = np.random.default_rng(11)
    octets = rng.choice(N // 8, size=12, replace=False)
    rows = (octets[:, None] * 8 + np.arange(8)[None, :]).reshape(-1)
    assert_pack_equal(W, 128, True, rows=rows)


def test_pack_deterministic_and_stream():
    W = workloads.weight(256, 4096, cfg=8, layer=0)
    a = gpu_pack(W, 128, True)
    s = torch.cuda.Stream()
    b = gpu_pack(W, 128, True, stream=s)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("zp", [True, False])
@pytest.mark.parametrize("g", [32, 128])
def test_dequant_bit_exact(g, zp):
    awq = G.lib()
    W = workloads.adversarial_weight(64, 1024, g, seed=3)
    qw, sc, qz = O.pack(W, g, zp)
    dqw, dsc, dqz = G.upload_packed(qw, sc, qz)
    out = awq.awq_dequant(dqw, dsc, dqz, 64, 1024, g, zp)
    torch.cuda.synchronize()
    want = O.dequant_packed(qw, sc, qz, 64, 1024, g, zp).astype(np.float16)
    got = G.host_f16(out)
    assert np.array_equal(got.view(np.uint16) & 0x7FFF == 0, want.view(np.uint16) & 0x7FFF == 0)
    assert np.array_equal(got.astype(np.float64), want.astype(np.float64))
