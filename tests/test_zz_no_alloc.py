"""awq_gemm_noalloc through the C ABI: the split-K workspace in the library's
fixed device scratch gives the same bits as awq_gemm with a caller workspace,
and the oracle's tolerance, on two calls in a row (the second with a smaller
input, reusing the scratch the first one left behind); shapes that need no
workspace pass through; shapes past the scratch are refused before any
launch."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest

import workloads
from oracle import awq_oracle as O
from tests import _gpu as G

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _p(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def noalloc(lib, x, qw, sc, qz, y, M, N, K, g, zp):
    return lib.awq_gemm_noalloc(_p(x), _p(qw), _p(sc), _p(qz) if zp else None, _p(y), M, N, K, g, int(zp),
                                ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


@pytest.mark.parametrize("zp", [True, False])
def test_noalloc_matches_gemm_twice_then_smaller(zp):
    awq = G.lib()
    lib = awq.load_library()
    g = 128
    # first call: 64 tokens on 11008 -> 4096 (matrix-core tiles, K split in
    # 8 slices); second: 16 tokens on 4096 x 4096 (skinny kernel, K split
    # across workgroups), a smaller input on the scratch the first one used;
    # then a ragged split-K shape and a shape with no workspace at all
    for M, N, K, gs in [(64, 4096, 11008, g), (16, 4096, 4096, g), (12, 264, 2080, 32), (4, 4096, 4096, g)]:
        need = awq.awq_gemm_workspace_bytes(M, N, K, gs)
        assert need <= lib.awq_gemm_noalloc_max_workspace_bytes()
        assert (need > 0) == (M > 8)
        W = workloads.weight(N, K, cfg=10, layer=M)
        X = workloads.activations(M, K, cfg=10, layer=M)
        packed = O.pack(W, gs, zp)
        qw, sc, qz = G.upload_packed(*packed)
        x = G.dev_f16(X)
        y = torch.empty((M, N), dtype=torch.float16, device="cuda")
        assert noalloc(lib, x, qw, sc, qz, y, M, N, K, gs, zp) == awq.AWQ_OK
        ref = awq.awq_gemm(x, qw, sc, qz, N, K, gs, zp,
                           workspace=torch.zeros(max(need, 1), dtype=torch.uint8, device="cuda"))
        torch.cuda.synchronize()
        what = f"M={M} N={N} K={K} g={gs} zp={zp}"
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), what
        y_ref, d = O.matmul_ref(X, O.dequant_packed(*packed, N, K, gs, zp))
        G.assert_within_tolerance(G.host_f16(y), y_ref, d, "noalloc " + what)


def test_noalloc_refuses_shapes_past_the_scratch():
    """1536 tokens on a 28672 -> 8192 layer split K into fp32 partials of
    192.5 MiB: refused with AWQ_ERR_SCRATCH, nothing launched (the tiny
    buffers passed are never touched)."""
    awq = G.lib()
    lib = awq.load_library()
    M, N, K, g = 1536, 8192, 28672, 128
    assert awq.awq_gemm_workspace_bytes(M, N, K, g) > lib.awq_gemm_noalloc_max_workspace_bytes()
    t = torch.zeros(64, dtype=torch.float16, device="cuda")
    u = torch.zeros(64, dtype=torch.int32, device="cuda")
    st = noalloc(lib, t, u, t, u, t, M, N, K, g, True)
    assert st == awq.AWQ_ERR_SCRATCH
    assert "scratch" in awq.awq_strerror(st)
    torch.cuda.synchronize()
    assert np.all(t.cpu().numpy() == 0)
