"""The kernels inside captured HIP graphs: every replay of a captured
awq_gemv / awq_gemm (single token, few tokens, skinny with K split across
workgroups, large with K split and a reduction launch, large over several
waves of tiles with the half-width tail launch) gives the eager result bit
for bit, with eager calls of other shapes on the same split-K workspace and
synchronizations between the replays."""
from __future__ import annotations

import numpy as np
import pytest

import workloads
from oracle import awq_oracle as O
from tests import _gpu as G

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.mark.parametrize("M,N,K,fn", [(1, 4096, 4096, "gemv"), (4, 4096, 4096, "gemv"), (8, 11008, 4096, "gemm"),
                                      (16, 4096, 4096, "gemm"), (64, 1032, 2048, "gemm"), (300, 1024, 2048, "gemm"),
                                      (2048, 28672, 1024, "gemm")])
def test_graph_replays_match_eager(M, N, K, fn):
    awq = G.lib()
    g = 128
    W = workloads.weight(N, K, cfg=9, layer=M)
    X = workloads.activations(M, K, cfg=9, layer=M)
    qw, sc, qz = G.upload_packed(*O.pack(W, g, True))
    x = G.dev_f16(X)
    f = awq.awq_gemv if fn == "gemv" else awq.awq_gemm
    eager = f(x, qw, sc, qz, N, K, g, True)
    torch.cuda.synchronize()
    y = torch.empty_like(eager)
    # warm on a side stream, as graph capture requires, then capture
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        f(x, qw, sc, qz, N, K, g, True, y=y)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    # captured on the warm-up stream, whose split-K workspace now exists
    with torch.cuda.graph(graph, stream=s):
        f(x, qw, sc, qz, N, K, g, True, y=y)
    # other eager work between replays, sharing the split-K workspace
    W2 = workloads.weight(2048, 4096, cfg=9, layer=99)
    q2 = G.upload_packed(*O.pack(W2, g, True))
    x2 = G.dev_f16(workloads.activations(8, 4096, cfg=9, layer=99))
    for _ in range(4):
        y.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), eager.view(torch.int16))
        awq.awq_gemm(x2, *q2, 2048, 4096, g, True)
        torch.cuda.synchronize()
    # the oracle on all rows, or on a sample of them for the large shape
    rows = np.arange(M) if M <= 512 else np.sort(np.random.default_rng(M).choice(M, 24, replace=False))
    y_ref, d = O.matmul_ref(X[rows], O.dequant_packed(*O.pack(W, g, True), N, K, g, True))
    G.assert_within_tolerance(G.host_f16(y)[rows], y_ref, d, f"graph {fn} M={M}")
