"""The C ABI library loads, exports every entry point declared in
include/awq.h, and rejects invalid arguments on the host, before any launch.

These tests run without a GPU: every call below fails validation, so no
pointer is ever dereferenced and nothing reaches the HIP runtime."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "awq.h")

awq = pytest.importorskip("bit_weight_only_awq_amd")


def declared_functions():
    src = open(HEADER, encoding="utf-8").read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(awq_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(awq.LIB_PATH):
        pytest.fail(f"{awq.LIB_PATH} not built; run python -m bit_weight_only_awq_amd.build")
    return awq.load_library()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert set(names) == set(awq.EXPORTED), names
    for name in names:
        assert hasattr(lib, name), name


def test_strerror_and_workspace(lib):
    for code in range(-7, 1):
        assert awq.awq_strerror(code) and awq.awq_strerror(code) != "unknown awq status"
    assert awq.awq_strerror(42) == "unknown awq status"
    assert awq.awq_gemm_workspace_bytes(2048, 28672, 8192, 128) == 0


def test_gemm_launch_plans_through_workspace_sizes(lib):
    """The GEMM launch plans, seen through the workspace they need: on a
    4096 x 4096 layer, up to 8 tokens run as 16-row tiles without a K split
    (no workspace); 16 and 64 tokens split K across workgroups (512 KiB of
    counters plus fp32 partial tiles), 33-64 tokens on layers with N >= 8192
    and 49-64 tokens on layers with K >= 8192 run on the matrix-core kernel's
    64-row tiles; the matrix-core kernel splits K only
    while its tiles (256 or 128 rows x 256) are too few for the compute units:
    on 4096 x 4096 up to M = 1024, not at M = 2048 (256 tiles of 128 rows) nor
    on the 70B MLP shapes at M = 2048 (896 and 256 tiles of 256 rows)."""
    ws = awq.awq_gemm_workspace_bytes
    counters = 512 * 1024
    for M in (1, 2, 4, 5, 8):
        assert ws(M, 4096, 4096, 128) == 0, M
    for M in (16, 64):
        need = ws(M, 4096, 4096, 128)
        assert need > counters and (need - counters) % (16 * 16 * 4) == 0, M
    # 33-64 tokens on wide layers: 64-row matrix-core tiles, K split into whole [splits][M][N] slices
    for M in (33, 64):
        need = ws(M, 11008, 4096, 128)
        assert need > counters and (need - counters) % (M * 11008 * 4) == 0, M
    need = ws(32, 11008, 4096, 128)
    assert (need - counters) % (16 * 16 * 4) == 0  # 32 tokens: still the skinny kernel's partial tiles
    # 49-64 tokens on layers with K >= 8192 (11008 -> 4096) take the 64-row tiles too
    for M in (49, 64):
        need = ws(M, 4096, 11008, 128)
        assert need > counters and (need - counters) % (M * 4096 * 4) == 0, M
    for M in (96, 256, 512, 1024):
        need = ws(M, 4096, 4096, 128)
        assert need > counters and (need - counters) % (M * 4096 * 4) == 0, M  # whole [splits][M][N] fp32 slices
    assert ws(2048, 4096, 4096, 128) == 0
    assert ws(4096, 4096, 4096, 128) == 0
    assert ws(2048, 28672, 8192, 128) == 0
    assert ws(2048, 8192, 28672, 128) == 0


# Fake, 16-byte aligned device addresses: validation must reject every call
# below before anything could touch them.
A = 0x7F0000000000
B = A + 0x100000
C = A + 0x200000
D = A + 0x300000
E = A + 0x400000


@pytest.mark.parametrize(
    "args,expect",
    [
        # (N, K, g, zp, w, qweight, scales, qzeros)
        ((8, 128, 48, 1, A, B, C, D), awq.AWQ_ERR_GROUP),
        ((8, 96, 64, 1, A, B, C, D), awq.AWQ_ERR_GROUP),
        ((12, 128, 32, 1, A, B, C, D), awq.AWQ_ERR_SHAPE),
        ((0, 128, 32, 1, A, B, C, D), awq.AWQ_ERR_SHAPE),
        ((8, 0, 32, 1, A, B, C, D), awq.AWQ_ERR_SHAPE),
        ((8, 128, 32, 1, 0, B, C, D), awq.AWQ_ERR_NULL),
        ((8, 128, 32, 1, A, 0, C, D), awq.AWQ_ERR_NULL),
        ((8, 128, 32, 1, A, B, C, 0), awq.AWQ_ERR_NULL),
        ((8, 128, 32, 1, A + 4, B, C, D), awq.AWQ_ERR_ALIGN),
        ((8, 128, 32, 1, A, B + 8, C, D), awq.AWQ_ERR_ALIGN),
    ],
)
def test_pack_validation(lib, args, expect):
    N, K, g, zp, w, qw, sc, qz = args
    assert lib.awq_pack(w or None, N, K, g, zp, qw or None, sc or None, qz or None, None) == expect


def test_gemv_gemm_validation(lib):
    ok = dict(x=A, qw=B, sc=C, qz=D, y=E)
    gemv = lambda M, N, K, g, zp, **kw: lib.awq_gemv(  # noqa: E731
        kw.get("x", A) or None, kw.get("qw", B) or None, kw.get("sc", C) or None, kw.get("qz", D) or None,
        kw.get("y", E) or None, M, N, K, g, zp, None)
    assert gemv(9, 8, 128, 32, 1) == awq.AWQ_ERR_UNSUPPORTED  # more than 8 tokens: awq_gemm
    assert gemv(0, 8, 128, 32, 1) == awq.AWQ_ERR_SHAPE
    assert gemv(1, 8, 128, 100, 1) == awq.AWQ_ERR_GROUP
    assert gemv(1, 8, 128, 32, 1, y=0) == awq.AWQ_ERR_NULL
    assert gemv(1, 8, 128, 32, 1, x=A + 2) == awq.AWQ_ERR_ALIGN
    assert gemv(1, 8, 128, 32, 1, qz=0) == awq.AWQ_ERR_NULL
    gemm = lambda M, N, K, g, zp, ws=0, wsb=0, **kw: lib.awq_gemm(  # noqa: E731
        kw.get("x", A) or None, kw.get("qw", B) or None, kw.get("sc", C) or None, kw.get("qz", D) or None,
        kw.get("y", E) or None, M, N, K, g, zp, ws or None, wsb, None)
    assert gemm(0, 8, 128, 32, 1) == awq.AWQ_ERR_SHAPE
    assert gemm(4, 10, 128, 32, 1) == awq.AWQ_ERR_SHAPE
    assert gemm(4, 8, 160, 64, 1) == awq.AWQ_ERR_GROUP
    assert gemm(4, 8, 128, 32, 1, sc=0) == awq.AWQ_ERR_NULL
    assert gemm(4, 8, 128, 32, 1, y=E + 6) == awq.AWQ_ERR_ALIGN
    assert gemm(4, 1 << 22, 128, 32, 1) == awq.AWQ_ERR_SHAPE
    assert gemv(1, 8, 1 << 22, 32, 1) == awq.AWQ_ERR_SHAPE
    assert ok  # silence unused


def test_gemm_split_k_workspace_contract(lib):
    """Shapes whose K is split across workgroups need a workspace: a 512 KiB
    counter region plus one fp32 partial tile per workgroup.  Too small, NULL
    or misaligned workspaces are rejected before any launch."""
    M, N, K, g = 16, 4096, 4096, 128
    need = awq.awq_gemm_workspace_bytes(M, N, K, g)
    assert need > 512 * 1024 and (need - 512 * 1024) % (16 * 16 * 4) == 0
    assert awq.awq_gemm_workspace_bytes(M, N, K, 100) == 0  # invalid shapes need nothing
    assert awq.awq_gemm_workspace_bytes(0, N, K, g) == 0
    call = lambda ws, wsb: lib.awq_gemm(A, B, C, D, E, M, N, K, g, 1, ws, wsb, None)  # noqa: E731
    assert call(None, need - 1) == awq.AWQ_ERR_WORKSPACE
    assert call(None, need) == awq.AWQ_ERR_NULL
    assert call(A + 8, need) == awq.AWQ_ERR_ALIGN


def test_dequant_validation(lib):
    assert lib.awq_dequant(B, C, D, None, 8, 128, 32, 1, None) == awq.AWQ_ERR_NULL
    assert lib.awq_dequant(B, C, None, A, 8, 128, 32, 1, None) == awq.AWQ_ERR_NULL
    assert lib.awq_dequant(B, C, D, A, 8, 100, 32, 1, None) == awq.AWQ_ERR_GROUP


def test_binding_rejects_host_tensors():
    torch = pytest.importorskip("torch")
    w = torch.zeros((8, 128), dtype=torch.float16)
    with pytest.raises(ValueError):
        awq.awq_pack(w, 32, True)


def test_scale_search_validation(lib):
    alphas = (ctypes.c_float * 2)(0.0, 0.5)
    cand = lambda M, K, cnt, **kw: lib.awq_scale_candidates(  # noqa: E731
        kw.get("x", A) or None, M, K, kw.get("w", None), kw.get("N", 0), kw.get("duo", 0),
        ctypes.cast(alphas, ctypes.c_void_p) if kw.get("al", 1) else None, cnt,
        kw.get("s", B) or None, kw.get("ws", C) or None, kw.get("wsb", 1 << 30), None)
    assert cand(0, 64, 2) == awq.AWQ_ERR_SHAPE
    assert cand(4, 12, 2) == awq.AWQ_ERR_SHAPE
    assert cand(4, 64, 0) == awq.AWQ_ERR_SHAPE
    assert cand(4, 64, 65) == awq.AWQ_ERR_SHAPE
    assert cand(4, 64, 2, al=0) == awq.AWQ_ERR_NULL
    assert cand(4, 64, 2, s=0) == awq.AWQ_ERR_NULL
    assert cand(4, 64, 2, x=A + 2) == awq.AWQ_ERR_ALIGN
    assert cand(4, 64, 2, wsb=0) == awq.AWQ_ERR_WORKSPACE
    assert cand(4, 64, 2, duo=1, N=8) == awq.AWQ_ERR_NULL  # duo scaling reads w
    assert cand(4, 64, 2, duo=1, N=0, w=D) == awq.AWQ_ERR_SHAPE
    assert cand(4, 64, 2, duo=1, N=8, w=D + 4) == awq.AWQ_ERR_ALIGN
    wsb = awq.load_library().awq_scale_candidates_workspace_bytes
    assert wsb(100, 0, 64) >= 2 * 64 * 4
    assert wsb(100, 300, 64) >= wsb(100, 0, 64) + 5 * 64 * 4  # the weight statistic's partial sums
    srch = lambda cnt, M, N, K, g, **kw: lib.awq_scale_search(  # noqa: E731
        kw.get("x", A) or None, kw.get("w", B) or None, M, N, K, g, 1,
        ctypes.cast(alphas, ctypes.c_void_p) if kw.get("al", 1) else None, cnt, kw.get("duo", 0),
        kw.get("s", C) or None, kw.get("best", D) or None, kw.get("losses", None), kw.get("ws", E) or None,
        kw.get("wsb", 1 << 40), None)
    assert srch(2, 4, 12, 128, 32) == awq.AWQ_ERR_SHAPE
    assert srch(2, 4, 8, 100, 32) == awq.AWQ_ERR_GROUP
    assert srch(0, 4, 8, 128, 32) == awq.AWQ_ERR_SHAPE
    assert srch(65, 4, 8, 128, 32) == awq.AWQ_ERR_SHAPE
    assert srch(2, 0, 8, 128, 32) == awq.AWQ_ERR_SHAPE
    assert srch(2, 4, 8, 128, 32, al=0) == awq.AWQ_ERR_NULL
    assert srch(2, 4, 8, 128, 32, best=0) == awq.AWQ_ERR_NULL
    assert srch(2, 4, 8, 128, 32, best=D + 2) == awq.AWQ_ERR_ALIGN
    assert srch(2, 4, 8, 128, 32, losses=E + 4) == awq.AWQ_ERR_ALIGN
    need = awq.load_library().awq_scale_search_workspace_bytes(2, 4, 8, 128)
    # the candidates' scales, their group parameters and the activations scaled by each
    assert need >= 2 * 128 * 4 + 2 * (128 // 32) * 8 * 4 + 2 * 4 * 128 * 2
    assert srch(2, 4, 8, 128, 32, wsb=need - 1) == awq.AWQ_ERR_WORKSPACE
    loss = lambda cnt, M, N, K, g, **kw: lib.awq_scale_loss(  # noqa: E731
        kw.get("x", A) or None, kw.get("w", B) or None, kw.get("s", C) or None, cnt, M, N, K, g, 1,
        kw.get("ws", D) or None, kw.get("wsb", 1 << 40), kw.get("loss", E) or None, None)
    assert loss(1, 4, 12, 128, 32) == awq.AWQ_ERR_SHAPE
    assert loss(1, 4, 8, 100, 32) == awq.AWQ_ERR_GROUP
    assert loss(0, 4, 8, 128, 32) == awq.AWQ_ERR_SHAPE
    assert loss(1, 0, 8, 128, 32) == awq.AWQ_ERR_SHAPE
    assert loss(1, 4, 8, 128, 32, loss=0) == awq.AWQ_ERR_NULL
    assert loss(1, 4, 8, 128, 32, loss=E + 4) == awq.AWQ_ERR_ALIGN
    assert loss(1, 4, 8, 128, 32, s=C + 8) == awq.AWQ_ERR_ALIGN
    need = awq.load_library().awq_scale_loss_workspace_bytes(3, 4, 8, 128)
    # group parameters (4 bytes per candidate, row and 32-channel group) and
    # the activations scaled by each candidate
    assert need >= 3 * (128 // 32) * 8 * 4 + 3 * 4 * 128 * 2
    assert loss(3, 4, 8, 128, 32, wsb=need - 1) == awq.AWQ_ERR_WORKSPACE
    # the loss product's parameter range: K * N < 2^34 (checked before anything runs)
    assert loss(1, 4, 1 << 17, 1 << 17, 128) == awq.AWQ_ERR_SHAPE
    assert srch(2, 4, 1 << 17, 1 << 17, 128) == awq.AWQ_ERR_SHAPE


def test_clip_and_scale_columns_validation(lib):
    ratios = (ctypes.c_float * 3)(1.0, 0.9, 0.8)
    bad = (ctypes.c_float * 2)(1.0, 1.5)
    rp = lambda arr: ctypes.cast(arr, ctypes.c_void_p)  # noqa: E731
    clip = lambda M, N, K, g, cnt, **kw: lib.awq_clip_search(  # noqa: E731
        kw.get("x", A) or None, kw.get("w", B) or None, M, N, K, g, 1, kw.get("r", rp(ratios)), cnt,
        kw.get("out", C) or None, kw.get("choice", D) or None, kw.get("ws", E) or None, kw.get("wsb", 1 << 40), None)
    assert clip(4, 12, 128, 32, 3) == awq.AWQ_ERR_SHAPE
    assert clip(4, 8, 100, 32, 3) == awq.AWQ_ERR_GROUP
    assert clip(0, 8, 128, 32, 3) == awq.AWQ_ERR_SHAPE
    assert clip(4, 8, 128, 32, 0) == awq.AWQ_ERR_SHAPE
    assert clip(4, 8, 128, 32, 65) == awq.AWQ_ERR_SHAPE
    assert clip(4, 8, 128, 32, 2, r=rp(bad)) == awq.AWQ_ERR_SHAPE
    assert clip(4, 8, 128, 32, 3, out=0) == awq.AWQ_ERR_NULL
    assert clip(4, 8, 128, 32, 3, choice=D + 2) == awq.AWQ_ERR_ALIGN
    assert clip(4, 8, 128, 32, 3, w=B + 8) == awq.AWQ_ERR_ALIGN
    need = awq.load_library().awq_clip_search_workspace_bytes(3, 4, 8, 128, 32)
    # every ratio's group parameters (8 bytes per row and group) and the
    # per-group partial errors of the 4 token quarters of one tile
    assert need >= 3 * (128 // 32) * 8 * 8 + 3 * 4 * (128 // 32) * 8 * 4
    assert clip(4, 8, 128, 32, 3, wsb=need - 1) == awq.AWQ_ERR_WORKSPACE
    assert clip(4, 1 << 16, 1 << 17, 128, 3) == awq.AWQ_ERR_SHAPE  # K * N < 2^33
    cols = lambda rows, K, **kw: lib.awq_scale_columns(  # noqa: E731
        kw.get("src", A) or None, rows, K, kw.get("s", B) or None, 0, kw.get("dst", C) or None, None)
    assert cols(0, 64) == awq.AWQ_ERR_SHAPE
    assert cols(4, 12) == awq.AWQ_ERR_SHAPE
    assert cols(4, 64, s=0) == awq.AWQ_ERR_NULL
    assert cols(4, 64, dst=C + 2) == awq.AWQ_ERR_ALIGN