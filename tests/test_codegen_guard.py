"""Code-generation guard for the kernels that stage tiles with buffer-to-LDS
loads (gemm_large_kernel, the fused loss kernels): no register-spill store may
be issued between such a load and the workgroup barrier after which the tile
is read.

Why: the compiler waits for a buffer-to-LDS load with a counted
`s_waitcnt vmcnt(N)`, N being the number of vector-memory operations issued
after it, which assumes they complete in issue order.  A spill store issued
after the load is counted among them, but it can be acknowledged before the
load has landed, so the count can drop to N while the load is still in
flight and the waves read LDS rows it has not written yet.  A build of the
GEMM whose register allocation placed a spill store right after the last
buffer-to-LDS load of its first K step gave tile rows 56-63 (that load's 8
rows) that changed from call to call; with the store placed before the loads
(or no spill) the output is bit-reproducible.  The check reads the device
assembly of a fresh compile with the library's own flags (CPU only)."""
from __future__ import annotations

import os
import re
import shutil
import subprocess

import pytest

from bit_weight_only_awq_amd import build as B

SOURCES = ["awq_gemm.hip", "awq_scale.hip"]


def lds_dma_spill_hazards(asm: str):
    """(function, line of the buffer-to-LDS load, line of the spill store) for
    every spill store that follows a buffer-to-LDS load with no workgroup
    barrier (or end of program) in between."""
    bad, fn, pending = [], None, None
    for ln, line in enumerate(asm.splitlines(), 1):
        m = re.match(r"^(_Z\S+):", line)
        if m:
            fn, pending = m.group(1), None
            continue
        s = line.split(";")[0].strip()
        if not s:
            continue
        if re.match(r"buffer_load_\w+ .* lds$", s) or re.match(r"(global|buffer)_load_lds_\w+", s):
            pending = ln
        elif s.startswith("s_barrier") or s.startswith("s_endpgm"):
            pending = None
        elif s.startswith("scratch_store") and pending is not None:
            bad.append((fn, pending, ln))
    return bad


def test_guard_flags_a_store_after_an_lds_load():
    asm = "\n".join([
        "_Zkernel:",
        "\tbuffer_load_dwordx4 v2, s[16:19], s6 offen lds",
        "\tscratch_store_dword off, v4, off offset:4 ; 4-byte Folded Spill",
        "\ts_waitcnt vmcnt(13)",
        "\ts_barrier",
        "\tscratch_store_dword off, v5, off ; after the barrier: harmless",
        "\ts_endpgm",
    ])
    assert lds_dma_spill_hazards(asm) == [("_Zkernel", 2, 3)]


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="needs hipcc")
@pytest.mark.parametrize("src", SOURCES)
def test_no_spill_store_between_lds_load_and_barrier(src, tmp_path):
    flags = [f for f in B.COMMON_FLAGS if f != "-fPIC"]
    out = tmp_path / (src + ".s")
    cmd = [B.hipcc(), *flags, "--cuda-device-only", "-S", os.path.join(B.CSRC, src), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    asm = out.read_text()
    assert " lds" in asm, "expected buffer-to-LDS loads in " + src
    bad = lds_dma_spill_hazards(asm)
    assert not bad, bad[:5]
