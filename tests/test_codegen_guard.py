"""Code-generation guard: in every kernel of the library, no register-spill
store may be issued between a buffer-to-LDS load and the workgroup barrier
after which its tile is read, nor while any vector-memory load may still be
in flight (after it, before an `s_waitcnt vmcnt(0)`).

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

SOURCES = ["awq_gemm.hip", "awq_scale.hip", "awq_gemv.hip", "awq_gemv_small.hip", "awq_pack.hip"]


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


def spill_stores_with_loads_in_flight(asm: str):
    """(function, line of the load, line of the spill store) for every spill
    store issued while a vector-memory load (or returning atomic) may still be
    in flight, i.e. after it with no `s_waitcnt vmcnt(0)` in between: the same
    counted-wait hazard for loads into registers."""
    bad, fn, pending = [], None, None
    for ln, line in enumerate(asm.splitlines(), 1):
        m = re.match(r"^(_Z\S+):", line)
        if m:
            fn, pending = m.group(1), None
            continue
        s = line.split(";")[0].strip()
        if not s:
            continue
        if re.match(r"(buffer|global|flat)_load", s) or re.match(r"(buffer|global)_atomic\S* .* sc0", s):
            pending = ln
        elif re.match(r"s_waitcnt .*vmcnt\(0\)", s) or s.startswith("s_endpgm"):
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
    # (no vmcnt(0) anywhere: both stores may overtake the load)
    assert spill_stores_with_loads_in_flight(asm) == [("_Zkernel", 2, 3), ("_Zkernel", 2, 6)]
    asm2 = "\n".join(["_Zk2:", "\tglobal_load_dwordx4 v[0:3], v[4:5], off", "\ts_waitcnt vmcnt(0)",
                      "\tscratch_store_dword off, v4, off", "\ts_endpgm"])
    assert spill_stores_with_loads_in_flight(asm2) == []


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="needs hipcc")
@pytest.mark.parametrize("src", SOURCES)
def test_no_spill_store_while_loads_are_in_flight(src, tmp_path):
    flags = [f for f in B.COMMON_FLAGS if f != "-fPIC"]
    out = tmp_path / (src + ".s")
    cmd = [B.hipcc(), *flags, "--cuda-device-only", "-S", os.path.join(B.CSRC, src), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    asm = out.read_text()
    bad = lds_dma_spill_hazards(asm)
    assert not bad, bad[:5]
    bad = spill_stores_with_loads_in_flight(asm)
    assert not bad, bad[:5]
