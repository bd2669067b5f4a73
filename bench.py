#!/usr/bin/env python3
"""Benchmark of the W4A16 AWQ linear layer on one MI355X.

Headline: single-token decode through the seven quantized linears (q, k, v, o
projections 4096->4096, gate/up 4096->11008, down 11008->4096; group size
128, zero points) of BLOCKS distinct Llama-7B-shaped decoder blocks.  One
step = one token through all blocks = 7 * BLOCKS awq_gemv launches, replayed
from a HIP graph.  Every block has its own copy of the packed weights, so a
step streams ~3.3 GB and no launch is served from the 256 MB Infinity Cache.

value  = algorithmic bytes of a step / step time, GB/s (whole job, one GPU)
roofline = the GEMV kernel against 8 TB/s HBM; its average launch time comes
         from HIP events around back-to-back launches on the launch stream.
legs   = awq_pack, fused-projection decode (qkv and gate_up as one awq_gemv
         each), batched-decode awq_gemm (M = 4/16/64; GEMV vs GEMM at M = 1),
         prefill awq_gemm (M = 2048, 70B-shaped MLP), activation-aware scale
         search (L(s) for 20 candidates over 512 calibration tokens), weight
         clipping search (20 ratios, same tokens), group-size / symmetry sweep
         (g = 32 / 128 / 256 with and without zero points, M = 1 and 8),
         single-token GEMV on the 70B MLP shapes (layers large enough that
         the launch floor no longer dominates); for context, torch's dense
         fp16 products on the unquantized weights (decode M = 1/4/16/64 and
         the prefill shapes) with the W4A16 speedup over them, and measured
         HBM ceilings (torch's 1 GiB copy and 1 GiB fp16 sum).
cpu_baseline = the CPU oracle on one block, timed on the host (quantize + pack;
         decode + fp64 product, which is its value; a 70B prefill sample): a
         reported reference, not a target.  The same oracle results check the
         run (self_check): the GPU packing bit for bit, and the last timed
         replay's outputs within 1e-3 * sum |x w'|.

Usage: python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--blocks 32]
                       [--legs all|none|<comma list>] [--no-cpu-baseline] [--no-layer-timing]
       python bench.py --leg-only pack|fused|batched|dense|prefill|scale|clip|sweep|gemv70b|power|ceiling
                       (one leg, for profiling)
       python bench.py --leg-only loop --shape M,N,K [--launches 200]   (awq_gemm on one shape, for profiling)
       python bench.py --copy-calibration | --summarize DB... [--kernel-filter NAME] [--last N]
       python bench.py --kernel-hash SRC...   (hash of kernel sources + compile flags)
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
FP16_MFMA_PEAK_TFLOPS = 2516.6  # MI355X dense fp16 matrix throughput (256 CU x 2.4 GHz x 4096 flop/clk)
METRIC = "W4A16 GEMV achieved GB/s + GEMM TFLOPS (fraction of MI355X roofline)"


def algorithmic_bytes(M, N, K, g, zp):
    """Minimum HBM bytes of one layer call: 4-bit codes, fp16 scales, 4-bit
    zero points, fp16 X in and fp16 Y out."""
    G = K // g
    return K * N // 2 + G * N * 2 + (G * N // 2 if zp else 0) + 2 * M * K + 2 * M * N


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--blocks", type=int, default=32)
    ap.add_argument("--legs", default="all")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (for scaling HBM counters)")
    ap.add_argument("--summarize", nargs="+", metavar="DB",
                    help="print a per-kernel summary of rocprofv3 result databases and exit")
    ap.add_argument("--kernel-filter", default=None, help="with --summarize: only kernels whose name contains this")
    ap.add_argument("--pool", action="store_true", help="with --summarize: one summary over all the databases")
    ap.add_argument("--kernel-hash", nargs="+", metavar="SRC",
                    help="print the hash of these kernel sources and the compile flags (for counter summaries)")
    ap.add_argument("--last", type=int, default=None,
                    help="with --summarize: only the last N matching dispatches (e.g. the timed replays)")
    ap.add_argument("--no-layer-timing", action="store_true",
                    help="skip the per-layer timing graphs after the timed steps (so that a kernel trace ends "
                         "with the timed replays)")
    ap.add_argument("--shape", default="16,4096,4096", help="with --leg-only loop: M,N,K")
    ap.add_argument("--launches", type=int, default=200, help="with --leg-only loop: launches")
    ap.add_argument("--leg-only", default=None, choices=["pack", "fused", "batched", "dense", "prefill", "scale", "clip", "sweep", "gemv70b", "power",
                             "ceiling", "loop"],
                    help="run just this leg (no headline, no CPU baseline) and print its JSON; for profiling")
    return ap.parse_args()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class Timer:
    """HIP events on the current stream."""

    def __init__(self, torch):
        self.torch = torch
        self.a = torch.cuda.Event(enable_timing=True)
        self.b = torch.cuda.Event(enable_timing=True)

    def start(self):
        self.a.record()

    def stop_ms(self):
        self.b.record()
        self.b.synchronize()
        return self.a.elapsed_time(self.b)


def build_decode_block(torch, awq, workloads, blocks, g=128, zp=True):
    """Pack one Llama-7B block on the GPU and replicate the packed buffers."""
    layers = []
    for li, (name, K, N) in enumerate(workloads.LLAMA7B_BLOCK):
        W = workloads.weight(N, K, cfg=2, layer=li)
        X = workloads.activations(1, K, cfg=2, layer=li)
        w = torch.from_numpy(W).cuda()
        qw, sc, qz = awq.awq_pack(w, g, zp)
        layers.append(dict(name=name, K=K, N=N, W=W, X=X, w_dev=w, qw=qw, sc=sc, qz=qz,
                           x=torch.from_numpy(X).cuda()))
    torch.cuda.synchronize()
    reps = []
    for b in range(blocks):
        rep = []
        for L in layers:
            rep.append(dict(qw=L["qw"].clone(), sc=L["sc"].clone(),
                            qz=L["qz"].clone() if L["qz"] is not None else None,
                            y=torch.empty((1, L["N"]), dtype=torch.float16, device="cuda")))
        reps.append(rep)
    torch.cuda.synchronize()
    return layers, reps


def decode_step(awq, layers, reps, g, zp):
    for rep in reps:
        for L, R in zip(layers, rep):
            awq.awq_gemv(L["x"], R["qw"], R["sc"], R["qz"], L["N"], L["K"], g, zp, y=R["y"])


def per_layer_launch_times(torch, awq, layers, reps, g, zp, replays=20):
    """Average device time of one awq_gemv launch per layer shape: a HIP graph
    holds that layer's launches over all blocks back to back (distinct weight
    copies), and HIP events on the launching stream bracket its replays."""
    out = {}
    for li, L in enumerate(layers):
        def fn(li=li, L=L):
            for rep in reps:
                R = rep[li]
                awq.awq_gemv(L["x"], R["qw"], R["sc"], R["qz"], L["N"], L["K"], g, zp, y=R["y"])

        ms, _ = time_graph(torch, fn, replays)
        out[L["name"]] = ms * 1e3 / len(reps)  # us per launch
    return out


def kernel_hash(rel_paths):
    """sha256 over the given kernel source files (repository-relative) and the
    library's compile flags: identifies the kernel a counter summary was
    taken on."""
    import hashlib

    from bit_weight_only_awq_amd import build as B

    h = hashlib.sha256()
    for rel in rel_paths:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    h.update(" ".join(B.COMMON_FLAGS).encode())
    return h.hexdigest()


def profile_record(name):
    """The key: value lines of a committed profile summary, if it was taken on
    the current kernel sources and build flags; else (None, reason)."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None, "no profile summary"
    rec = {}
    with open(path) as f:
        for line in f:
            if line.startswith("#") or ":" not in line or line.startswith("_Z"):
                continue
            k, v = line.split(":", 1)
            rec[k.strip()] = v.strip()
    if kernel_hash(rec["sources"].split()) != rec["sources_sha256"]:
        return None, "kernel source or build flags changed since the profile was taken"
    return rec, None


def hbm_traffic(step_launches):
    """Measured HBM bytes per GEMV launch from the committed counter summary,
    if it was taken on the current kernel source and build flags; else None."""
    rec, why = profile_record("gemv_llama7b_decode_traffic.txt")
    if rec is None:
        return None, why
    return int(rec["hbm_bytes_per_launch"]), rec["note"]


def dispatch_stats():
    """Per-shape rocprofv3 dispatch durations (median, p10, p90) of the timed
    decode replays from the committed kernel-trace summary, if it was taken
    on the current kernel; else None."""
    rec, why = profile_record("gemv_llama7b_decode_kernel_trace.txt")
    if rec is None:
        return {"note": why}
    return dict(json.loads(rec["dispatch_stats"]), source="profiles/gemv_llama7b_decode_kernel_trace.txt "
                "(rocprofv3 --kernel-trace of the timed replays; the tracer adds per-dispatch overhead)")


def leg_pack(torch, awq, layers, g, zp, reps=5):
    tm = Timer(torch)
    total_w = sum(L["N"] * L["K"] for L in layers)
    out_bytes = sum(algorithmic_bytes(0, L["N"], L["K"], g, zp) for L in layers)
    in_bytes = 2 * total_w
    for L in layers:  # warm
        awq.awq_pack(L["w_dev"], g, zp, qweight=L["qw"], scales=L["sc"], qzeros=L["qz"])
    torch.cuda.synchronize()
    tm.start()
    for _ in range(reps):
        for L in layers:
            awq.awq_pack(L["w_dev"], g, zp, qweight=L["qw"], scales=L["sc"], qzeros=L["qz"])
    ms = tm.stop_ms() / reps
    return {"what": "awq_pack of the 7 Llama-7B block linears (g=128, zero_point)", "us": round(ms * 1e3, 2),
            "GB/s": round((in_bytes + out_bytes) / (ms * 1e-3) / 1e9, 1),
            "bytes": in_bytes + out_bytes,
            "frac_hbm": round((in_bytes + out_bytes) / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 3)}


def time_graph(torch, fn, iters, warm=3):
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    # capture on the warm-up stream: awq_gemm's split-K workspace is per
    # stream and is not created under capture
    with torch.cuda.graph(graph, stream=s):
        fn()
    for _ in range(warm):
        graph.replay()
    torch.cuda.synchronize()
    tm = Timer(torch)
    tm.start()
    for _ in range(iters):
        graph.replay()
    return tm.stop_ms() / iters, graph


def leg_fused_decode(torch, awq, workloads, g=128, zp=True, blocks=32, replays=20):
    """Single-token decode with the pages' fused projections: q/k/v as one
    4096 -> 12288 layer and gate/up as one 4096 -> 22016 layer, so a block is 4
    awq_gemv launches (qkv, o, gate_up, down) instead of 7.  Same weights and
    bytes as the unfused step; outputs are the concatenations."""
    names = [n for n, _, _ in workloads.LLAMA7B_BLOCK]
    Ws = {}
    for li, (name, K, N) in enumerate(workloads.LLAMA7B_BLOCK):
        Ws[name] = torch.from_numpy(workloads.weight(N, K, cfg=2, layer=li)).cuda()
    groups = [("qkv", ["q_proj", "k_proj", "v_proj"]), ("o", ["o_proj"]), ("gate_up", ["gate_proj", "up_proj"]),
              ("down", ["down_proj"])]
    fused = [(gname, awq.pack_fused([Ws[n] for n in parts], g, zp)) for gname, parts in groups]
    del Ws
    torch.cuda.synchronize()
    reps = []
    for _ in range(blocks):
        reps.append([awq.PackedWeight(pw.qweight.clone(), pw.scales.clone(), pw.qzeros.clone() if zp else None, pw.N,
                                      pw.K, pw.group_size, pw.zero_point) for _, pw in fused])
    xs = [torch.from_numpy(workloads.activations(1, pw.K, cfg=2, layer=i)).cuda() for i, (_, pw) in enumerate(fused)]
    ys = [torch.empty((1, pw.N), dtype=torch.float16, device="cuda") for _, pw in fused]

    def step():
        for rep in reps:
            for i, pw in enumerate(rep):
                awq.awq_gemv(xs[i], pw.qweight, pw.scales, pw.qzeros, pw.N, pw.K, g, zp, y=ys[i])

    ms, _ = time_graph(torch, step, replays)
    nbytes = blocks * sum(algorithmic_bytes(1, pw.N, pw.K, g, zp) for _, pw in fused)
    per = {}
    for i, (gname, pw) in enumerate(fused):
        def one(i=i):
            for rep in reps:
                pwr = rep[i]
                awq.awq_gemv(xs[i], pwr.qweight, pwr.scales, pwr.qzeros, pwr.N, pwr.K, g, zp, y=ys[i])

        ms_i, _ = time_graph(torch, one, replays)
        us = ms_i * 1e3 / blocks
        b = algorithmic_bytes(1, pw.N, pw.K, g, zp)
        per[gname] = {"K": pw.K, "N": pw.N, "us": round(us, 3), "GB/s": round(b / (us * 1e-6) / 1e9, 1)}
    del reps
    torch.cuda.empty_cache()
    return {"what": "decode through %d Llama-7B blocks with fused qkv and gate_up (4 awq_gemv per block)" % blocks,
            "ms_per_step": round(ms, 4), "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "per_layer": per}


def leg_batched_decode(torch, awq, workloads, g=128, zp=True, blocks=16, iters=20):
    """M = 4 / 16 / 64 tokens (and 1 and 256 for context) through the 7 linears
    of `blocks` distinct blocks."""
    out = {}
    base = []
    for li, (name, K, N) in enumerate(workloads.LLAMA7B_BLOCK):
        W = torch.from_numpy(workloads.weight(N, K, cfg=3, layer=li)).cuda()
        qw, sc, qz = awq.awq_pack(W, g, zp)
        base.append((K, N, qw, sc, qz))
    torch.cuda.synchronize()
    reps = [[(K, N, qw.clone(), sc.clone(), qz.clone()) for (K, N, qw, sc, qz) in base] for _ in range(blocks)]
    for M in (1, 4, 16, 64, 256):
        xs = [torch.from_numpy(workloads.activations(M, K, cfg=3, layer=li)).cuda()
              for li, (_, K, _) in enumerate(workloads.LLAMA7B_BLOCK)]
        ys = [torch.empty((M, N), dtype=torch.float16, device="cuda") for (_, _, N) in workloads.LLAMA7B_BLOCK]

        def step():
            for rep in reps:
                for i, (K, N, qw, sc, qz) in enumerate(rep):
                    awq.awq_gemm(xs[i], qw, sc, qz, N, K, g, zp, y=ys[i])

        ms, _ = time_graph(torch, step, iters)
        nbytes = blocks * sum(algorithmic_bytes(M, N, K, g, zp) for (_, K, N) in workloads.LLAMA7B_BLOCK)
        flops = blocks * sum(2 * M * N * K for (_, K, N) in workloads.LLAMA7B_BLOCK)
        out[f"M{M}"] = {"us_per_block": round(ms * 1e3 / blocks, 2), "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                        "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 3),
                        "TFLOPS": round(flops / (ms * 1e-3) / 1e12, 2)}
        if M == 1:
            def step_gemv():
                for rep in reps:
                    for i, (K, N, qw, sc, qz) in enumerate(rep):
                        awq.awq_gemv(xs[i], qw, sc, qz, N, K, g, zp, y=ys[i])

            ms_v, _ = time_graph(torch, step_gemv, iters)
            out["M1_gemv_vs_gemm"] = {"gemv_us_per_block": round(ms_v * 1e3 / blocks, 2),
                                      "gemm_us_per_block": round(ms * 1e3 / blocks, 2),
                                      "gemv_speedup": round(ms / ms_v, 3)}
    return out


def leg_dense_decode(torch, workloads, blocks=4, iters=20):
    """Context for the decode legs: torch's dense fp16 matrix product (the
    vendor library) on the unquantized weights of `blocks` distinct Llama-7B
    blocks (405 MB each, so no launch is served from the Infinity Cache), M =
    1 / 4 / 16 / 64, replayed from a HIP graph whose first replay is checked
    against the same products run eagerly.  A measured ceiling for the pages'
    "4-bit against FP16" comparison, not a product path."""
    out = {}
    Ws = [[torch.from_numpy(workloads.weight(N, K, cfg=3, layer=li)).cuda()
           for li, (_, K, N) in enumerate(workloads.LLAMA7B_BLOCK)]]
    for _ in range(blocks - 1):
        Ws.append([w.clone() for w in Ws[0]])
    for M in (1, 4, 16, 64):
        xs = [torch.from_numpy(workloads.activations(M, K, cfg=3, layer=li)).cuda()
              for li, (_, K, _) in enumerate(workloads.LLAMA7B_BLOCK)]
        ys = [torch.empty((M, N), dtype=torch.float16, device="cuda") for (_, _, N) in workloads.LLAMA7B_BLOCK]

        def step():
            for blk in Ws:
                for i, w in enumerate(blk):
                    torch.mm(xs[i], w.t(), out=ys[i])

        step()
        torch.cuda.synchronize()
        eager = [y.clone() for y in ys]
        for y in ys:
            y.zero_()
        ms, graph = time_graph(torch, step, iters)
        torch.cuda.synchronize()
        same = all(torch.equal(a, b) for a, b in zip(eager, ys))
        nbytes = blocks * sum(2 * K * N + 2 * M * K + 2 * M * N for (_, K, N) in workloads.LLAMA7B_BLOCK)
        out[f"M{M}"] = {"us_per_block": round(ms * 1e3 / blocks, 2), "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                        "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 3),
                        "graph_matches_eager": same}
        del graph
    del Ws
    torch.cuda.empty_cache()
    return out


def leg_sweep(torch, awq, workloads, blocks=16, iters=20):
    """Group-size and symmetry sweep over one Llama-7B block's 7 linears (the
    weights with per-row mean offsets, so that the zero points matter): for
    g = 32 / 128 / 256, with and without zero points, one token (awq_gemv) and
    8 tokens (awq_gemm).  Each step runs `blocks` distinct copies of the packed
    block, so no launch is served from the Infinity Cache."""
    Ws = [torch.from_numpy(workloads.weight(N, K, cfg=5, layer=li, row_offset=True)).cuda()
          for li, (_, K, N) in enumerate(workloads.LLAMA7B_BLOCK)]
    out = {}
    for g in (32, 128, 256):
        for zp in (True, False):
            base = [(K, N) + tuple(awq.awq_pack(W, g, zp)) for W, (_, K, N) in zip(Ws, workloads.LLAMA7B_BLOCK)]
            torch.cuda.synchronize()
            reps = [[(K, N, qw.clone(), sc.clone(), None if qz is None else qz.clone()) for (K, N, qw, sc, qz) in base]
                    for _ in range(blocks)]
            for M in (1, 8):
                xs = [torch.from_numpy(workloads.activations(M, K, cfg=5, layer=li)).cuda()
                      for li, (_, K, _) in enumerate(workloads.LLAMA7B_BLOCK)]
                ys = [torch.empty((M, N), dtype=torch.float16, device="cuda") for (_, _, N) in workloads.LLAMA7B_BLOCK]
                call = awq.awq_gemv if M == 1 else awq.awq_gemm

                def step():
                    for rep in reps:
                        for i, (K, N, qw, sc, qz) in enumerate(rep):
                            call(xs[i], qw, sc, qz, N, K, g, zp, y=ys[i])

                ms, _ = time_graph(torch, step, iters)
                nbytes = blocks * sum(algorithmic_bytes(M, N, K, g, zp) for (_, K, N) in workloads.LLAMA7B_BLOCK)
                out[f"g{g}_{'zp' if zp else 'sym'}_M{M}"] = {
                    "kernel": "awq_gemv" if M == 1 else "awq_gemm", "us_per_block": round(ms * 1e3 / blocks, 2),
                    "MB_per_block": round(nbytes / blocks / 1e6, 2), "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                    "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 3)}
            del reps, base
            torch.cuda.empty_cache()
    return out


def leg_gemv_70b(torch, awq, workloads, g=128, zp=True, replays=5):
    """Single-token awq_gemv on the two 70B-shaped MLP linears (122 MB each):
    at this size the launch floor that caps the 7B layers is a small part of a
    launch.  Enough distinct copies of each packed layer to total >= 1 GiB per
    graph replay, so no launch is served from the Infinity Cache."""
    out = {}
    for li, (name, K, N) in enumerate(workloads.LLAMA70B_MLP):
        W = torch.from_numpy(workloads.weight(N, K, cfg=4, layer=li)).cuda()
        base = awq.awq_pack(W, g, zp)
        del W
        nbytes = algorithmic_bytes(1, N, K, g, zp)
        copies = max(8, -(-(1 << 30) // nbytes))
        reps = [tuple(t.clone() for t in base) for _ in range(copies)]
        x = torch.from_numpy(workloads.activations(1, K, cfg=4, layer=li)).cuda()
        y = torch.empty((1, N), dtype=torch.float16, device="cuda")

        def step():
            for qw, sc, qz in reps:
                awq.awq_gemv(x, qw, sc, qz, N, K, g, zp, y=y)

        ms, _ = time_graph(torch, step, replays)
        us = ms * 1e3 / copies
        out[name] = {"K": K, "N": N, "MB": round(nbytes / 1e6, 1), "us": round(us, 2),
                     "GB/s": round(nbytes / us / 1e3, 1), "frac_hbm": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 3)}
        del reps, base
        torch.cuda.empty_cache()
    return out


def leg_prefill(torch, awq, workloads, g=128, zp=True, iters=30, warm=20, dense=True):
    """M = 2048 prefill through the two 70B-shaped MLP linears (matrix-core bound).

    The kernel runs at the chip's power limit, where the clock takes several
    milliseconds of load to settle: ``warm`` untimed launches (about 20 ms)
    come before the ``iters`` timed ones.  With ``dense``, torch's fp16 matrix
    product on the unquantized weights is timed the same way, as context (a
    measured ceiling from the vendor library, not a product path)."""
    out = {}
    M = 2048
    for li, (name, K, N) in enumerate(workloads.LLAMA70B_MLP):
        W = torch.from_numpy(workloads.weight(N, K, cfg=4, layer=li)).cuda()
        qw, sc, qz = awq.awq_pack(W, g, zp)
        if not dense:
            del W
        X = torch.from_numpy(workloads.activations(M, K, cfg=4, layer=li)).cuda()
        Y = torch.empty((M, N), dtype=torch.float16, device="cuda")
        for _ in range(warm):
            awq.awq_gemm(X, qw, sc, qz, N, K, g, zp, y=Y)
        torch.cuda.synchronize()
        tm = Timer(torch)
        tm.start()
        for _ in range(iters):
            awq.awq_gemm(X, qw, sc, qz, N, K, g, zp, y=Y)
        ms = tm.stop_ms() / iters
        tf = 2 * M * N * K / (ms * 1e-3) / 1e12
        out[name] = {"M": M, "K": K, "N": N, "us": round(ms * 1e3, 1), "TFLOPS": round(tf, 1),
                     "frac_mfma_fp16": round(tf / FP16_MFMA_PEAK_TFLOPS, 3)}
        if dense:
            # context: the vendor library's dense fp16 product on the same
            # (unquantized) weights and activations, same warm-up
            for _ in range(warm):
                torch.mm(X, W.t(), out=Y)
            torch.cuda.synchronize()
            tm.start()
            for _ in range(iters):
                torch.mm(X, W.t(), out=Y)
            dms = tm.stop_ms() / iters
            dtf = 2 * M * N * K / (dms * 1e-3) / 1e12
            out[name]["dense_fp16_torch_mm"] = {"us": round(dms * 1e3, 1), "TFLOPS": round(dtf, 1),
                                                "awq_speedup": round(dms / ms, 3)}
            del W
        del qw, sc, qz, X, Y
        torch.cuda.empty_cache()
    tot_f = sum(2 * M * N * K for (_, K, N) in workloads.LLAMA70B_MLP)
    tot_us = sum(v["us"] for v in out.values())
    out["both"] = {"TFLOPS": round(tot_f / (tot_us * 1e-6) / 1e12, 1),
                   "frac_mfma_fp16": round(tot_f / (tot_us * 1e-6) / 1e12 / FP16_MFMA_PEAK_TFLOPS, 3)}
    return out


def leg_scale_search(torch, awq, workloads, g=128, zp=True, M=512, count=20, iters=20):
    """Activation-aware scale search: L(s) for `count` candidate scale vectors
    s = a^alpha over M calibration tokens, on the Llama-7B q (4096x4096) and
    gate (4096->11008) shapes.  One pass over W gives every candidate's group
    scales and zero points; then per candidate one M x N x K product whose
    weight operand, the quantization error of W diag(s), is built in LDS next
    to the matrix cores, with a sum-of-squares epilogue."""
    out = {}
    alphas = [i / count for i in range(count)]
    for li, name in ((0, "q_proj"), (4, "gate_proj")):
        _, K, N = workloads.LLAMA7B_BLOCK[li]
        W = torch.from_numpy(workloads.weight(N, K, cfg=6, layer=li)).cuda()
        X = torch.from_numpy(workloads.activations(M, K, cfg=6, layer=li)).cuda()
        S = awq.awq_scale_candidates(X, alphas)
        for _ in range(3):
            L = awq.awq_scale_loss(X, W, S, g, zp)
        torch.cuda.synchronize()
        # one call after a synchronize, then the mean of back-to-back calls
        # (the steady state of a quantization run, which searches layer after
        # layer)
        tm = Timer(torch)
        tm.start()
        L = awq.awq_scale_loss(X, W, S, g, zp)
        first = tm.stop_ms()
        tm.start()
        for _ in range(iters):
            L = awq.awq_scale_loss(X, W, S, g, zp)
        ms = tm.stop_ms() / iters
        losses = L.cpu().tolist()
        best = min(range(count), key=lambda i: (losses[i], i))
        flops = 2.0 * M * N * K * count
        out[name] = {"M": M, "K": K, "N": N, "candidates": count, "us": round(ms * 1e3, 1),
                     "calls": iters, "us_first_call": round(first * 1e3, 1),
                     "us_per_candidate": round(ms * 1e3 / count, 2),
                     "TFLOPS_product": round(flops / (ms * 1e-3) / 1e12, 1),
                     "best_alpha": alphas[best], "L_rtn": round(losses[0], 4), "L_best": round(losses[best], 4)}
        del W, X, S, L
        torch.cuda.empty_cache()
    return out


def leg_clip_search(torch, awq, workloads, g=128, zp=True, M=512, iters=20):
    """Weight-clipping search (20 ratios, 1.0 down to 0.525) over M calibration
    tokens on the Llama-7B q (4096x4096) and gate (4096->11008) shapes: one
    pass over W gives every ratio's clipped bounds, scales and zero points;
    per ratio one M x N x K product whose weight operand, the
    clipped-quantization error, is built in LDS, with squares summed per
    weight group; then the choice and the clipped weights."""
    out = {}
    ratios = list(awq.DEFAULT_CLIP_RATIOS)
    for li, name in ((0, "q_proj"), (4, "gate_proj")):
        _, K, N = workloads.LLAMA7B_BLOCK[li]
        W = torch.from_numpy(workloads.weight(N, K, cfg=7, layer=li)).cuda()
        X = torch.from_numpy(workloads.activations(M, K, cfg=7, layer=li)).cuda()
        for _ in range(3):
            wc, choice = awq.awq_clip_search(X, W, g, zp, ratios)
        torch.cuda.synchronize()
        tm = Timer(torch)
        tm.start()
        wc, choice = awq.awq_clip_search(X, W, g, zp, ratios)
        first = tm.stop_ms()
        tm.start()
        for _ in range(iters):
            wc, choice = awq.awq_clip_search(X, W, g, zp, ratios)
        ms = tm.stop_ms() / iters
        hist = torch.bincount(choice.flatten().long(), minlength=len(ratios)).cpu().tolist()
        flops = 2.0 * M * N * K * len(ratios)
        out[name] = {"M": M, "K": K, "N": N, "ratios": len(ratios), "us": round(ms * 1e3, 1),
                     "calls": iters, "us_first_call": round(first * 1e3, 1),
                     "us_per_ratio": round(ms * 1e3 / len(ratios), 2),
                     "TFLOPS_product": round(flops / (ms * 1e-3) / 1e12, 1),
                     "groups_clipped": round(1.0 - hist[0] / sum(hist), 4)}
        del W, X, wc, choice
        torch.cuda.empty_cache()
    return out


def leg_loop(torch, awq, workloads, shape, launches=200, g=128, zp=True):
    """One shape for profiling: awq_gemm (M tokens, K -> N) launched
    ``launches`` times in a row, eagerly, over enough distinct copies of the
    packed weight to total >= 1 GiB (every launch reads HBM)."""
    M, N, K = shape
    W = torch.from_numpy(workloads.weight(N, K, cfg=3, layer=0)).cuda()
    base = awq.awq_pack(W, g, zp)
    del W
    nbytes = algorithmic_bytes(M, N, K, g, zp)
    copies = max(2, -(-(1 << 30) // (K * N // 2)))
    reps = [tuple(t.clone() if t is not None else None for t in base) for _ in range(copies)]
    x = torch.from_numpy(workloads.activations(M, K, cfg=3, layer=0)).cuda()
    y = torch.empty((M, N), dtype=torch.float16, device="cuda")
    for i in range(10):
        awq.awq_gemm(x, *reps[i % copies], N, K, g, zp, y=y)
    torch.cuda.synchronize()
    tm = Timer(torch)
    tm.start()
    for i in range(launches):
        awq.awq_gemm(x, *reps[i % copies], N, K, g, zp, y=y)
    us = tm.stop_ms() * 1e3 / launches
    return {"M": M, "N": N, "K": K, "copies": copies, "launches": launches, "us_per_launch_eager": round(us, 3),
            "GB/s": round(nbytes / us / 1e3, 1)}


def _smi_sample():
    """Socket power (amd-smi) and graphics clock (rocm-smi) of GPU 0, as text."""
    import subprocess

    out = {}
    try:
        r = subprocess.run(["amd-smi", "metric", "-p"], capture_output=True, text=True, timeout=20)
        for line in r.stdout.splitlines():
            if "SOCKET_POWER" in line:
                out["socket_power"] = line.split(":", 1)[1].strip()
                break
    except (OSError, subprocess.SubprocessError) as e:
        out["socket_power"] = f"unavailable ({e.__class__.__name__})"
    try:
        r = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True, timeout=20)
        for line in r.stdout.splitlines():
            if "sclk" in line:
                out["sclk"] = line.split(":", 2)[-1].strip()
                break
    except (OSError, subprocess.SubprocessError) as e:
        out["sclk"] = f"unavailable ({e.__class__.__name__})"
    return out


def leg_ceiling(torch, iters=20):
    """Measured HBM ceilings, for context only (never a roofline denominator):
    torch's device copy of 1 GiB (1 GiB read + 1 GiB written) and torch's sum
    over 1 GiB of fp16 (1 GiB read), each as GB/s of HBM bytes moved."""
    n = 1 << 30
    src = torch.empty(n // 2, dtype=torch.float16, device="cuda").normal_()
    dst = torch.empty_like(src)
    out = {}
    for name, fn, nbytes in (("copy_1GiB", lambda: dst.copy_(src), 2 * n), ("sum_1GiB_fp16", lambda: src.sum(), n)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        tm = Timer(torch)
        tm.start()
        for _ in range(iters):
            fn()
        ms = tm.stop_ms() / iters
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[name] = {"us": round(ms * 1e3, 1), "GB/s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 3)}
    del src, dst
    torch.cuda.empty_cache()
    return out


def leg_power(torch, awq, workloads, g=128, zp=True, seconds=2.0):
    """Power and clock of the prefill GEMM (70B down_proj, M = 2048) under
    sustained load, with the synthetic activations and with all-zero ones
    (the same kernel and instruction stream; fewer operand bit flips).  Shows
    whether the matrix-core kernel runs at the part's power limit."""
    import threading

    M = 2048
    name, K, N = workloads.LLAMA70B_MLP[1]
    W = torch.from_numpy(workloads.weight(N, K, cfg=4, layer=1)).cuda()
    qw, sc, qz = awq.awq_pack(W, g, zp)
    del W
    X = torch.from_numpy(workloads.activations(M, K, cfg=4, layer=1)).cuda()
    Y = torch.empty((M, N), dtype=torch.float16, device="cuda")
    out = {"shape": {"M": M, "K": K, "N": N}, "idle": _smi_sample()}
    for label, xin in (("synthetic_x", X), ("zero_x", torch.zeros_like(X))):
        stop = []

        def spin():
            while not stop:
                for _ in range(10):
                    awq.awq_gemm(xin, qw, sc, qz, N, K, g, zp, y=Y)
                torch.cuda.synchronize()

        th = threading.Thread(target=spin)
        th.start()
        time.sleep(seconds)
        sample = _smi_sample()
        stop.append(True)
        th.join()
        tm = Timer(torch)
        tm.start()
        for _ in range(20):
            awq.awq_gemm(xin, qw, sc, qz, N, K, g, zp, y=Y)
        ms = tm.stop_ms() / 20
        out[label] = dict(sample, us=round(ms * 1e3, 1), TFLOPS=round(2 * M * N * K / (ms * 1e-3) / 1e12, 1))
    return out


def _cpu_model():
    """Host CPU model name from lscpu (text), or 'unknown'."""
    import subprocess

    try:
        r = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10)
        for line in r.stdout.splitlines():
            if line.lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    return "unknown"


def cpu_baseline(layers, g, zp, timed=None, min_seconds=8.0, max_passes=40, pack_runs=2):
    """The CPU oracle as it stands on the seven linears of one block, M = 1:
    (i) quantize + pack, best of ``pack_runs``; (ii) unpack + fp64 decode +
    fp64 product, repeated for at least ``min_seconds`` (this is ``value``);
    and a prefill sample on a 70B-shaped layer (quantize + pack once, decode,
    fp64 product for 64 of the 2048 tokens).

    With ``timed`` (the GPU's packed block and the outputs of the timed decode
    graph), the oracle's results also check the run: the GPU packing of all
    seven layers must be bit-identical to the oracle's, and the last timed
    replay's outputs of block 0 must be within 1e-3 * sum |x w'| of the fp64
    product (every block's outputs bit-identical to block 0's, since the
    blocks hold copies of the same weights)."""
    import numpy as np

    import workloads
    from oracle import awq_oracle as O

    try:
        from threadpoolctl import threadpool_info

        blas_threads = max([d.get("num_threads", 1) for d in threadpool_info() if d.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover - threadpoolctl missing
        blas_threads = 1
    weights = sum(L["N"] * L["K"] for L in layers)
    pack_s = []
    packed = None
    for _ in range(pack_runs):
        t0 = time.perf_counter()
        packed = [O.pack(L["W"], g, zp) for L in layers]
        pack_s.append(time.perf_counter() - t0)
    pack_bytes = sum(2 * L["N"] * L["K"] + algorithmic_bytes(0, L["N"], L["K"], g, zp) for L in layers)

    t0 = time.perf_counter()
    nbytes = 0
    passes = 0
    refs = []
    while passes < max_passes and (passes == 0 or time.perf_counter() - t0 < min_seconds):
        for L, (qw, sc, qz) in zip(layers, packed):
            wdq = O.dequant_packed(qw, sc, qz, L["N"], L["K"], g, zp)
            yd = O.matmul_ref(L["X"], wdq)
            if passes == 0:
                refs.append(yd)
            nbytes += algorithmic_bytes(1, L["N"], L["K"], g, zp)
        passes += 1
    dt = time.perf_counter() - t0

    # prefill sample: the 70B-shaped up projection, 64 of the 2048 tokens
    _, Kp, Np = workloads.LLAMA70B_MLP[0]
    Mp = 64
    Wp = workloads.weight(Np, Kp, cfg=4, layer=0)
    Xp = workloads.activations(2048, Kp, cfg=4, layer=0)[:Mp]
    t1 = time.perf_counter()
    pp = O.pack(Wp, g, zp)
    t_pack = time.perf_counter() - t1
    t1 = time.perf_counter()
    O.matmul_ref(Xp, O.dequant_packed(*pp, Np, Kp, g, zp))
    t_prod = time.perf_counter() - t1
    del Wp, pp

    out = {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": blas_threads, "kind": "oracle",
           "seconds": round(dt, 2),
           "sample": f"{passes} passes over one Llama-7B block (7 linears, M=1, g=128, zero_point): oracle unpack + "
                     "fp64 decode + fp64 matmul (numpy; the product runs on the BLAS threads, the decode on one "
                     "core); value = algorithmic bytes / time",
           "host_cpu_count": os.cpu_count(), "cpu_model": _cpu_model(), "blas_threads": blas_threads,
           "quantize_pack": {"what": "oracle pack (quantize + store) of the same 7 linears, one core",
                             "seconds_best": round(min(pack_s), 3), "runs": pack_runs,
                             "Mweights_per_s": round(weights / min(pack_s) / 1e6, 2),
                             "GB/s": round(pack_bytes / min(pack_s) / 1e9, 4)},
           "decode_matmul": {"seconds_per_block": round(dt / passes, 3), "passes": passes},
           "prefill_sample": {"what": f"70B up_proj {Kp}->{Np}: oracle pack once, then decode + fp64 product "
                                      f"of {Mp} of the 2048 prefill tokens",
                              "pack_s": round(t_pack, 2), "decode_product_s": round(t_prod, 2),
                              "GFLOP/s_product_incl_decode": round(2.0 * Mp * Np * Kp / t_prod / 1e9, 2)}}
    check = None
    if timed is not None:
        pack_ok = True
        for L, (qw, sc, qz) in zip(layers, packed):
            pack_ok &= bool(np.array_equal(L["qw"].cpu().numpy().view(np.uint32), qw))
            pack_ok &= bool(np.array_equal(L["sc"].cpu().numpy().view(np.uint16), sc))
            if zp:
                pack_ok &= bool(np.array_equal(L["qz"].cpu().numpy().view(np.uint32), qz))
        worst = 0.0
        for y, (y_ref, d) in zip(timed["y_block0"], refs):
            r = O.tolerance_ratio(y.cpu().numpy().astype(np.float64), y_ref, d)
            worst = max(worst, float(np.max(r)))
        check = {"pack_bit_exact": pack_ok, "pack_layers": len(layers),
                 "gemv_worst_err_over_D": worst, "tolerance": 1e-3,
                 "blocks_identical": timed["blocks_identical"],
                 "what": "oracle packing of the block vs the GPU's, bit for bit; the timed graph's last outputs "
                         "(block 0, 7 layers) vs the fp64 product, |y - y_ref| <= 1e-3 * sum |x w'|",
                 "pass": bool(pack_ok and worst <= 1e-3 and timed["blocks_identical"])}
    return out, check


def summarize(db_paths, name_filter=None, last=None, pool=False):
    """Per-kernel summary of rocprofv3 SQLite databases (kernel-trace and/or
    --pmc runs): dispatch count, duration statistics (mean, median, minimum,
    10th and 90th percentiles) and, when present, the per-dispatch average of
    each collected counter.  With ``pool`` the selected dispatches of all the
    databases (each one's last ``last``) are summarized as one set.  Prints
    text."""
    import sqlite3
    import statistics

    def select(db):
        con = sqlite3.connect(db)
        rows = list(con.execute("select dispatch_id, name, duration, grid_x, workgroup_x from kernels "
                                "order by dispatch_id"))
        if name_filter:
            rows = [r for r in rows if name_filter in r[1]]
        if last:
            rows = rows[-last:]  # e.g. only the timed replays at the end of the run
        pmc = {}
        try:
            for kid, cname, val in con.execute("select dispatch_id, counter_name, counter_value from pmc_events"):
                pmc.setdefault(kid, {}).setdefault(cname, 0.0)
                pmc[kid][cname] += val
        except sqlite3.Error:
            pass
        return rows, pmc

    groups = []
    if pool:
        rows, pmc = [], {}
        for i, db in enumerate(db_paths):
            r, p = select(db)
            rows += [((i, kid), name, dur, grid, wg) for kid, name, dur, grid, wg in r]
            pmc.update({(i, kid): v for kid, v in p.items()})
        groups.append(("# pooled: " + " ".join(db_paths), rows, pmc))
    else:
        groups = [(f"# {db}",) + select(db) for db in db_paths]
    lines = []
    for head, rows, pmc in groups:
        lines.append(head)
        if last:
            lines.append(f"# the last {last} matching dispatches of each run: {len(rows)}")
        by = {}
        for kid, name, dur, grid, wg in rows:
            by.setdefault((name, grid, wg), []).append((kid, dur))
        for (name, grid, wg), ds in sorted(by.items(), key=lambda kv: -sum(d for _, d in kv[1])):
            durs = sorted(d for _, d in ds)
            p10 = durs[int(0.1 * (len(durs) - 1))]
            p90 = durs[int(0.9 * (len(durs) - 1))]
            line = (f"{name[:90]:90s} grid={grid:8d} wg={wg:4d} n={len(durs):5d} "
                    f"avg_us={statistics.mean(durs) / 1e3:9.3f} med_us={statistics.median(durs) / 1e3:9.3f} "
                    f"min_us={durs[0] / 1e3:9.3f} p10_us={p10 / 1e3:9.3f} p90_us={p90 / 1e3:9.3f}")
            cnt = {}
            for kid, _ in ds:
                for c, v in pmc.get(kid, {}).items():
                    cnt.setdefault(c, []).append(v)
            for c, vs in sorted(cnt.items()):
                line += f" {c}_avg={statistics.mean(vs):.1f}"
            lines.append(line)
    return "\n".join(lines)


def main():
    args = parse()
    if args.summarize:
        print(summarize(args.summarize, args.kernel_filter, args.last, args.pool))
        return 0
    if args.kernel_hash:
        print(kernel_hash(args.kernel_hash))
        return 0
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}))
        log("bench.py: the W4A16 layer benchmark is single-GPU; run with --gpus 1")
        return 2

    import torch

    import bit_weight_only_awq_amd as awq
    import workloads

    if not torch.cuda.is_available():
        log("bench.py needs a GPU")
        return 1
    awq.load_library()

    if args.copy_calibration:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "dispatches": 3}))
        return 0

    g, zp = 128, True
    if args.leg_only in ("fused", "batched", "dense", "prefill", "scale", "clip", "sweep", "gemv70b", "power",
                         "ceiling", "loop"):
        fn = {"fused": lambda: leg_fused_decode(torch, awq, workloads, g, zp, blocks=args.blocks),
              "batched": lambda: leg_batched_decode(torch, awq, workloads, g, zp),
              "dense": lambda: leg_dense_decode(torch, workloads),
              "prefill": lambda: leg_prefill(torch, awq, workloads, g, zp),
              "scale": lambda: leg_scale_search(torch, awq, workloads, g, zp),
              "clip": lambda: leg_clip_search(torch, awq, workloads, g, zp),
              "sweep": lambda: leg_sweep(torch, awq, workloads),
              "gemv70b": lambda: leg_gemv_70b(torch, awq, workloads, g, zp),
              "power": lambda: leg_power(torch, awq, workloads, g, zp),
              "ceiling": lambda: leg_ceiling(torch),
              "loop": lambda: leg_loop(torch, awq, workloads, tuple(int(v) for v in args.shape.split(",")),
                                       args.launches)}[args.leg_only]
        print(json.dumps({"leg": args.leg_only, "result": fn()}), flush=True)
        return 0
    log(f"building {args.blocks} decode blocks")
    layers, reps = build_decode_block(torch, awq, workloads, args.blocks, g, zp)
    step_bytes = args.blocks * sum(algorithmic_bytes(1, L["N"], L["K"], g, zp) for L in layers)
    launches = args.blocks * len(layers)

    def step():
        decode_step(awq, layers, reps, g, zp)

    log("capturing decode step")
    for _ in range(2):
        step()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        step()
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    t_wall = time.perf_counter()
    tm = Timer(torch)
    tm.start()
    for _ in range(args.steps):
        graph.replay()
    total_ms = tm.stop_ms()
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t_wall
    ms_per_step = total_ms / args.steps
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    # the timed graph holds nothing but back-to-back GEMV launches, so its
    # event-timed length per launch is the kernel's average launch duration
    avg_us = ms_per_step * 1e3 / launches
    bytes_per_launch = step_bytes / launches
    achieved = bytes_per_launch / (avg_us * 1e-6) / 1e9
    # outputs of the last timed replay, for the oracle check in the CPU baseline
    timed = {"y_block0": [R["y"].clone() for R in reps[0]],
             "blocks_identical": all(torch.equal(R["y"], R0["y"]) for rep in reps[1:]
                                     for R, R0 in zip(rep, reps[0]))}
    layer_stats = {}
    if not args.no_layer_timing:
        log("timing each layer shape")
        per_layer = per_layer_launch_times(torch, awq, layers, reps, g, zp)
        for L in layers:
            mu = per_layer[L["name"]]
            b = algorithmic_bytes(1, L["N"], L["K"], g, zp)
            layer_stats[L["name"]] = {"K": L["K"], "N": L["N"], "us": round(mu, 3),
                                      "GB/s": round(b / (mu * 1e-6) / 1e9, 1)}
    traffic, traffic_note = hbm_traffic(launches)

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": "llama7b_decode_gemv", "M": 1, "blocks": args.blocks,
                   "layers": "q,k,v,o 4096->4096; gate,up 4096->11008; down 11008->4096",
                   "group_size": g, "zero_point": zp, "launches_per_step": launches,
                   "bytes_per_step": step_bytes, "timed_wall_s": round(wall_s, 3)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic, "traffic_note": traffic_note,
                     "kernel": "gemv_kernel", "avg_launch_us": round(avg_us, 3),
                     "dispatch_stats": dispatch_stats(),
                     "bytes_per_launch": int(bytes_per_launch), "per_layer": layer_stats},
    }

    legs = set(args.legs.split(",")) if args.legs not in ("all", "none") else (
        {"pack", "fused", "batched", "dense", "prefill", "scale", "clip", "sweep", "gemv70b", "ceiling"}
        if args.legs == "all" else set())
    out_legs = {}
    if args.leg_only == "pack":
        print(json.dumps({"leg": "pack", "result": leg_pack(torch, awq, layers, g, zp)}), flush=True)
        return 0
    if "pack" in legs:
        log("leg: pack")
        out_legs["pack"] = leg_pack(torch, awq, layers, g, zp)
    del reps, graph
    torch.cuda.empty_cache()
    if "fused" in legs:
        log("leg: fused decode")
        out_legs["fused_decode_gemv"] = leg_fused_decode(torch, awq, workloads, g, zp, blocks=args.blocks)
    if "batched" in legs:
        log("leg: batched decode")
        out_legs["batched_decode_gemm"] = leg_batched_decode(torch, awq, workloads, g, zp)
    if "dense" in legs:
        log("leg: dense fp16 decode (torch, context)")
        dense = leg_dense_decode(torch, workloads)
        bd = out_legs.get("batched_decode_gemm")
        if bd:
            for M in (1, 4, 16, 64):
                ours = bd["M1_gemv_vs_gemm"]["gemv_us_per_block"] if M == 1 else bd[f"M{M}"]["us_per_block"]
                dense[f"M{M}"]["awq_speedup"] = round(dense[f"M{M}"]["us_per_block"] / ours, 3)
        out_legs["dense_fp16_decode_context"] = dense
    if "prefill" in legs:
        log("leg: prefill")
        out_legs["prefill_gemm_70b"] = leg_prefill(torch, awq, workloads, g, zp)
    if "scale" in legs:
        log("leg: scale search")
        out_legs["scale_search"] = leg_scale_search(torch, awq, workloads, g, zp)
    if "clip" in legs:
        log("leg: clip search")
        out_legs["clip_search"] = leg_clip_search(torch, awq, workloads, g, zp)
    if "sweep" in legs:
        log("leg: group-size / symmetry sweep")
        out_legs["sweep_7b_block"] = leg_sweep(torch, awq, workloads)
    if "gemv70b" in legs:
        log("leg: GEMV on the 70B MLP shapes")
        out_legs["gemv_70b_mlp"] = leg_gemv_70b(torch, awq, workloads, g, zp)
    if "ceiling" in legs:
        log("leg: HBM ceilings (torch copy and sum, context)")
        out_legs["hbm_ceiling_context"] = leg_ceiling(torch)
    if out_legs:
        result["legs"] = out_legs
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) and oracle check of the timed run")
        cb, check = cpu_baseline(layers, g, zp, timed)
        result["cpu_baseline"] = cb
        result["self_check"] = check
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
