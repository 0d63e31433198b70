#!/usr/bin/env python3
"""Benchmark of the MTP draft-layer tail on one MI355X.

A step is one mtpd_draft_tail call (residual add + RMSNorm + packed FP8,
then the block-scaled FP8 LM head with the fused argmax) over one batch of
synthetic input already resident in HBM.  Default workload: the largest
single-GPU configuration, the compute-bound stress case (M=8192, H=6144,
V=151552), whose roofline is the FP8 MFMA peak.  The two decode
configurations that share its weight (c=64 on the full vocab, M=64; c=1 on
one GPU's TP8 vocab shard, M=1, V=18944) are timed in the same run and
reported as extra keys against the HBM peak ("companions").  Measured
achievable peaks (a streaming read of HBM and a loop of the same FP8 MFMA)
are reported beside the published ones ("measured_peaks").

Timing: W eager warmup steps, then K steps captured in one HIP graph and
replayed once, bracketed by device synchronizations and HIP events on the
stream the kernels run on.  The weight is rotated over enough copies that
the working set exceeds the 256 MB Infinity Cache.  The LM-head kernel is
also timed alone the same way (K launches in one graph).  The roofline is
taken on the step's dominant kernel: the fused tail when the library runs
the step as one kernel (then the step time is that kernel's time), else the
LM-head kernel timed alone.

Variants (--variant), each the same path computed another way, for the
steps next to it under tensor parallelism, on one GPU's share:
  tail           the step above (default)
  vocab_shards   norm_quant, then the LM head as 8 vocab-shard launches
                 (V/8 rows each) whose local (max, index) pairs one
                 argmax_combine launch reduces to the global draft token;
                 roofline on one shard launch
  allreduce_tail allreduce_norm_quant over 8 row-parallel bf16 partials
                 (standing in for the peers' outputs) + the LM head;
                 roofline on the all-reduce + norm kernel (the partial sets
                 are rotated past the Infinity Cache too)
  chain          5 successive MTP positions per step, each a draft_tail call
                 whose hidden input is the previous position's recycled bf16
                 hidden (an identity stand-in for the layer body, which needs
                 real weights; the residual is kept); the step is one graph
                 segment of 5 dependent tails, and the line reports the time
                 per position against a lone tail
  topk           norm_quant, then the LM head's top-k (--topk, default 8)
                 instead of the argmax: the streaming kernel writes sorted
                 per-(tile, wave) candidate lists and a merge launch selects;
                 roofline on the streaming kernel.  The same top-k as 8
                 vocab-shard launches merged by one topk_combine launch is
                 timed too (key topk_vocab_shards)

Prints ONE JSON line.  --gpus above 1 is refused: this build drives one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "draft rows/s + LM-head HBM GB/s (% of peak) for fused norm-quant-FP8-GEMM-argmax"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
FP8_PEAK_TFLOPS = 5000.0        # MI355X dense FP8 MFMA
CACHE_DEFEAT_BYTES = 768 << 20  # rotate weight copies past the 256 MB Infinity Cache
CSRC = "mtp_draft_head_amd/csrc/"
# the source a kernel is defined in; a traffic summary stays valid while that
# file and the shared headers are unchanged
KERNEL_SOURCE = {"lmhead_gemm_kernel": "lmhead_gemm.hip", "lmhead_gemm2_kernel": "lmhead_gemm.hip",
                 "lmhead_decode_kernel": "lmhead_decode.hip",
                 "lmhead_argmax_kernel": "lmhead_argmax.hip", "lmhead_stream_kernel": "lmhead_stream.hip",
                 "lmhead_stream_rows_kernel": "lmhead_stream.hip", "draft_tail1_kernel": "lmhead_stream.hip",
                 "lmhead_kouter_kernel": "lmhead_stream.hip",
                 "allreduce_norm_quant_kernel": "norm_quant.hip", "norm_quant_kernel": "norm_quant.hip",
                 "argmax_combine_kernel": "argmax_combine.hip"}
SHARED_HEADERS = ["lmhead_common.h", "device_common.h", "kernels.h"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_hash(kernel: str) -> str:
    """Digest of the kernel's own source file and the shared headers."""
    h = hashlib.sha256()
    for name in [KERNEL_SOURCE.get(kernel, "lmhead_argmax.hip")] + SHARED_HEADERS:
        with open(os.path.join(ROOT, CSRC + name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def lmhead_bytes(M, H, V) -> int:
    """Algorithmic bytes of one LM-head launch: weight codes and block scales,
    the packed activation (codes + scales) and the (max, idx) outputs."""
    return V * H + (V // 128) * (H // 128) * 4 + M * H + M * (H // 128) * 4 + M * 8


def tail_bytes(M, H, V) -> int:
    """Algorithmic bytes of one fused draft-tail launch: the LM head's weight
    codes and block scales, the rows' bf16 hidden and residual and the fp32
    norm weight read; the bf16 recycled hidden, the packed activation (codes
    + scales) and the (max, idx) outputs written."""
    return V * H + (V // 128) * (H // 128) * 4 + M * H * 2 * 2 + H * 4 + M * H * 2 + M * H + M * (H // 128) * 4 + M * 8


def dominant_kernel(M, H, V):
    """(kernel name, 'tail' | 'lmhead', algorithmic bytes per launch) of the
    launch that dominates a draft_tail step: the fused tail when the library
    runs the step as one kernel, else the LM-head kernel."""
    import mtp_draft_head_amd as mtpd

    plan = mtpd.draft_tail_plan(M, V, H)
    if "+" not in plan:
        return plan.split()[0], "tail", tail_bytes(M, H, V), plan
    lm = mtpd.lmhead_plan(M, V, H)
    return lm.split("<")[0].split()[0], "lmhead", lmhead_bytes(M, H, V), lm


N_SHARDS = 8      # vocab shards of the vocab_shards variant
N_PARTIALS = 8    # row-parallel partials of the allreduce_tail variant
N_CHAIN = 5       # MTP positions per step of the chain variant
TOPK_K = 8        # k of the topk variant (--topk)


def topk_list_bytes(M, V, k) -> int:
    """Candidate-list bytes one top-k pass writes: k keys per row for each of
    the 4 waves of every workgroup (one per CU, at most one per 128-row tile)."""
    return M * min(V // 128, 256) * 4 * k * 8


def allreduce_norm_bytes(P, M, H) -> int:
    """Algorithmic bytes of one allreduce_norm_quant launch: P partials and the
    residual read (bf16), the fp32 norm weight read once; the bf16 recycled
    hidden, the codes and the scales written."""
    return 2 * M * H * (P + 1) + 4 * H + 2 * M * H + M * H + M * (H // 128) * 4


def roofline_kernel(variant, M, H, V):
    """(kernel name, kind, algorithmic bytes per launch, plan, flops per launch)
    of the kernel a variant's roofline is taken on."""
    import mtp_draft_head_amd as mtpd

    if variant == "vocab_shards":
        Vs = V // N_SHARDS
        plan = mtpd.lmhead_plan(M, Vs, H)
        return plan.split("<")[0].split()[0], "lmhead", lmhead_bytes(M, H, Vs), plan, 2.0 * M * H * Vs
    if variant == "chain":
        variant = "tail"
    if variant == "topk":
        mt = 2 if M <= 32 else 4
        name = "lmhead_stream_rows_kernel"
        tiles = V // 128
        return (name, "lmhead", lmhead_bytes(min(M, 64), H, V) + topk_list_bytes(min(M, 64), V, TOPK_K),
                f"{name}<{mt},2,4,3,topk> grid={min(tiles, 256)}x256", 2.0 * min(M, 64) * H * V)
    if variant == "allreduce_tail":
        name = "allreduce_norm_quant_kernel"
        return name, "norm", allreduce_norm_bytes(N_PARTIALS, M, H), f"{name} grid={M}x256 P={N_PARTIALS}", 0.0
    kname, kind, alg, plan = dominant_kernel(M, H, V)
    return kname, kind, alg, plan, 2.0 * M * H * V


def traffic_path(kernel: str, workload: str, variant: str = "tail") -> str:
    tag = workload if variant == "tail" else f"{workload}_{variant}"
    return os.path.join(ROOT, "profiles", f"{kernel}_{tag}_traffic.json")


def traffic_from_profile(kernel: str, workload: str, variant: str = "tail"):
    """HBM bytes per launch measured by rocprofv3 counters (committed summary),
    or None when absent or taken on a different kernel source."""
    p = traffic_path(kernel, workload, variant)
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    if t.get("kernel_hash") != kernel_hash(kernel):
        return None
    return t.get("bytes_per_launch")


def _read_counters(path):
    """rocprofv3 counter-collection CSV -> list of (kernel_name, counter, value,
    dispatch id, grid size in threads) per dispatch."""
    import csv

    rows = []
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            rows.append((r.get("Kernel_Name", ""), r.get("Counter_Name", ""), float(r.get("Counter_Value", 0) or 0),
                         r.get("Dispatch_Id", ""), int(float(r.get("Grid_Size", 0) or 0))))
    return rows


def _plan_grid_threads(plan: str):
    """Threads of the launch a plan string names ("... grid=GxT ..."), or None."""
    import re

    m = re.search(r"grid=(\d+)x(\d+)", plan)
    return int(m.group(1)) * int(m.group(2)) if m else None


def summarize_pmc(workload: str, fetch_csv: str, write_csv: str, copy_mib: int, variant: str = "tail") -> int:
    """HBM bytes per launch of the step's dominant kernel from FETCH_SIZE /
    WRITE_SIZE (KiB per dispatch), each scaled by the reading of the same
    counter for the calibration copy, which reads and writes exactly
    copy_mib MiB.  Writes profiles/<kernel>_<workload>_traffic.json (and
    prints it)."""
    from mtp_draft_head_amd import inputs

    if copy_mib <= 0:
        print("--copy-calibration-mib must give the calibration copy size", file=sys.stderr)
        return 1
    w = inputs.get(workload)
    kname, _, alg, plan, _ = roofline_kernel(variant, w.M, w.H, w.V)
    out = {"workload": workload, "variant": variant, "kernel": plan, "kernel_hash": kernel_hash(kname),
           "algorithmic_bytes_per_launch": alg,
           "calibration_copy_bytes": copy_mib << 20}
    total = 0.0
    # the roofline launch only (a variant may run the same kernel at other
    # grid sizes, e.g. per-shard launches beside the full one)
    gthreads = _plan_grid_threads(plan)
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = [r for r in _read_counters(path) if r[1] == counter]
        copy = [v for k, c, v, _, _ in rows if "copy" in k.lower()]
        lm = [v for k, c, v, _, gs in rows if kname in k and (gthreads is None or gs in (0, gthreads))]
        if not copy or not lm:
            print(f"no copy or {kname} dispatches with {counter} in {path}", file=sys.stderr)
            return 1
        copy_kib = max(copy)                       # the calibration copy is the largest copy
        factor = (copy_mib << 20) / (copy_kib * 1024.0)
        lm_bytes = sum(lm) / len(lm) * 1024.0 * factor
        total += lm_bytes
        out[counter] = {"kernel_kib_per_dispatch": sum(lm) / len(lm), "kernel_dispatches": len(lm),
                        "copy_kib": copy_kib, "scale": factor, "bytes_per_launch": lm_bytes}
    out["bytes_per_launch"] = total
    out["traffic_over_algorithmic"] = total / alg
    vflag = "" if variant == "tail" else f" --variant {variant}"
    tag = workload if variant == "tail" else f"{workload}_{variant}"
    run = (f"python3 bench.py --no-cpu-baseline --no-peaks --no-companions --workload {workload}{vflag} "
           f"--steps 20 --warmup 5 "
           f"--copy-calibration-mib {copy_mib}")
    out["commands"] = [
        f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/pmcf_{tag} -o run -- {run}",
        f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/pmcw_{tag} -o run -- {run}",
        f"python3 bench.py --workload {workload}{vflag} --copy-calibration-mib {copy_mib} --summarize-pmc "
        f"gpurun_out/pmcf_{tag}/run_counter_collection.csv gpurun_out/pmcw_{tag}/run_counter_collection.csv",
    ]
    dst = traffic_path(kname, workload, variant)
    with open(dst, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))
    return 0


MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE", "SQ_INSTS_VALU_MFMA_MOPS_F8",
                 "SQ_INSTS_VALU_MFMA_MOPS_F6F4")
N_XCC, N_SIMD = 8, 1024   # MI355X: 8 XCDs, 256 CUs x 4 SIMDs


def summarize_mfma(workload: str, csv_path: str, bench_log: str) -> int:
    """Matrix-core utilisation of the step's dominant kernel from one
    rocprofv3 --pmc run of MFMA_COUNTERS: busy = SQ_VALU_MFMA_BUSY_CYCLES
    (summed over every SIMD) / (GRBM_GUI_ACTIVE per XCC x 1024 SIMDs);
    flops = (MOPS_F8 + MOPS_F6F4) x 512 (one MOP is 512 flops); the clock is
    GRBM_GUI_ACTIVE per XCC over the kernel's time in the same run's bench
    line.  Writes profiles/<kernel>_<workload>_mfma.json (and prints it)."""
    from mtp_draft_head_amd import inputs

    w = inputs.get(workload)
    kname, _, _, plan, flops_alg = roofline_kernel("tail", w.M, w.H, w.V)
    per = {}
    gthreads = _plan_grid_threads(plan)
    for k, c, v, disp, gs in _read_counters(csv_path):
        if kname in k and c in MFMA_COUNTERS and (gthreads is None or gs in (0, gthreads)):
            per.setdefault(disp, {}).setdefault(c, 0.0)
            per[disp][c] += v
    runs = [d for d in per.values() if all(c in d for c in MFMA_COUNTERS)]
    if not runs:
        print(f"no {kname} dispatch with all of {MFMA_COUNTERS} in {csv_path}", file=sys.stderr)
        return 1
    line = None
    with open(bench_log) as f:
        for ln in f:
            if ln.startswith("{"):
                line = json.loads(ln)
    us = line["lmhead"]["us"] if line and "lmhead" in line else None
    avg = {c: sum(d[c] for d in runs) / len(runs) for c in MFMA_COUNTERS}
    gui = avg["GRBM_GUI_ACTIVE"] / N_XCC
    mops = avg["SQ_INSTS_VALU_MFMA_MOPS_F8"] + avg["SQ_INSTS_VALU_MFMA_MOPS_F6F4"]
    out = {"workload": workload, "kernel": plan, "kernel_hash": kernel_hash(kname), "dispatches": len(runs),
           "counters_per_dispatch": avg,
           "mfma_busy_frac": avg["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui * N_SIMD),
           "mfma_flops_per_dispatch": mops * 512.0, "algorithmic_flops_per_launch": flops_alg,
           "kernel_us_in_bench_line": us,
           "clock_ghz": gui / (us * 1e3) if us else None,
           "commands": [
               f"rocprofv3 --pmc {' '.join(MFMA_COUNTERS)} --output-format csv -d gpurun_out/pmcm_{workload} -o run "
               f"-- python3 bench.py --no-cpu-baseline --no-peaks --no-companions --workload {workload} "
               f"--steps 5 --warmup 2",
               f"python3 bench.py --no-cpu-baseline --no-peaks --no-companions --workload {workload} "
               f"--steps 50 --warmup 5 > gpurun_out/pmcm_{workload}.log",
               f"python3 bench.py --workload {workload} --summarize-mfma "
               f"gpurun_out/pmcm_{workload}/run_counter_collection.csv gpurun_out/pmcm_{workload}.log"]}
    dst = os.path.join(ROOT, "profiles", f"{kname}_{workload}_mfma.json")
    with open(dst, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))
    return 0


def cpu_baseline(d, seconds: float, variant: str = "tail", parts=None):
    """The CPU oracle, as it stands, on a bounded sample of the same workload:
    the variant's full tail (norm + pack + LM head + argmax, with the partial
    sum or the shard combine where the variant has one) for n rows, n sized
    to take about `seconds`: a seeded draw of n distinct rows when n is below
    the workload's row count, else its rows taken cyclically."""
    import numpy as np

    import oracle

    w = d["workload"]
    H, V = w.H, w.V

    def pick(n):
        if n < w.M:
            return np.sort(np.random.default_rng(1234).choice(w.M, size=n, replace=False))
        return np.arange(n) % w.M

    def run(n):
        rows = pick(n)
        t0 = time.perf_counter()
        if variant == "allreduce_tail":
            nq = oracle.allreduce_norm_quant(parts[:, rows], d["residual"][rows], d["norm_weight"], d["eps"])
        else:
            nq = oracle.norm_quant(d["hidden"][rows], d["residual"][rows], d["norm_weight"], d["eps"])
        if variant == "vocab_shards":
            oracle.argmax_sharded(nq["codes"], nq["scales"], d["w_codes"], d["w_scales"], V // N_SHARDS)
        elif variant == "topk":
            oracle.topk(nq["codes"], nq["scales"], d["w_codes"], d["w_scales"], TOPK_K)
        else:
            oracle.argmax(nq["codes"], nq["scales"], d["w_codes"], d["w_scales"])
        return time.perf_counter() - t0

    t1 = run(1)
    n = max(1, min(4096, int(seconds / max(t1, 1e-4))))
    t = run(n)
    what = {"tail": "full tail", "chain": "full tail (one MTP position)",
            "topk": f"norm + pack + LM head + top-{TOPK_K}", "vocab_shards": f"full tail with {N_SHARDS} vocab shards combined",
            "allreduce_tail": f"full tail with the {N_PARTIALS}-partial sum"}[variant]
    return {"value": n / t, "unit": "rows/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{n} rows of {w.name} (M={w.M} H={H} V={V}, "
                      f"{'a seeded draw of distinct rows' if n < w.M else 'rows taken cyclically'}), {what} "
                      f"incl. the whole {V}-row LM head per row, fp64, {t:.1f} s"}


def measure_peaks(dev, log_fn):
    """Achievable peaks measured on this GPU by libmtpd_peaks: a streaming
    read of a 4 GiB buffer (non-temporal 16-byte loads, 4096 workgroups) and
    a register-only loop of the 16x16x128 E4M3 MFMA (1024 workgroups of 4
    waves, 8 independent accumulations each); best of 5 launches each."""
    import ctypes

    import torch

    from mtp_draft_head_amd import build as lib_build

    path = lib_build.peaks_library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built")
    L = ctypes.CDLL(path)
    L.mtpd_peak_read.restype = ctypes.c_int
    L.mtpd_peak_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    L.mtpd_peak_mfma.restype = ctypes.c_int
    L.mtpd_peak_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    L.mtpd_peak_mfma_random.restype = ctypes.c_int
    L.mtpd_peak_mfma_random.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p]
    stream = torch.cuda.current_stream(dev)
    nbytes, grid = 4 << 30, 4096
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    sink = torch.empty(grid * 256, dtype=torch.int32, device=dev)
    mgrid, iters = 1024, 2048
    mout = torch.empty(mgrid * 256, dtype=torch.float32, device=dev)
    # random E4M3 operand codes for the second MFMA loop, NaN codes (0x7f, 0xff) moved one step down
    gen = torch.Generator(device=dev)
    gen.manual_seed(20260)
    codes = torch.randint(0, 256, (mgrid * 256 * 32 * 4,), dtype=torch.int32, device=dev, generator=gen)
    codes = torch.where((codes & 0x7F) == 0x7F, codes - 1, codes).to(torch.uint8)
    words = codes.view(torch.int32)

    def best(fn, n=5):
        times = []
        for _ in range(n + 1):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            if fn() != 0:
                raise RuntimeError("peak probe launch failed")
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) * 1e-3)
        return min(times[1:])

    log_fn("[bench] measuring achievable peaks (HBM streaming read, FP8 MFMA loop)")
    t_read = best(lambda: L.mtpd_peak_read(buf.data_ptr(), nbytes, grid, sink.data_ptr(), stream.cuda_stream))
    t_mfma = best(lambda: L.mtpd_peak_mfma(iters, mgrid, mout.data_ptr(), stream.cuda_stream))
    t_mfma_r = best(lambda: L.mtpd_peak_mfma_random(iters, mgrid, words.data_ptr(), mout.data_ptr(),
                                                    stream.cuda_stream))
    flops = mgrid * 4 * iters * 8 * 65536.0
    del buf, sink, mout, codes, words
    return {"hbm_read_GBps": round(nbytes / t_read / 1e9, 1),
            "fp8_mfma_TFLOPs": round(flops / t_mfma / 1e12, 1),
            "fp8_mfma_random_operands_TFLOPs": round(flops / t_mfma_r / 1e12, 1),
            "how": "streaming read of 4 GiB (4096 workgroups, nt 16-byte loads); register-only loop of "
                   "v_mfma_f32_16x16x128_f8f6f4 (1024 workgroups x 4 waves x 8 accumulations) on near-constant "
                   "operands, and again on random E4M3 operands alternating between two sets per lane; best of 5"}


NQ_SHAPES = [(1, 6144), (8, 6144), (64, 6144), (320, 7168), (1024, 6144), (8192, 6144)]


def norm_quant_shapes(steps: int) -> int:
    """norm_quant in its two launch shapes, a workgroup per row (the library's)
    and a wavefront per row (plan override norm_quant=wave), at the decode,
    batched-drafting and compute-stress row counts: per shape, `steps`
    launches captured in one HIP graph and timed with HIP events, each kind
    twice, interleaved.  Prints one JSON line per shape (microseconds per
    launch and GB/s of the algorithmic bytes 7H + H/32 per row)."""
    import torch

    import mtp_draft_head_amd as mtpd

    dev = "cuda:0"
    for M, H in NQ_SHAPES:
        g = torch.Generator(device=dev).manual_seed(M)
        n = max(1, min(8, (256 << 20) // (M * H * 4)))   # input copies rotated past the Infinity Cache
        hs = [torch.randn(M, H, device=dev, generator=g).to(torch.bfloat16) for _ in range(n)]
        rs = [torch.randn(M, H, device=dev, generator=g).to(torch.bfloat16) for _ in range(n)]
        w = torch.rand(H, device=dev, generator=g) + 0.5
        out = (torch.empty(M, H, dtype=torch.bfloat16, device=dev), torch.empty(M, H, dtype=torch.uint8, device=dev),
               torch.empty(M, H // 128, dtype=torch.float32, device=dev))
        row = {"M": M, "H": H}
        for kind in ["workgroup", "wave", "workgroup", "wave"]:
            with mtpd.plan_override(norm_quant=kind):
                plan = mtpd.draft_tail_plan(max(M, 2), 256, H).split(" + ")[0]
                for i in range(3):
                    mtpd.norm_quant(hs[i % n], rs[i % n], w, 1e-6, out=out)
                torch.cuda.synchronize()
                s = torch.cuda.Stream()
                s.wait_stream(torch.cuda.current_stream())
                graph = torch.cuda.CUDAGraph()
                with torch.cuda.graph(graph, stream=s):
                    for i in range(steps):
                        mtpd.norm_quant(hs[i % n], rs[i % n], w, 1e-6, out=out)
                torch.cuda.synchronize()
                graph.replay()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(s)
                with torch.cuda.stream(s):
                    graph.replay()
                e1.record(s)
                torch.cuda.synchronize()
                row.setdefault(kind, {"kernel": plan, "us": []})["us"].append(round(e0.elapsed_time(e1) * 1e3 / steps, 2))
        nbytes = 7 * M * H + M * H // 32
        for kind in ("workgroup", "wave"):
            row[kind]["GB/s"] = round(nbytes / min(row[kind]["us"]) / 1e3, 1)
        print(json.dumps(row), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="compute_stress")
    ap.add_argument("--no-companions", action="store_true",
                    help="skip timing the decode configurations that share the workload's weight")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured achievable peaks")
    ap.add_argument("--variant", default="tail", choices=["tail", "vocab_shards", "allreduce_tail", "chain", "topk"])
    ap.add_argument("--topk", type=int, default=8, help="k of the topk variant (1..32)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one device-to-device copy of this many MiB first (a counter reference for PMC runs)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter CSVs (FETCH_SIZE, WRITE_SIZE) of a run with "
                         "--copy-calibration-mib into the traffic summary under profiles/")
    ap.add_argument("--summarize-mfma", nargs=2, metavar=("PMC_CSV", "BENCH_LOG"),
                    help="turn a rocprofv3 --pmc CSV of the MFMA counters and a bench log of the same workload "
                         "into the matrix-core utilisation summary under profiles/")
    ap.add_argument("--norm-quant-shapes", action="store_true",
                    help="time norm_quant as a workgroup per row and as a wavefront per row at six row counts "
                         "(one JSON line per shape) instead of the step")
    args = ap.parse_args()
    global TOPK_K
    TOPK_K = args.topk
    if args.summarize_mfma:
        return summarize_mfma(args.workload, *args.summarize_mfma)
    if args.summarize_pmc:
        return summarize_pmc(args.workload, *args.summarize_pmc, args.copy_calibration_mib, args.variant)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py drives exactly one GPU: the multi-GPU path (vocab shards combined by a u64 max "
              "all-reduce) is design-only in this build; run with --gpus 1", file=sys.stderr)
        return 2

    if args.norm_quant_shapes:
        return norm_quant_shapes(min(args.steps, 50))

    import numpy as np
    import torch

    import mtp_draft_head_amd as mtpd
    from mtp_draft_head_amd import inputs

    variant = args.variant
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    w = inputs.get(args.workload)
    M, H, V = w.M, w.H, w.V
    if variant == "vocab_shards" and V % (N_SHARDS * 128):
        print(f"{w.name}: V={V} does not split into {N_SHARDS} shards of whole 128-row blocks", file=sys.stderr)
        return 2
    log(f"[bench] drawing workload {w.name}: M={M} H={H} V={V} (variant {variant})")
    d = inputs.make(w.name)

    hid = torch.from_numpy(d["hidden"].view(np.int16)).to(dev).view(torch.bfloat16)
    res = torch.from_numpy(d["residual"].view(np.int16)).to(dev).view(torch.bfloat16)
    g = torch.from_numpy(d["norm_weight"]).to(dev)
    wbytes = d["w_codes"].nbytes
    n_copies = max(1, math.ceil(CACHE_DEFEAT_BYTES / wbytes))
    wc0 = torch.from_numpy(d["w_codes"]).to(dev)
    ws0 = torch.from_numpy(d["w_scales"]).to(dev)
    wcs = [wc0] + [wc0.clone() for _ in range(n_copies - 1)]
    wss = [ws0] + [ws0.clone() for _ in range(n_copies - 1)]
    out = (torch.empty((M, H), dtype=torch.bfloat16, device=dev),
           torch.empty((M, H), dtype=torch.uint8, device=dev),
           torch.empty((M, H // 128), dtype=torch.float32, device=dev),
           torch.empty((M,), dtype=torch.float32, device=dev),
           torch.empty((M,), dtype=torch.int32, device=dev))
    lm_out = (torch.empty((M,), dtype=torch.float32, device=dev), torch.empty((M,), dtype=torch.int32, device=dev))
    wsp = mtpd.Workspace(dev, any_stream=True)   # eager warmup and graph capture share it, in order
    wsp.get(M)
    K, W = args.steps, args.warmup
    extra = {}

    parts_np = None
    if variant == "chain":
        chain_out = [tuple(torch.empty_like(x) for x in out) for _ in range(N_CHAIN - 1)] + [out]

        def step(i):
            hin = hid
            for p in range(N_CHAIN):
                mtpd.draft_tail(hin, res, g, d["eps"], wcs[(i * N_CHAIN + p) % n_copies],
                                wss[(i * N_CHAIN + p) % n_copies], workspace=wsp, out=chain_out[p])
                hin = chain_out[p][0]

        def kernel_step(i):
            mtpd.draft_tail(hid, res, g, d["eps"], wcs[i % n_copies], wss[i % n_copies], workspace=wsp, out=out)
    elif variant == "topk":
        tk_out = (torch.empty((M, TOPK_K), dtype=torch.float32, device=dev),
                  torch.empty((M, TOPK_K), dtype=torch.int32, device=dev))
        tk_ws = mtpd.Workspace(dev, any_stream=True)
        tk_ws.get_bytes(mtpd.topk_workspace_bytes(M, V, TOPK_K))

        def step(i):
            mtpd.norm_quant(hid, res, g, d["eps"], out=out[:3])
            mtpd.fp8_lmhead_topk(out[1], out[2], wcs[i % n_copies], wss[i % n_copies], TOPK_K, workspace=tk_ws,
                                 out=tk_out)

        def kernel_step(i):
            mtpd.fp8_lmhead_topk(out[1], out[2], wcs[i % n_copies], wss[i % n_copies], TOPK_K, workspace=tk_ws,
                                 out=tk_out)

        # the same top-k as N_SHARDS vocab-shard launches whose lists one
        # topk_combine launch merges (one GPU's share of each shard, timed as a step)
        tk_shards = V % (N_SHARDS * 128) == 0
        if tk_shards:
            S = V // N_SHARDS
            tk_offs = [k * S for k in range(N_SHARDS)]
            tk_parts = [[(wcs[c][k * S:(k + 1) * S], wss[c][k * S // 128:(k + 1) * S // 128])
                         for k in range(N_SHARDS)] for c in range(n_copies)]
            tk_lv = torch.empty((N_SHARDS, M, TOPK_K), dtype=torch.float32, device=dev)
            tk_li = torch.empty((N_SHARDS, M, TOPK_K), dtype=torch.int32, device=dev)
            tk_cout = (torch.empty((M, TOPK_K), dtype=torch.float32, device=dev),
                       torch.empty((M, TOPK_K), dtype=torch.int32, device=dev))
            tk_ws_s = mtpd.Workspace(dev, any_stream=True)
            tk_ws_s.get_bytes(mtpd.topk_workspace_bytes(M, S, TOPK_K))

            def topk_shard_step(i):
                mtpd.norm_quant(hid, res, g, d["eps"], out=out[:3])
                for k, (c, sc) in enumerate(tk_parts[i % n_copies]):
                    mtpd.fp8_lmhead_topk(out[1], out[2], c, sc, TOPK_K, workspace=tk_ws_s, out=(tk_lv[k], tk_li[k]))
                mtpd.topk_combine(tk_lv, tk_li, tk_offs, out=tk_cout)

            def topk_combine_step(i):
                mtpd.topk_combine(tk_lv, tk_li, tk_offs, out=tk_cout)
    elif variant == "tail":
        def step(i):
            mtpd.draft_tail(hid, res, g, d["eps"], wcs[i % n_copies], wss[i % n_copies], workspace=wsp, out=out)

        def kernel_step(i):
            mtpd.fp8_lmhead_argmax(out[1], out[2], wcs[i % n_copies], wss[i % n_copies], workspace=wsp, out=lm_out)
    elif variant == "vocab_shards":
        S = V // N_SHARDS
        offs = [k * S for k in range(N_SHARDS)]
        shards = [[(wcs[c][k * S:(k + 1) * S], wss[c][k * S // 128:(k + 1) * S // 128]) for k in range(N_SHARDS)]
                  for c in range(n_copies)]
        lmax = torch.empty((N_SHARDS, M), dtype=torch.float32, device=dev)
        lidx = torch.empty((N_SHARDS, M), dtype=torch.int32, device=dev)

        def step(i):
            mtpd.norm_quant(hid, res, g, d["eps"], out=out[:3])
            for k, (c, sc) in enumerate(shards[i % n_copies]):
                mtpd.fp8_lmhead_argmax(out[1], out[2], c, sc, workspace=wsp, out=(lmax[k], lidx[k]))
            mtpd.argmax_combine(lmax, lidx, offs, out=(out[3], out[4]))

        def kernel_step(i):
            c, sc = shards[(i // N_SHARDS) % n_copies][i % N_SHARDS]
            mtpd.fp8_lmhead_argmax(out[1], out[2], c, sc, workspace=wsp, out=lm_out)

        def combine_step(i):
            mtpd.argmax_combine(lmax, lidx, offs, out=lm_out)
    else:
        parts_np = inputs.partials(w.name, N_PARTIALS)
        pset = [torch.from_numpy(parts_np[p].view(np.int16)).to(dev).view(torch.bfloat16) for p in range(N_PARTIALS)]
        n_sets = max(1, math.ceil(CACHE_DEFEAT_BYTES / (N_PARTIALS * M * H * 2)))
        psets = [pset] + [[t.clone() for t in pset] for _ in range(n_sets - 1)]
        extra["partial_sets_rotated"] = n_sets

        def step(i):
            mtpd.allreduce_norm_quant(psets[i % n_sets], res, g, d["eps"], out=out[:3])
            mtpd.fp8_lmhead_argmax(out[1], out[2], wcs[i % n_copies], wss[i % n_copies], workspace=wsp,
                                   out=(out[3], out[4]))

        def kernel_step(i):
            mtpd.allreduce_norm_quant(psets[i % n_sets], res, g, d["eps"], out=out[:3])

        def lm_alone(i):
            mtpd.fp8_lmhead_argmax(out[1], out[2], wcs[i % n_copies], wss[i % n_copies], workspace=wsp, out=lm_out)

    if args.copy_calibration_mib:
        nb = args.copy_calibration_mib << 20
        src = torch.ones(nb, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy of {nb} bytes done")
        del src, dst

    plan = mtpd.lmhead_plan(M, V, H)
    tail_plan = mtpd.draft_tail_plan(M, V, H)
    kname, kind, alg, kplan, kflops = roofline_kernel(variant, M, H, V)
    if variant == "tail":
        log(f"[bench] draft_tail plan: {tail_plan}")
    log(f"[bench] roofline kernel: {kplan} ({kind})")
    log(f"[bench] warmup {W} eager steps ({n_copies} weight copies, {n_copies * wbytes / 2**20:.0f} MiB)")
    for i in range(W):
        step(i)
    torch.cuda.synchronize()

    # eager rate (host launch cost included), for reference only
    t0 = time.perf_counter()
    for i in range(K):
        step(i)
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / K

    def timed_graph(fn):
        graph = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream(device=dev)
        s.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(s):
            fn(0)    # one eager call on the capture stream before capture
        torch.cuda.current_stream(dev).wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            for i in range(K):
                fn(i)
        graph.replay()                       # untimed: graph upload
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream(dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / K, graph

    log(f"[bench] timing {K} steps (one HIP graph)")
    ms_step, g1 = timed_graph(step)
    # sanity: the timed outputs are the real ones
    result = tk_out[1] if variant == "topk" else out[4]
    torch.cuda.synchronize()
    ref_idx = result.clone()
    step(0)
    torch.cuda.synchronize()
    assert torch.equal(ref_idx, result), "graph replay and eager call disagree"
    log(f"[bench] timing {K} launches of the roofline kernel (one HIP graph)")
    ms_kernel, g2 = timed_graph(kernel_step)
    del g1, g2
    if variant == "vocab_shards":
        ms_comb, g3 = timed_graph(combine_step)
        del g3
        extra["argmax_combine_us"] = round(ms_comb * 1e3, 3)
    if variant == "topk" and tk_shards:
        ms_ts, g3 = timed_graph(topk_shard_step)
        ms_tc, g4 = timed_graph(topk_combine_step)
        del g3, g4
        extra["topk_vocab_shards"] = {"shards": N_SHARDS, "step_us": round(ms_ts * 1e3, 3),
                                      "topk_combine_us": round(ms_tc * 1e3, 3)}
    if variant == "allreduce_tail":
        ms_lm_alone, g3 = timed_graph(lm_alone)
        del g3

    flops = 2.0 * M * H * V
    # the roofline kernel's time: the fused tail is the whole step (one launch
    # per step); otherwise the kernel timed alone
    if variant == "chain":
        k_us = ms_kernel * 1e3 if kind == "tail" else None
    else:
        k_us = ms_step * 1e3 if kind == "tail" else ms_kernel * 1e3
    if k_us is None:
        raise SystemExit("the chain variant is defined for the one-row fused tail (decode_c1_tp8_shard)")
    gbps = alg / (k_us * 1e-6) / 1e9
    tflops = kflops / (k_us * 1e-6) / 1e12
    compute_bound = kflops / alg > (FP8_PEAK_TFLOPS * 1e12) / (HBM_PEAK_GBPS * 1e9)
    # the chain's roofline kernel is the lone tail's: same launch, same traffic summary
    traffic = traffic_from_profile(kname, w.name, "tail" if variant == "chain" else variant)
    if compute_bound:
        roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tflops / FP8_PEAK_TFLOPS, 4), "traffic": traffic}
    else:
        roof = {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": traffic}
    roof.update({"kernel": kplan, "avg_launch_us": round(k_us, 3),
                 "algorithmic_bytes_per_launch": alg, "flops_per_launch": kflops})

    # the full-vocab LM head alone (the tail's second launch), for reference
    if variant == "tail":
        lm_us = ms_kernel * 1e3
    elif variant == "chain":
        lm_us = None
        extra["positions_per_step"] = N_CHAIN
        extra["us_per_position_chained"] = round(ms_step * 1e3 / N_CHAIN, 3)
        extra["us_lone_tail"] = round(ms_kernel * 1e3, 3)
    elif variant == "allreduce_tail":
        lm_us = ms_lm_alone * 1e3
    else:
        lm_us = None
    lm_alg = lmhead_bytes(M, H, V)

    # the decode configurations that share this workload's weight, timed the
    # same way (a graph of K steps, weight copies rotated past the cache)
    companions = {}
    if variant == "tail" and not args.no_companions:
        for cname in ("decode_c64_full", "decode_c1_tp8_shard"):
            cw = inputs.get(cname)
            if cname == w.name or cw.H != H or cw.v_full != w.v_full or cw.V > V:
                continue
            cd = inputs.make(cname)
            assert np.array_equal(cd["w_codes"][:256], d["w_codes"][:256])   # the same weight family
            Mc, Vc = cw.M, cw.V
            ch = torch.from_numpy(cd["hidden"].view(np.int16)).to(dev).view(torch.bfloat16)
            cr = torch.from_numpy(cd["residual"].view(np.int16)).to(dev).view(torch.bfloat16)
            cg = torch.from_numpy(cd["norm_weight"]).to(dev)
            nc = max(1, math.ceil(CACHE_DEFEAT_BYTES / (Vc * H)))
            cwc = [wc0[:Vc]] + [wc0[:Vc].clone() for _ in range(nc - 1)]
            cws = [ws0[:Vc // 128]] + [ws0[:Vc // 128].clone() for _ in range(nc - 1)]
            cout = (torch.empty((Mc, H), dtype=torch.bfloat16, device=dev),
                    torch.empty((Mc, H), dtype=torch.uint8, device=dev),
                    torch.empty((Mc, H // 128), dtype=torch.float32, device=dev),
                    torch.empty((Mc,), dtype=torch.float32, device=dev),
                    torch.empty((Mc,), dtype=torch.int32, device=dev))
            clm = (torch.empty((Mc,), dtype=torch.float32, device=dev),
                   torch.empty((Mc,), dtype=torch.int32, device=dev))

            def cstep(i, ch=ch, cr=cr, cg=cg, cwc=cwc, cws=cws, cout=cout, nc=nc, eps=cd["eps"]):
                mtpd.draft_tail(ch, cr, cg, eps, cwc[i % nc], cws[i % nc], workspace=wsp, out=cout)

            def cker(i, cwc=cwc, cws=cws, cout=cout, clm=clm, nc=nc):
                mtpd.fp8_lmhead_argmax(cout[1], cout[2], cwc[i % nc], cws[i % nc], workspace=wsp, out=clm)

            log(f"[bench] companion {cname}: M={Mc} V={Vc}, {nc} weight copies; timing {K} steps")
            for i in range(W):
                cstep(i)
            ms_cs, gc1 = timed_graph(cstep)
            cref = cout[4].clone()
            cstep(0)
            torch.cuda.synchronize()
            assert torch.equal(cref, cout[4]), "companion graph replay and eager call disagree"
            ms_ck, gc2 = timed_graph(cker)
            del gc1, gc2
            ckname, ckind, calg, ckplan, _ = roofline_kernel("tail", Mc, H, Vc)
            ck_us = ms_cs * 1e3 if ckind == "tail" else ms_ck * 1e3
            cgbps = calg / (ck_us * 1e-6) / 1e9
            lm_alg_c = lmhead_bytes(Mc, H, Vc)
            companions[cname] = {
                "M": Mc, "H": H, "V": Vc, "weight_copies_rotated": nc,
                "ms_per_step": round(ms_cs, 5), "rows_per_s": round(Mc / (ms_cs * 1e-3), 1),
                "draft_tail_plan": mtpd.draft_tail_plan(Mc, Vc, H),
                "roofline": {"bound": "hbm", "achieved": round(cgbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                             "frac": round(cgbps / HBM_PEAK_GBPS, 4),
                             "traffic": traffic_from_profile(ckname, cname, "tail"),
                             "kernel": ckplan, "avg_launch_us": round(ck_us, 3),
                             "algorithmic_bytes_per_launch": calg},
                "lmhead": {"kernel": mtpd.lmhead_plan(Mc, Vc, H), "us": round(ms_ck * 1e3, 3),
                           "hbm_frac": round(lm_alg_c / (ms_ck * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)},
            }
            del cwc, cws, cout
    peaks = None if args.no_peaks else measure_peaks(dev, log)

    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] timing the CPU oracle (~{args.cpu_seconds:.0f} s)")
        cpu = cpu_baseline(d, args.cpu_seconds, variant, parts_np)

    config = {"workload": w.name, "M": M, "H": H, "V": V, "eps": d["eps"],
              "weight_copies_rotated": n_copies, "timing": "K steps in one HIP graph"}
    if variant != "tail":
        config["variant"] = variant
        config.update({"vocab_shards": {"shards": N_SHARDS}, "allreduce_tail": {"partials": N_PARTIALS},
                       "chain": {"positions": N_CHAIN}, "topk": {"k": TOPK_K}}[variant])
    rows_per_step = M * (N_CHAIN if variant == "chain" else 1)
    rec = {
        "metric": METRIC,
        "value": round(rows_per_step / (ms_step * 1e-3), 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic",
        "config": config,
    }
    if variant in ("tail", "chain"):
        rec["draft_tail_plan"] = tail_plan
    if lm_us is not None:
        rec["lmhead"] = {"kernel": plan, "us": round(lm_us, 3), "GB/s": round(lm_alg / (lm_us * 1e-6) / 1e9, 1),
                         "TFLOP/s": round(flops / (lm_us * 1e-6) / 1e12, 2),
                         "hbm_frac": round(lm_alg / (lm_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                         "fp8_frac": round(flops / (lm_us * 1e-6) / 1e12 / FP8_PEAK_TFLOPS, 4)}
    rec.update(extra)
    if peaks is not None:
        roof["frac_of_measured"] = round(roof["achieved"] / (peaks["fp8_mfma_TFLOPs"] if roof["unit"] == "TFLOP/s"
                                                             else peaks["hbm_read_GBps"]), 4)
        for c in companions.values():
            c["roofline"]["frac_of_measured"] = round(c["roofline"]["achieved"] / peaks["hbm_read_GBps"], 4)
        rec["measured_peaks"] = peaks
    if companions:
        rec["companions"] = companions
    rec.update({"eager_ms_per_step": round(eager_ms, 5), "roofline": roof, "cpu_baseline": cpu})
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
