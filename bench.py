#!/usr/bin/env python3
"""Benchmark of the MTP draft-layer tail on one MI355X.

A step is one mtpd_draft_tail call (residual add + RMSNorm + packed FP8,
then the block-scaled FP8 LM head with the fused argmax) over one batch of
synthetic input already resident in HBM.  Default workload: decode c=1 on one
GPU's TP8 vocab shard (M=1, H=6144, V=18944).

Timing: W eager warmup steps, then K steps captured in one HIP graph and
replayed once, bracketed by device synchronizations and HIP events on the
stream the kernels run on.  The weight is rotated over enough copies that
the working set exceeds the 256 MB Infinity Cache.  The LM-head kernel is
also timed alone the same way (K launches in one graph).  The roofline is
taken on the step's dominant kernel: the fused tail when the library runs
the step as one kernel (then the step time is that kernel's time), else the
LM-head kernel timed alone.

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
KERNEL_SOURCES = ["mtp_draft_head_amd/csrc/lmhead_argmax.hip", "mtp_draft_head_amd/csrc/lmhead_decode.hip",
                  "mtp_draft_head_amd/csrc/lmhead_gemm.hip", "mtp_draft_head_amd/csrc/lmhead_stream.hip",
                  "mtp_draft_head_amd/csrc/norm_quant.hip",
                  "mtp_draft_head_amd/csrc/lmhead_common.h", "mtp_draft_head_amd/csrc/device_common.h",
                  "mtp_draft_head_amd/csrc/kernels.h"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
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


def traffic_path(kernel: str, workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")


def traffic_from_profile(kernel: str, workload: str):
    """HBM bytes per launch measured by rocprofv3 counters (committed summary),
    or None when absent or taken on a different kernel source."""
    p = traffic_path(kernel, workload)
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    if t.get("kernel_hash") != kernel_hash():
        return None
    return t.get("bytes_per_launch")


def _read_counters(path):
    """rocprofv3 counter-collection CSV -> list of (kernel_name, counter, value) per dispatch."""
    import csv

    rows = []
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            rows.append((r.get("Kernel_Name", ""), r.get("Counter_Name", ""), float(r.get("Counter_Value", 0) or 0),
                         r.get("Dispatch_Id", "")))
    return rows


def summarize_pmc(workload: str, fetch_csv: str, write_csv: str, copy_mib: int) -> int:
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
    kname, _, alg, plan = dominant_kernel(w.M, w.H, w.V)
    out = {"workload": workload, "kernel": plan, "kernel_hash": kernel_hash(), "algorithmic_bytes_per_launch": alg,
           "calibration_copy_bytes": copy_mib << 20}
    total = 0.0
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = [r for r in _read_counters(path) if r[1] == counter]
        copy = [v for k, c, v, _ in rows if "copy" in k.lower()]
        lm = [v for k, c, v, _ in rows if kname in k]
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
    run = f"python3 bench.py --no-cpu-baseline --workload {workload} --steps 20 --warmup 5 --copy-calibration-mib {copy_mib}"
    out["commands"] = [
        f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/pmcf_{workload} -o run -- {run}",
        f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/pmcw_{workload} -o run -- {run}",
        f"python3 bench.py --workload {workload} --copy-calibration-mib {copy_mib} --summarize-pmc "
        f"gpurun_out/pmcf_{workload}/run_counter_collection.csv gpurun_out/pmcw_{workload}/run_counter_collection.csv",
    ]
    dst = traffic_path(kname, workload)
    with open(dst, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))
    return 0


def cpu_baseline(d, seconds: float):
    """The CPU oracle, as it stands, on a bounded sample of the same workload:
    the full tail (norm + pack + LM head + argmax) for n rows drawn cyclically
    from the workload's rows, n sized to take about `seconds`."""
    import numpy as np

    import oracle

    w = d["workload"]
    H, V = w.H, w.V

    def run(n):
        rows = np.arange(n) % w.M
        t0 = time.perf_counter()
        nq = oracle.norm_quant(d["hidden"][rows], d["residual"][rows], d["norm_weight"], d["eps"])
        oracle.argmax(nq["codes"], nq["scales"], d["w_codes"], d["w_scales"])
        return time.perf_counter() - t0

    t1 = run(1)
    n = max(1, min(4096, int(seconds / max(t1, 1e-4))))
    t = run(n)
    return {"value": n / t, "unit": "rows/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{n} rows of {w.name} (M={w.M} H={H} V={V}, rows taken cyclically), full tail "
                      f"incl. the whole {V}-row LM head per row, fp64, {t:.1f} s"}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode_c1_tp8_shard")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one device-to-device copy of this many MiB first (a counter reference for PMC runs)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter CSVs (FETCH_SIZE, WRITE_SIZE) of a run with "
                         "--copy-calibration-mib into the LM-head traffic summary under profiles/")
    args = ap.parse_args()
    if args.summarize_pmc:
        return summarize_pmc(args.workload, *args.summarize_pmc, args.copy_calibration_mib)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py drives exactly one GPU: the multi-GPU path (vocab shards combined by a u64 max "
              "all-reduce) is design-only in this build; run with --gpus 1", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import mtp_draft_head_amd as mtpd
    from mtp_draft_head_amd import inputs

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    w = inputs.get(args.workload)
    M, H, V = w.M, w.H, w.V
    log(f"[bench] drawing workload {w.name}: M={M} H={H} V={V}")
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
    wsp = mtpd.Workspace(dev)
    wsp.get(M)
    K, W = args.steps, args.warmup

    def step(i):
        mtpd.draft_tail(hid, res, g, d["eps"], wcs[i % n_copies], wss[i % n_copies], workspace=wsp, out=out)

    def lm_step(i):
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
    kname, kind, alg, kplan = dominant_kernel(M, H, V)
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

    log(f"[bench] timing {K} draft_tail steps (one HIP graph)")
    ms_step, g1 = timed_graph(step)
    log(f"[bench] timing {K} LM-head launches (one HIP graph)")
    ms_lm, g2 = timed_graph(lm_step)
    del g1, g2

    # sanity: the timed outputs are the real ones
    torch.cuda.synchronize()
    ref_idx = out[4].clone()
    step(0)
    torch.cuda.synchronize()
    assert torch.equal(ref_idx, out[4]), "graph replay and eager call disagree"

    lm_us = ms_lm * 1e3
    lm_alg = lmhead_bytes(M, H, V)
    # the dominant kernel: the fused tail is the whole step (one launch per
    # step), else the LM-head kernel timed alone
    k_us = ms_step * 1e3 if kind == "tail" else lm_us
    flops = 2.0 * M * H * V
    gbps = alg / (k_us * 1e-6) / 1e9
    tflops = flops / (k_us * 1e-6) / 1e12
    compute_bound = flops / alg > (FP8_PEAK_TFLOPS * 1e12) / (HBM_PEAK_GBPS * 1e9)
    traffic = traffic_from_profile(kname, w.name)
    if compute_bound:
        roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tflops / FP8_PEAK_TFLOPS, 4), "traffic": traffic}
    else:
        roof = {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": traffic}
    roof.update({"kernel": kplan, "avg_launch_us": round(k_us, 3),
                 "algorithmic_bytes_per_launch": alg, "flops_per_launch": flops})

    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] timing the CPU oracle (~{args.cpu_seconds:.0f} s)")
        cpu = cpu_baseline(d, args.cpu_seconds)

    rec = {
        "metric": METRIC,
        "value": round(M / (ms_step * 1e-3), 1),
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
        "config": {"workload": w.name, "M": M, "H": H, "V": V, "eps": d["eps"],
                   "weight_copies_rotated": n_copies, "timing": "K steps in one HIP graph"},
        "draft_tail_plan": tail_plan,
        "lmhead": {"kernel": plan, "us": round(lm_us, 3), "GB/s": round(lm_alg / (lm_us * 1e-6) / 1e9, 1),
                   "TFLOP/s": round(flops / (lm_us * 1e-6) / 1e12, 2),
                   "hbm_frac": round(lm_alg / (lm_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                   "fp8_frac": round(flops / (lm_us * 1e-6) / 1e12 / FP8_PEAK_TFLOPS, 4)},
        "eager_ms_per_step": round(eager_ms, 5),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
