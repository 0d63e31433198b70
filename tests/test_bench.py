"""Host logic of bench.py (CPU only): the one-GPU guard, the algorithmic byte
counts the roofline divides by, which kernel each workload's roofline is taken
on, and the two rocprofv3 summarizers (counter scaling, utilisation, clock),
run on small synthetic counter files in a scratch directory."""
import csv
import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr


# LM-head bytes per launch (weight codes + block scales + packed activation +
# outputs) as the survey's roofline table derives them for the five workloads
@pytest.mark.parametrize("M,H,V,want", [(4, 256, 1024, 263296), (1, 6144, 18944, 116426696),
                                        (64, 6144, 151552, 931768832), (320, 7168, 129280, 929273280),
                                        (8192, 6144, 151552, 983332864)])
def test_lmhead_bytes_match_the_derived_table(M, H, V, want):
    assert bench.lmhead_bytes(M, H, V) == want


def test_tail_bytes_add_the_rows_inputs_and_outputs():
    M, H, V = 1, 6144, 18944
    # bf16 hidden + residual read, fp32 norm weight read, bf16 hidden + codes + scales written
    assert bench.tail_bytes(M, H, V) - bench.lmhead_bytes(M, H, V) == 4 * H + 4 * H + 2 * H


@pytest.mark.parametrize("workload,kernel,kind", [("decode_c1_tp8_shard", "draft_tail1_kernel", "tail"),
                                                  ("decode_c64_full", "lmhead_kouter_kernel", "lmhead"),
                                                  ("mtp5_batch", "lmhead_gemm2_kernel", "lmhead"),
                                                  ("compute_stress", "lmhead_gemm2_kernel", "lmhead")])
def test_roofline_kernel_per_workload(workload, kernel, kind):
    from mtp_draft_head_amd import inputs

    w = inputs.get(workload)
    name, k, alg, plan, flops = bench.roofline_kernel("tail", w.M, w.H, w.V)
    assert (name, k) == (kernel, kind)
    assert plan.startswith(kernel)
    assert flops == 2.0 * w.M * w.H * w.V
    assert alg == (bench.tail_bytes if kind == "tail" else bench.lmhead_bytes)(w.M, w.H, w.V)


@pytest.fixture
def scratch_root(tmp_path, monkeypatch):
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_hash", lambda kernel: "hash-of-" + kernel)
    return tmp_path


def _counter_csv(path, rows):
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for i, (k, c, v) in enumerate(rows):
            wr.writerow({"Dispatch_Id": i, "Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})


def test_summarize_pmc_scales_each_counter_by_the_calibration_copy(scratch_root):
    kern = "void mtpd::lmhead_kouter_kernel<4, 2, 4, 5, 5>(unsigned char const*)"
    copy = "__amd_rocclr_copyBuffer"
    # a 1024 MiB copy: FETCH_SIZE reads half of it, WRITE_SIZE all of it
    _counter_csv(scratch_root / "f.csv", [(copy, "FETCH_SIZE", 524288.0), (copy, "FETCH_SIZE", 8.0),
                                          (kern, "FETCH_SIZE", 400000.0), (kern, "FETCH_SIZE", 500000.0)])
    _counter_csv(scratch_root / "w.csv", [(copy, "WRITE_SIZE", 1048576.0), (kern, "WRITE_SIZE", 600.0),
                                          (kern, "WRITE_SIZE", 700.0)])
    assert bench.summarize_pmc("decode_c64_full", str(scratch_root / "f.csv"), str(scratch_root / "w.csv"),
                               1024) == 0
    with open(bench.traffic_path("lmhead_kouter_kernel", "decode_c64_full")) as f:
        out = json.load(f)
    assert out["FETCH_SIZE"]["scale"] == 2.0 and out["WRITE_SIZE"]["scale"] == 1.0
    fetch = 450000.0 * 1024 * 2.0
    write = 650.0 * 1024 * 1.0
    assert out["bytes_per_launch"] == pytest.approx(fetch + write)
    assert out["traffic_over_algorithmic"] == pytest.approx((fetch + write) / 931768832)
    assert out["kernel_hash"] == "hash-of-lmhead_kouter_kernel"


def test_summarize_pmc_takes_only_the_roofline_launch_grid(scratch_root):
    """A variant that runs the same kernel at another grid (per-shard top-k
    launches beside the full one) does not dilute the per-launch traffic."""
    kern = "void mtpd::lmhead_stream_rows_kernel<4, 2, 4, 3, true>(unsigned char const*)"
    copy = "__amd_rocclr_copyBuffer"
    grid = 256 * 256   # the topk variant's roofline launch at c=64: grid=256x256

    def write(path, counter, rows):
        with open(path, "w", newline="") as f:
            wr = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name",
                                               "Counter_Value"])
            wr.writeheader()
            for i, (k, g, v) in enumerate(rows):
                wr.writerow({"Dispatch_Id": i, "Kernel_Name": k, "Grid_Size": g, "Counter_Name": counter,
                             "Counter_Value": v})
    write(scratch_root / "f.csv", "FETCH_SIZE", [(copy, 4096, 524288.0), (kern, grid, 455000.0),
                                                 (kern, 148 * 256, 57000.0), (kern, grid, 455000.0)])
    write(scratch_root / "w.csv", "WRITE_SIZE", [(copy, 4096, 1048576.0), (kern, grid, 100.0),
                                                 (kern, 148 * 256, 10.0)])
    assert bench.summarize_pmc("decode_c64_full", str(scratch_root / "f.csv"), str(scratch_root / "w.csv"),
                               1024, "topk") == 0
    with open(bench.traffic_path("lmhead_stream_rows_kernel", "decode_c64_full", "topk")) as f:
        out = json.load(f)
    assert out["FETCH_SIZE"]["kernel_dispatches"] == 2 and out["WRITE_SIZE"]["kernel_dispatches"] == 1
    assert out["bytes_per_launch"] == pytest.approx(455000.0 * 1024 * 2.0 + 100.0 * 1024)


def test_summarize_pmc_refuses_a_run_without_the_calibration_copy(scratch_root):
    kern = "void mtpd::lmhead_kouter_kernel<4, 2, 4, 5, 5>(unsigned char const*)"
    _counter_csv(scratch_root / "f.csv", [(kern, "FETCH_SIZE", 1.0)])
    _counter_csv(scratch_root / "w.csv", [(kern, "WRITE_SIZE", 1.0)])
    assert bench.summarize_pmc("decode_c64_full", str(scratch_root / "f.csv"), str(scratch_root / "w.csv"),
                               1024) == 1


def test_summarize_mfma_busy_fraction_flops_and_clock(scratch_root):
    kern = "void mtpd::lmhead_gemm2_kernel<8>(unsigned char const*)"
    gui = 8 * 14_000_000.0          # GRBM_GUI_ACTIVE summed over 8 XCCs: 14 M cycles each
    rows = []
    for _ in range(2):               # two dispatches, each counter in two pieces
        rows += [(kern, "SQ_VALU_MFMA_BUSY_CYCLES", 0.5 * 14_000_000.0 * 1024 / 2)] * 2
        rows += [(kern, "GRBM_GUI_ACTIVE", gui / 2)] * 2
        rows += [(kern, "SQ_INSTS_VALU_MFMA_MOPS_F8", 1000.0), (kern, "SQ_INSTS_VALU_MFMA_MOPS_F8", 1000.0)]
        rows += [(kern, "SQ_INSTS_VALU_MFMA_MOPS_F6F4", 0.0)]
    # dispatch ids must group a dispatch's counters: give both dispatches' rows their own id
    path = scratch_root / "m.csv"
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        half = len(rows) // 2
        for i, (k, c, v) in enumerate(rows):
            wr.writerow({"Dispatch_Id": 0 if i < half else 1, "Kernel_Name": k, "Counter_Name": c,
                         "Counter_Value": v})
    log = scratch_root / "bench.log"
    log.write_text("[bench] text\n" + json.dumps({"lmhead": {"us": 7000.0}}) + "\n")
    assert bench.summarize_mfma("compute_stress", str(path), str(log)) == 0
    with open(scratch_root / "profiles" / "lmhead_gemm2_kernel_compute_stress_mfma.json") as f:
        out = json.load(f)
    assert out["dispatches"] == 2
    assert out["mfma_busy_frac"] == pytest.approx(0.5)
    assert out["mfma_flops_per_dispatch"] == 2000.0 * 512
    assert out["clock_ghz"] == pytest.approx(14_000_000.0 / 7000e3)
