"""Build libmtpd.so (gfx950) in-tree with hipcc.

Output: mtp_draft_head_amd/_build/libmtpd.so.  Each translation unit is
compiled separately (in parallel), then linked.  Packed fp32 VALU ops are
disabled for all device code.
"""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["mtpd_api.cpp", "norm_quant.hip", "lmhead_argmax.hip", "lmhead_decode.hip", "lmhead_gemm.hip",
           "lmhead_stream.hip", "argmax_combine.hip"]

COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]


# per-file extras: the streaming kernel keeps MFMA results in VGPRs (its
# promotion FMAs read them at once; the AGPR form adds a copy per value)
EXTRA = {"lmhead_stream.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


# measured-peak probes (a streaming read and an FP8 MFMA loop) used by the
# benchmark's roofline; a library of their own, never linked into libmtpd
PEAK_SOURCES = ["peak_probe.hip"]


def library_path() -> str:
    return os.path.join(OUT_DIR, "libmtpd.so")


def peaks_library_path() -> str:
    return os.path.join(OUT_DIR, "libmtpd_peaks.so")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(OUT_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, *EXTRA.get(src, []), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, out: str, verbose: bool) -> str:
    tmp = out + f".tmp{os.getpid()}"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    srcs = SOURCES + PEAK_SOURCES
    with ThreadPoolExecutor(len(srcs)) as ex:
        objs = dict(zip(srcs, ex.map(lambda s: _compile(s, verbose), srcs)))
    _link([objs[s] for s in PEAK_SOURCES], peaks_library_path(), verbose)
    return _link([objs[s] for s in SOURCES], library_path(), verbose)


if __name__ == "__main__":
    print(build(verbose=True))
