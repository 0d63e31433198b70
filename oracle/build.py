"""Build the CPU oracle (plain C, gcc, OpenMP) into oracle/_build/.

Strict IEEE arithmetic: no -ffast-math, no contraction into FMA, so every
fp64 operation in mtpd_oracle.c rounds exactly as written.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mtpd_oracle.c")
OUT_DIR = os.path.join(HERE, "_build")


def library_path() -> str:
    return os.path.join(OUT_DIR, "libmtpd_oracle.so")


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    out = library_path()
    tmp = out + f".tmp{os.getpid()}"
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-Wall", "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
