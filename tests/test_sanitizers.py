"""Host AddressSanitizer + UndefinedBehaviorSanitizer runs (CPU only).

Two drivers under tests/sanitize/ are built with -fsanitize=address,undefined
(-fno-sanitize-recover, so any report fails the run):
  - oracle_main.c with the oracle's C source (gcc): every oracle function on
    small ragged shapes;
  - abi_main.cpp with every libmtpd source (hipcc; the sanitizers apply to the
    host code only, the gfx950 code objects are built as usual): argument
    validation, size arithmetic, the plan strings and override parser, the
    error slot, on inputs that never reach a launch.
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "mtp_draft_head_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
LIB_SOURCES = ["mtpd_api.cpp", "norm_quant.hip", "lmhead_argmax.hip", "lmhead_decode.hip", "lmhead_gemm.hip",
               "lmhead_stream.hip", "argmax_combine.hip"]
# host-only sanitizer flags for hipcc: each -fsanitize= goes to the host pass
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_oracle_under_asan_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fopenmp", "-ffp-contract=off", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-Wall", "-o", exe,
          os.path.join(SAN, "oracle_main.c"), os.path.join(ROOT, "oracle", "mtpd_oracle.c"), "-lm"])
    r = _run([exe], env=dict(ENV, OMP_NUM_THREADS="4"), timeout=120)
    assert "oracle sanitizer run ok" in r.stdout
    assert "runtime error" not in r.stderr


def test_library_host_code_under_asan_ubsan(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]

    def compile_one(src):
        obj = str(tmp_path / (src + ".o"))
        _run([HIPCC, "-O1", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
              "-packed-fp32-ops", *HOST_SAN, "-Xarch_host", "-g", *inc, "-x", "hip", "-c",
              os.path.join(CSRC, src), "-o", obj])
        return obj

    with ThreadPoolExecutor(min(len(LIB_SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, LIB_SOURCES))
    main_obj = str(tmp_path / "abi_main.o")
    _run([HIPCC, "-O1", "-g", "-std=c++17", *HOST_SAN, *inc, "-c", os.path.join(SAN, "abi_main.cpp"), "-o",
          main_obj])
    exe = str(tmp_path / "abi_san")
    _run([HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
          "-fsanitize=undefined", "-o", exe, main_obj, *objs])
    r = _run([exe], env=ENV, timeout=120)
    assert "abi sanitizer run ok" in r.stdout
    assert "runtime error" not in r.stderr
