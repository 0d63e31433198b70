"""Fixtures under tests/golden/, each citing where its values come from."""
import os

import numpy as np

import oracle
from mtp_draft_head_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


def test_e4m3fn_format_table():
    for code, value in _rows("e4m3fn_format.txt"):
        c = np.uint8(int(code, 16))
        got = oracle.e4m3_decode(c)
        if value == "nan":
            assert np.isnan(got)
        else:
            assert got == float(value) and np.signbit(got) == value.startswith("-")
            assert oracle.e4m3_encode(np.array([float(value)]))[0] == c


def test_decode_c64_workload_matches_pages_gather_size():
    kv = dict(_rows("pages_logit_gather_bytes.txt"))
    w = inputs.get("decode_c64_full")
    assert w.M == int(kv["rows"]) and w.V == int(kv["vocab"])
    mb = w.M * w.V * int(kv["bytes_per_logit"]) / 1e6
    assert round(mb) == int(kv["approx_megabytes"])
