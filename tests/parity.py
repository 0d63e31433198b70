"""Element-wise comparison of GPU results with the CPU oracle, to the tolerances
the tail is held to:

  E4M3 codes      bit-exact on >= 99.9% of elements, within 1 code elsewhere
                  (distance in the ordered list of finite E4M3 values, +0 and
                  -0 counted as one value)
  scales          within 1e-6 relative (zero exactly where the oracle's is zero)
  bf16 hidden     within 1 bf16 ulp (adjacent in the ordered list of bf16 values)
  max logit       within 1e-3 relative
  argmax index    exact, except on near-ties: when the oracle's top-2 gap
                  (z1 - z2) / |z1| is below 1e-3 and the two are not an exact
                  tie, any index whose logit is >= z1 - 1e-3 |z1| is accepted.
                  Exact ties (identical logits) must give the lowest index.
"""
from __future__ import annotations

import numpy as np

CODE_EXACT_FRACTION = 0.999
SCALE_RTOL = 1e-6
MAX_RTOL = 1e-3
NEAR_TIE_RTOL = 1e-3


def e4m3_rank(codes: np.ndarray) -> np.ndarray:
    """Position of each finite code in the ordered list of E4M3 values; +-0 -> 0."""
    c = codes.astype(np.int64)
    mag = c & 0x7F
    if np.any(mag == 0x7F):
        raise AssertionError("NaN code present")
    return np.where(c & 0x80, -mag, mag)


def bf16_ordinal(bits: np.ndarray) -> np.ndarray:
    b = bits.astype(np.int64) & 0xFFFF
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def check_codes(gpu: np.ndarray, ref: np.ndarray, what="codes"):
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    d = np.abs(e4m3_rank(gpu) - e4m3_rank(ref))
    exact = float(np.mean(d == 0)) if d.size else 1.0
    worst = int(d.max()) if d.size else 0
    assert worst <= 1, f"{what}: a code differs by {worst} steps"
    assert exact >= CODE_EXACT_FRACTION, f"{what}: only {exact:.6f} bit-exact"
    return dict(exact_fraction=exact, max_steps=worst, mismatches=int(np.sum(d != 0)))


def check_scales(gpu: np.ndarray, ref: np.ndarray):
    assert gpu.shape == ref.shape
    g, r = gpu.astype(np.float64), ref.astype(np.float64)
    assert np.array_equal(g == 0, r == 0), "scale zero pattern differs"
    rel = np.abs(g - r) / np.where(r == 0, 1.0, np.abs(r))
    worst = float(rel.max()) if rel.size else 0.0
    assert worst <= SCALE_RTOL, f"scale rel err {worst:.3e}"
    return dict(max_rel=worst)


def check_bf16(gpu: np.ndarray, ref: np.ndarray):
    assert gpu.shape == ref.shape
    d = np.abs(bf16_ordinal(gpu) - bf16_ordinal(ref))
    worst = int(d.max()) if d.size else 0
    assert worst <= 1, f"bf16 differs by {worst} ulp"
    return dict(max_ulp=worst, exact_fraction=float(np.mean(d == 0)) if d.size else 1.0)


def check_argmax(gpu_max, gpu_idx, ora, logit_row=None):
    """ora: dict from oracle.argmax on the same packed activation and weight.

    logit_row(i) -> the oracle's fp64 logits of row i (only called for rows
    where the GPU picked another index inside the near-tie band)."""
    gpu_max = np.asarray(gpu_max, np.float32)
    gpu_idx = np.asarray(gpu_idx, np.int64)
    omax, oidx, z1, z2 = ora["max"], ora["idx"].astype(np.int64), ora["z1"], ora["z2"]
    n = len(oidx)
    assert gpu_max.shape == (n,) and gpu_idx.shape == (n,)
    rel = np.abs(gpu_max.astype(np.float64) - omax) / np.maximum(np.abs(omax.astype(np.float64)), 1e-30)
    worst = float(rel.max()) if n else 0.0
    assert worst <= MAX_RTOL, f"max logit rel err {worst:.3e}"
    gap = (z1 - z2) / np.maximum(np.abs(z1), 1e-300)
    near = (gap < NEAR_TIE_RTOL) & (z1 != z2)
    diff = gpu_idx != oidx
    bad = diff & ~near
    assert not np.any(bad), (
        f"argmax differs outside the near-tie band at rows {np.nonzero(bad)[0][:10].tolist()}: "
        f"gpu {gpu_idx[bad][:10].tolist()} oracle {oidx[bad][:10].tolist()} gap {gap[bad][:10].tolist()}")
    for i in np.nonzero(diff & near)[0]:
        z = logit_row(int(i))
        assert z[gpu_idx[i]] >= z1[i] - NEAR_TIE_RTOL * abs(z1[i]), f"row {i}: index outside near-tie band"
    return dict(max_rel=worst, near_tie_rows=int(np.sum(near)), near_tie_differ=int(np.sum(diff & near)))


def check_topk(gpu_val, gpu_idx, ora_val, ora_idx, logit_row):
    """Top-k lists against the oracle's, row by row.

    The GPU list must be in non-increasing value order with distinct indices;
    its values must match the oracle's sorted values position by position
    within MAX_RTOL; an index may differ from the oracle's only inside the
    near-tie band: its oracle logit lies within NEAR_TIE_RTOL |z| of the
    oracle's value at that position.  logit_row(i) -> the oracle's fp64 logits
    of row i (called only for rows with a differing index)."""
    gv = np.asarray(gpu_val, np.float32).astype(np.float64)
    gi = np.asarray(gpu_idx, np.int64)
    ov = np.asarray(ora_val, np.float32).astype(np.float64)
    oi = np.asarray(ora_idx, np.int64)
    assert gv.shape == ov.shape and gi.shape == oi.shape
    n, k = gv.shape
    rel = np.abs(gv - ov) / np.maximum(np.abs(ov), 1e-30)
    worst = float(rel.max()) if rel.size else 0.0
    assert worst <= MAX_RTOL, f"top-k value rel err {worst:.3e}"
    assert np.all(np.diff(gv, axis=1) <= 0), "top-k values not in descending order"
    differ = 0
    for i in range(n):
        assert len(set(gi[i].tolist())) == k, f"row {i}: repeated index"
        if np.array_equal(gi[i], oi[i]):
            continue
        z = logit_row(i)
        for e in np.nonzero(gi[i] != oi[i])[0]:
            differ += 1
            assert abs(z[gi[i, e]] - ov[i, e]) <= NEAR_TIE_RTOL * abs(ov[i, e]), (
                f"row {i} position {e}: index {gi[i, e]} (logit {z[gi[i, e]]}) outside the near-tie band of "
                f"{ov[i, e]}")
    return dict(max_rel=worst, near_tie_differ=differ)
