"""Seeded synthetic workloads for the MTP draft-layer tail.

This module only draws random inputs and shapes them; it holds none of the
tail's own arithmetic (no RMSNorm, no activation quantization, no GEMM, no
argmax).  Both the GPU path and the CPU oracle are fed from here.

The LM-head weight is an input that arrives already packed (E4M3FN codes plus
one fp32 scale per 128x128 block, scale = amax/448); the packing of the fp32
draw into codes is done with torch's own float8_e4m3fn cast, not with either
side's codec.

Workloads (M rows, H hidden, V vocab rows of this GPU's LM-head slice):

  tiny                 M=4,    H=256,  V=1024    no outliers; two planted exact
                                                 ties (rows 0 and 1)
  decode_c1_tp8_shard  M=1,    H=6144, V=18944   one GPU's 1/8 vocab shard of the
                                                 151552-row head (its first 148
                                                 blocks); 1% outlier channels x20
  decode_c64_full      M=64,   H=6144, V=151552  full vocab on one GPU
  mtp5_batch           M=320,  H=7168, V=129280  64 requests x 5 draft positions;
                                                 16 rows (5%) planted with a top-2
                                                 gap below 1e-3 relative
  compute_stress       M=8192, H=6144, V=151552  same weight as decode_c64_full

Distributions: hidden and residual N(0,1) in fp32, rounded to bf16; the
outlier channels (round(0.01*H) distinct columns, the same set in hidden and
residual and in every row) are scaled x20 before rounding.  Norm weight
U(0.5, 1.5) fp32; eps = 1e-6.  Weight N(0, 0.02) fp32, packed per 128x128
block.

Row-parallel partials (the inputs of the all-reduce folded into the norm):
P arrays [M, H], each N(0, 1/P) in fp32 with the workload's outlier channels
x20, rounded to bf16, so their sum has the spread of the hidden draw.

Seeding: numpy PCG64 from SeedSequence(entropy=0x4D545044, spawn_key=...).
Activations use spawn_key (workload_id, stream) with one stream per array.
The weight uses spawn_key (100, H, V_full, block) with one stream per 128-row
vocab block, so any block or shard can be regenerated on its own and blocks
are drawn in parallel; the 18944-row shard is literally blocks 0..147 of the
151552-row weight.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

ENTROPY = 0x4D545044
BLOCK = 128
EPS = 1e-6


@dataclasses.dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    M: int
    H: int
    V: int
    v_full: int          # vocab of the full head the weight family is drawn for
    outliers: bool
    description: str


WORKLOADS = {
    w.name: w
    for w in [
        Workload(1, "tiny", 4, 256, 1024, 1024, False,
                 "M=4 H=256 V=1024, two planted exact logit ties"),
        Workload(2, "decode_c1_tp8_shard", 1, 6144, 18944, 151552, True,
                 "decode c=1 on one GPU's TP8 vocab shard: M=1 H=6144 V=18944"),
        Workload(3, "decode_c64_full", 64, 6144, 151552, 151552, True,
                 "decode c=64, full vocab on one GPU: M=64 H=6144 V=151552"),
        Workload(4, "mtp5_batch", 320, 7168, 129280, 129280, True,
                 "64 requests x 5 draft positions: M=320 H=7168 V=129280, 5% near-tie rows"),
        Workload(5, "compute_stress", 8192, 6144, 151552, 151552, True,
                 "compute-bound stress: M=8192 H=6144 V=151552"),
    ]
}
BY_ID = {w.wid: w for w in WORKLOADS.values()}


def get(name_or_id) -> Workload:
    if isinstance(name_or_id, int):
        return BY_ID[name_or_id]
    return WORKLOADS[name_or_id]


def _rng(*key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(entropy=ENTROPY, spawn_key=tuple(key))))


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), via torch's round-to-nearest-even cast."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def _pack_e4m3_blocks(w: np.ndarray):
    """Pack an fp32 [R, H] weight (R a multiple of 128) per 128x128 block.

    scale = amax/448 in fp32; codes = torch float8_e4m3fn cast of w/scale
    (clamped to +-448 first, since that cast maps overflow to NaN).  A block
    whose amax is 0 gets scale 0 and zero codes.
    Returns (codes uint8 [R, H], scales float32 [R/128, H/128]).
    """
    R, H = w.shape
    t = torch.from_numpy(np.ascontiguousarray(w, dtype=np.float32))
    w4 = t.view(R // BLOCK, BLOCK, H // BLOCK, BLOCK)
    scales = w4.abs().amax(dim=(1, 3)) / 448.0
    safe = torch.where(scales == 0, torch.ones_like(scales), scales)
    q = (w4 / safe[:, None, :, None]).clamp_(-448.0, 448.0)
    q = torch.where(scales[:, None, :, None] == 0, torch.zeros_like(q), q)
    codes = q.reshape(R, H).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.numpy().copy(), scales.numpy().copy()


def _weight_block_fp32(H: int, v_full: int, b: int) -> np.ndarray:
    return _rng(100, H, v_full, b).standard_normal((BLOCK, H), dtype=np.float32) * np.float32(0.02)


def weight_family(H: int, v_full: int, n_blocks: int | None = None):
    """Packed weight for the first n_blocks 128-row blocks of the (H, v_full) family."""
    nb = v_full // BLOCK if n_blocks is None else n_blocks
    codes = np.empty((nb * BLOCK, H), np.uint8)
    scales = np.empty((nb, H // BLOCK), np.float32)

    def task(b):
        c, s = _pack_e4m3_blocks(_weight_block_fp32(H, v_full, b))
        codes[b * BLOCK:(b + 1) * BLOCK] = c
        scales[b] = s[0]

    torch_threads = torch.get_num_threads()
    torch.set_num_threads(1)
    try:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(task, range(nb)))
    finally:
        torch.set_num_threads(torch_threads)
    return codes, scales


def _activations(w: Workload):
    rng_h, rng_r, rng_g, rng_o = (_rng(w.wid, k) for k in range(4))
    h = rng_h.standard_normal((w.M, w.H), dtype=np.float32)
    r = rng_r.standard_normal((w.M, w.H), dtype=np.float32)
    g = rng_g.uniform(0.5, 1.5, size=w.H).astype(np.float32)
    outl = np.zeros((0,), np.int64)
    if w.outliers:
        n = int(round(0.01 * w.H))
        outl = np.sort(rng_o.choice(w.H, size=n, replace=False))
        h[:, outl] *= np.float32(20.0)
        r[:, outl] *= np.float32(20.0)
    return h, r, g, outl


def _align_row(h, r, m, w_code_row):
    """Give activation row m the signs of a weight code row, so that row's
    logit dominates every other logit of row m."""
    sgn = np.where(w_code_row & 0x80, np.float32(-1.0), np.float32(1.0))
    h[m] = np.abs(h[m]) * sgn
    r[m] = np.abs(r[m]) * sgn


def _tiny():
    w = WORKLOADS["tiny"]
    h, r, g, outl = _activations(w)
    rng_p = _rng(w.wid, 5)
    wf = np.concatenate([_weight_block_fp32(w.H, w.v_full, b) for b in range(w.V // BLOCK)])
    # keep every magnitude below the sentinel used for the cross-block tie
    np.clip(wf, -0.1, 0.1, out=wf)
    # tie 1 (row 0): an exact copy of the aligned row at a lower index of the
    # same 128-row block; same block => same scales => identical codes.
    t1_hi, t1_lo = 3 * BLOCK + 116, 3 * BLOCK + 16
    wf[t1_lo] = wf[t1_hi]
    # tie 2 (row 1): a copy across blocks 1 (lower) and 6.  A sentinel 0.12 in
    # one row of each block, once per 128-column block, pins every block amax
    # (hence every scale) of the two blocks to the same value.
    t2_hi, t2_lo = 6 * BLOCK + 40, 1 * BLOCK + 99
    for blk, sent_row in ((1, 1 * BLOCK + 5), (6, 6 * BLOCK + 77)):
        for kb in range(w.H // BLOCK):
            col = kb * BLOCK + int(rng_p.integers(BLOCK))
            wf[sent_row, col] = np.float32(0.12) * (1 if rng_p.integers(2) else -1)
    wf[t2_lo] = wf[t2_hi]
    codes, scales = _pack_e4m3_blocks(wf)
    _align_row(h, r, 0, codes[t1_hi])
    _align_row(h, r, 1, codes[t2_hi])
    meta = dict(outliers=outl, ties=[(0, t1_lo, t1_hi), (1, t2_lo, t2_hi)], near_tie_rows=[])
    return w, h, r, g, codes, scales, meta


def _mtp5_near_ties(w, h, r, codes, outl):
    """Plant 16 rows whose top-2 logits differ by well under 1e-3 relative.

    Each chosen row m is aligned with a weight row v*; a copy of v*'s codes goes
    to another row v' of the same 128-row block (same scales), and in the copy
    a few of the largest-magnitude codes outside the outlier channels move one
    code step toward zero.  Row m then has its best logit at v* and the
    runner-up at v', a small relative step below it.
    """
    rng_p = _rng(w.wid, 5)
    n_plant = 16
    rows = np.sort(rng_p.choice(w.M, size=n_plant, replace=False))
    blocks = rng_p.choice(w.V // BLOCK, size=n_plant, replace=False)
    mask = np.ones(w.H, bool)
    mask[outl] = False
    planted = []
    for m, blk in zip(rows, blocks):
        vs, vc = rng_p.choice(BLOCK, size=2, replace=False) + blk * BLOCK
        codes[vc] = codes[vs]
        mag = (codes[vs] & 0x7F).astype(np.int64)
        mag[~mask] = -1
        nudge = np.argsort(-mag, kind="stable")[:2]
        for k in nudge:
            c = int(codes[vc, k])
            if c & 0x7F:
                codes[vc, k] = np.uint8((c & 0x80) | ((c & 0x7F) - 1))
        _align_row(h, r, m, codes[vs])
        planted.append((int(m), int(vs), int(vc)))
    return planted


_WEIGHT_CACHE: dict = {}


def clear_cache():
    _WEIGHT_CACHE.clear()


def _weights_for(w: Workload):
    key = (w.H, w.v_full, w.V // BLOCK)
    full = (w.H, w.v_full, w.v_full // BLOCK)
    if key in _WEIGHT_CACHE:
        return _WEIGHT_CACHE[key]
    if full in _WEIGHT_CACHE:
        c, s = _WEIGHT_CACHE[full]
        return c[: w.V], s[: w.V // BLOCK]
    c, s = weight_family(w.H, w.v_full, w.V // BLOCK)
    _WEIGHT_CACHE[key] = (c, s)
    return c, s


def make(name_or_id):
    """Draw one workload.

    Returns dict with numpy arrays
      hidden, residual: uint16 [M, H] bf16 bit patterns
      norm_weight: float32 [H]; eps: float
      w_codes: uint8 [V, H]; w_scales: float32 [V/128, H/128]
    and meta: outlier channels; planted exact ties as (row, expected lower
    index, higher twin); planted near-tie rows as (row, best, runner-up).
    The weight arrays of the 6144-hidden family are cached and shared: treat
    them as read-only.
    """
    w = get(name_or_id)
    if w.name == "tiny":
        w, h, r, g, codes, scales, meta = _tiny()
    else:
        h, r, g, outl = _activations(w)
        codes, scales = _weights_for(w)
        meta = dict(outliers=outl, ties=[], near_tie_rows=[])
        if w.name == "mtp5_batch":
            codes = codes.copy()
            meta["near_tie_rows"] = _mtp5_near_ties(w, h, r, codes, outl)
    return dict(
        workload=w,
        hidden=to_bf16_bits(h),
        residual=to_bf16_bits(r),
        norm_weight=g,
        eps=EPS,
        w_codes=codes,
        w_scales=scales,
        meta=meta,
    )


def partials(name_or_id, P: int) -> np.ndarray:
    """P row-parallel partial outputs for a workload: uint16 [P, M, H] bf16 bits.

    Partial p is drawn from its own stream (spawn_key (workload_id, 10, P, p)).
    """
    w = get(name_or_id)
    _, _, _, outl = _activations(w) if w.outliers else (None, None, None, np.zeros((0,), np.int64))
    return _partials(lambda p: _rng(w.wid, 10, P, p), P, w.M, w.H, outl)


def random_partials(seed: int, P: int, M: int, H: int, outliers: bool = False) -> np.ndarray:
    """P partials of arbitrary shape for edge-case tests: uint16 [P, M, H]."""
    outl = np.zeros((0,), np.int64)
    if outliers and H >= 100:
        outl = _rng(201, seed, M, H).choice(H, size=max(1, H // 100), replace=False)
    return _partials(lambda p: _rng(202, seed, P, M, H, p), P, M, H, outl)


def _partials(rng_for, P, M, H, outl):
    out = np.empty((P, M, H), np.uint16)
    sd = np.float32(1.0 / np.sqrt(P))
    for p in range(P):
        x = rng_for(p).standard_normal((M, H), dtype=np.float32) * sd
        if len(outl):
            x[:, outl] *= np.float32(20.0)
        out[p] = to_bf16_bits(x)
    return out


def random_case(seed: int, M: int, H: int, V: int, outliers: bool = False, zero_rows=()):
    """A small seeded case of arbitrary shape for edge-case tests."""
    rng = _rng(200, seed, M, H, V)
    h = rng.standard_normal((M, H), dtype=np.float32)
    r = rng.standard_normal((M, H), dtype=np.float32)
    if outliers and H >= 100:
        outl = rng.choice(H, size=max(1, H // 100), replace=False)
        h[:, outl] *= 20
        r[:, outl] *= 20
    for m in zero_rows:
        h[m] = 0
        r[m] = 0
    g = rng.uniform(0.5, 1.5, size=H).astype(np.float32)
    wf = rng.standard_normal((V, H), dtype=np.float32) * np.float32(0.02)
    codes, scales = _pack_e4m3_blocks(wf) if V else (np.zeros((0, H), np.uint8), np.zeros((0, H // BLOCK), np.float32))
    return dict(hidden=to_bf16_bits(h), residual=to_bf16_bits(r), norm_weight=g, eps=EPS,
                w_codes=codes, w_scales=scales)
