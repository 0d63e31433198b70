"""CPU oracle for the MTP draft-layer tail -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg import this package.  The HIP library and its binding never do, and the
two share no code.  The arithmetic lives in ``mtpd_oracle.c`` (plain C, fp64,
one plain loop per step); this module marshals numpy arrays into it and adds
the sharded argmax combine, which is plain Python over the C results.

Function map (method steps as described on the pages):
  norm_quant      residual add, RMSNorm, bf16 recycled hidden + packed FP8
                  ("[Quant][MTP] Reuse packed FP8 logits inputs", Purpose)
  allreduce_norm_quant
                  the same step with the MTP layer's trailing all-reduce in
                  front: norm input = sum of P partials + residual ("[Spec
                  Decode][Perf] Fuse the MTP trailing all-reduce; local-argmax
                  draft tokens", Summary)
  block_quant     the packing step alone (amax/448 scale per 128 columns)
  logits          block-scaled FP8 LM head on the packed activation
                  (same page, Purpose and Dependencies)
  argmax          greedy local argmax, lowest index on equal maxima
                  ("[Spec Decode][Perf] Fuse the MTP trailing all-reduce;
                  local-argmax draft tokens", Summary)
  topk            the k largest fp32 logits per row, descending, lowest index
                  first among equal values ("feat(glm52): add checkpoint-native
                  MTP speculative decoding", Accuracy: top-8 / top-32 overlap)
  argmax_sharded  the vocab-parallel view: per-shard local argmaxes combined
                  by (max desc, global index asc) (same page, Summary and
                  Accuracy)
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

BLOCK = 128

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = _build.library_path()
    if not os.path.exists(path):
        _build.build()
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.ora_e4m3_decode.restype = ctypes.c_double
    lib.ora_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.ora_e4m3_encode.restype = ctypes.c_uint8
    lib.ora_e4m3_encode.argtypes = [ctypes.c_double]
    lib.ora_bf16_decode.restype = ctypes.c_double
    lib.ora_bf16_decode.argtypes = [ctypes.c_uint16]
    lib.ora_bf16_encode.restype = ctypes.c_uint16
    lib.ora_bf16_encode.argtypes = [ctypes.c_double]
    lib.ora_e4m3_encode_array.restype = None
    lib.ora_e4m3_encode_array.argtypes = [P, I64, P]
    lib.ora_bf16_encode_array.restype = None
    lib.ora_bf16_encode_array.argtypes = [P, I64, P]
    lib.ora_block_quant.restype = None
    lib.ora_block_quant.argtypes = [P, I64, I64, P, P]
    lib.ora_norm_quant.restype = None
    lib.ora_norm_quant.argtypes = [P, P, P, ctypes.c_float, I64, I64, P, P, P, P, P]
    lib.ora_allreduce_norm_quant.restype = None
    lib.ora_allreduce_norm_quant.argtypes = [P, I64, P, P, ctypes.c_float, I64, I64, P, P, P, P, P]
    lib.ora_logits.restype = None
    lib.ora_logits.argtypes = [P, P, I64, P, I64, P, P, I64, P]
    lib.ora_argmax.restype = None
    lib.ora_argmax.argtypes = [P, P, I64, P, I64, P, P, I64, P, P, P, P]
    lib.ora_topk.restype = None
    lib.ora_topk.argtypes = [P, P, I64, P, I64, P, P, I64, I64, P, P]
    lib.ora_num_threads.restype = ctypes.c_int
    lib.ora_num_threads.argtypes = []
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


def num_threads() -> int:
    """Threads the oracle's OpenMP loops use."""
    return int(_load().ora_num_threads())


# --------------------------------------------------------------------------
# codecs (scalar, from the format definitions; see mtpd_oracle.c)
# --------------------------------------------------------------------------

def e4m3_decode(codes) -> np.ndarray:
    lib = _load()
    c = np.asarray(codes, dtype=np.uint8)
    return np.array([lib.ora_e4m3_decode(int(x)) for x in c.ravel()], dtype=np.float64).reshape(c.shape)


def e4m3_encode(values) -> np.ndarray:
    lib = _load()
    v = np.ascontiguousarray(values, dtype=np.float64)
    out = np.empty(v.shape, np.uint8)
    lib.ora_e4m3_encode_array(_ptr(v), v.size, _ptr(out))
    return out


def bf16_decode(bits) -> np.ndarray:
    lib = _load()
    b = np.asarray(bits, dtype=np.uint16)
    return np.array([lib.ora_bf16_decode(int(x)) for x in b.ravel()], dtype=np.float64).reshape(b.shape)


def bf16_encode(values) -> np.ndarray:
    lib = _load()
    v = np.ascontiguousarray(values, dtype=np.float64)
    out = np.empty(v.shape, np.uint16)
    lib.ora_bf16_encode_array(_ptr(v), v.size, _ptr(out))
    return out


# --------------------------------------------------------------------------
# the path
# --------------------------------------------------------------------------

def norm_quant(hidden, residual, norm_weight, eps: float):
    """Residual add + RMSNorm + (bf16 recycled hidden, E4M3 codes, fp32 scales).

    hidden, residual: uint16 [M, H] (bf16 bit patterns); norm_weight float32 [H].
    Returns dict(hidden=uint16 [M,H], codes=uint8 [M,H], scales=float32 [M,H/128],
    y=float64 [M,H], rstd=float64 [M]).
    """
    lib = _load()
    h = _c(hidden, np.uint16)
    r = _c(residual, np.uint16)
    g = _c(norm_weight, np.float32)
    M, H = h.shape
    if r.shape != (M, H) or g.shape != (H,) or H % BLOCK:
        raise ValueError("shape mismatch")
    out_h = np.empty((M, H), np.uint16)
    codes = np.empty((M, H), np.uint8)
    scales = np.empty((M, H // BLOCK), np.float32)
    y = np.empty((M, H), np.float64)
    rstd = np.empty((M,), np.float64)
    lib.ora_norm_quant(_ptr(h), _ptr(r), _ptr(g), ctypes.c_float(eps), M, H,
                       _ptr(out_h), _ptr(codes), _ptr(scales), _ptr(y), _ptr(rstd))
    return dict(hidden=out_h, codes=codes, scales=scales, y=y, rstd=rstd)


def allreduce_norm_quant(partials, residual, norm_weight, eps: float):
    """norm_quant with norm input sum(partials) + residual, summed in fp64.

    partials: uint16 [P, M, H] bf16 bit patterns; residual uint16 [M, H];
    norm_weight float32 [H].  Returns norm_quant's dict.
    """
    lib = _load()
    pp = _c(partials, np.uint16)
    r = _c(residual, np.uint16)
    g = _c(norm_weight, np.float32)
    if pp.ndim != 3 or pp.shape[0] < 1:
        raise ValueError("partials must be [P, M, H] with P >= 1")
    P, M, H = pp.shape
    if r.shape != (M, H) or g.shape != (H,) or H % BLOCK:
        raise ValueError("shape mismatch")
    out_h = np.empty((M, H), np.uint16)
    codes = np.empty((M, H), np.uint8)
    scales = np.empty((M, H // BLOCK), np.float32)
    y = np.empty((M, H), np.float64)
    rstd = np.empty((M,), np.float64)
    lib.ora_allreduce_norm_quant(_ptr(pp), P, _ptr(r), _ptr(g), ctypes.c_float(eps), M, H,
                                 _ptr(out_h), _ptr(codes), _ptr(scales), _ptr(y), _ptr(rstd))
    return dict(hidden=out_h, codes=codes, scales=scales, y=y, rstd=rstd)


def block_quant(y):
    """Packed FP8 activation of fp64 rows y [M, H]: (codes uint8 [M,H], scales float32 [M,H/128])."""
    lib = _load()
    yy = _c(y, np.float64)
    M, H = yy.shape
    if H % BLOCK:
        raise ValueError("H must be a multiple of 128")
    codes = np.empty((M, H), np.uint8)
    scales = np.empty((M, H // BLOCK), np.float32)
    lib.ora_block_quant(_ptr(yy), M, H, _ptr(codes), _ptr(scales))
    return codes, scales


def _rows_arg(rows, n_act):
    if rows is None:
        return None, n_act
    rr = np.ascontiguousarray(rows, dtype=np.int32)
    if rr.size and (rr.min() < 0 or rr.max() >= n_act):
        raise IndexError("row index out of range")
    return rr, rr.size


def _check_lmhead(codes, scales, w_codes, w_scales):
    a = _c(codes, np.uint8)
    sa = _c(scales, np.float32)
    wq = _c(w_codes, np.uint8)
    ws = _c(w_scales, np.float32)
    A, H = a.shape
    V = wq.shape[0]
    if (H % BLOCK or V % BLOCK or wq.shape != (V, H) or sa.shape != (A, H // BLOCK)
            or ws.shape != (V // BLOCK, H // BLOCK)):
        raise ValueError("shape mismatch")
    return a, sa, wq, ws, A, H, V


def logits(codes, scales, w_codes, w_scales, rows=None) -> np.ndarray:
    """fp64 logits [n_rows, V] of the block-scaled FP8 LM head."""
    lib = _load()
    a, sa, wq, ws, A, H, V = _check_lmhead(codes, scales, w_codes, w_scales)
    rr, n = _rows_arg(rows, A)
    z = np.empty((n, V), np.float64)
    lib.ora_logits(_ptr(a), _ptr(sa), H, _ptr(rr), n, _ptr(wq), _ptr(ws), V, _ptr(z))
    return z


def argmax(codes, scales, w_codes, w_scales, rows=None):
    """Greedy local argmax.  Returns dict(max=float32, idx=int32, z1=f64, z2=f64), each [n_rows]."""
    lib = _load()
    a, sa, wq, ws, A, H, V = _check_lmhead(codes, scales, w_codes, w_scales)
    rr, n = _rows_arg(rows, A)
    out_max = np.empty((n,), np.float32)
    out_idx = np.empty((n,), np.int32)
    z1 = np.empty((n,), np.float64)
    z2 = np.empty((n,), np.float64)
    if n:
        lib.ora_argmax(_ptr(a), _ptr(sa), H, _ptr(rr), n, _ptr(wq), _ptr(ws), V,
                       _ptr(out_max), _ptr(out_idx), _ptr(z1), _ptr(z2))
    return dict(max=out_max, idx=out_idx, z1=z1, z2=z2)


def topk(codes, scales, w_codes, w_scales, k: int, rows=None):
    """Top-k per row: (values float32 [n, k], indices int32 [n, k]), descending."""
    lib = _load()
    a, sa, wq, ws, A, H, V = _check_lmhead(codes, scales, w_codes, w_scales)
    rr, n = _rows_arg(rows, A)
    if not 1 <= k <= V:
        raise ValueError("k must lie in [1, V]")
    vals = np.empty((n, k), np.float32)
    idx = np.empty((n, k), np.int32)
    if n:
        lib.ora_topk(_ptr(a), _ptr(sa), H, _ptr(rr), n, _ptr(wq), _ptr(ws), V, int(k), _ptr(vals), _ptr(idx))
    return vals, idx


def combine_shards(local_max, local_idx, offsets):
    """Combine per-shard local (max, idx) pairs into the global draft token.

    local_max, local_idx: [n_shards, n_rows]; offsets: [n_shards] first global
    vocab row of each shard.  The winner is the largest max; among equal
    maxima (+0 == -0) the smallest global index.
    """
    local_max = np.asarray(local_max, np.float32)
    local_idx = np.asarray(local_idx, np.int64)
    n_shards, n_rows = local_max.shape
    out_max = np.empty((n_rows,), np.float32)
    out_idx = np.empty((n_rows,), np.int64)
    for i in range(n_rows):
        best_m, best_g = None, None
        for s in range(n_shards):
            m = float(local_max[s, i])
            g = int(offsets[s]) + int(local_idx[s, i])
            if best_m is None or m > best_m or (m == best_m and g < best_g):
                best_m, best_g = m, g
        out_max[i] = best_m
        out_idx[i] = best_g
    return out_max, out_idx


def combine_topk_shards(local_val, local_idx, offsets, k: int):
    """Combine per-shard local top-k lists into the global top-k.

    Under vocab parallelism each shard returns, per row, its own largest
    logits with local indices; the global top-k is taken from those lists
    rather than from gathered full-vocab logits ("[Spec Decode][Perf] Fuse
    the MTP trailing all-reduce; local-argmax draft tokens", Summary; the
    top-8 and top-32 sets are what "feat(glm52): add checkpoint-native MTP
    speculative decoding", Accuracy, compares).

    local_val, local_idx: [n_shards, n_rows, kk] (any order within a list);
    offsets: [n_shards] first global vocab row of each shard.  For each row:
    the k pairs of largest value over all shards' pairs, in descending
    value, equal values (+0 == -0) by ascending global index; -0 is returned
    as +0.  Returns (values float32 [n_rows, k], indices int64 [n_rows, k]).
    """
    local_val = np.asarray(local_val, np.float32)
    local_idx = np.asarray(local_idx, np.int64)
    n_shards, n_rows, kk = local_val.shape
    if not 1 <= k <= n_shards * kk:
        raise ValueError("k must lie in [1, n_shards * list length]")
    out_val = np.empty((n_rows, k), np.float32)
    out_idx = np.empty((n_rows, k), np.int64)
    for i in range(n_rows):
        pairs = []
        for s in range(n_shards):
            for j in range(kk):
                v = float(local_val[s, i, j]) + 0.0   # -0 and +0 compare and sort as one value
                pairs.append((-v, int(offsets[s]) + int(local_idx[s, i, j])))
        pairs.sort()
        for e in range(k):
            out_val[i, e] = -pairs[e][0] + 0.0
            out_idx[i, e] = pairs[e][1]
    return out_val, out_idx


def argmax_sharded(codes, scales, w_codes, w_scales, shard_rows, rows=None):
    """Argmax over a vocab split into shards of ``shard_rows`` vocab rows each.

    Every shard runs the local argmax on its own slice (local indices), then
    ``combine_shards`` reduces them.  Shard boundaries must fall on 128-row
    weight-scale blocks.
    """
    wq = _c(w_codes, np.uint8)
    ws = _c(w_scales, np.float32)
    V = wq.shape[0]
    if shard_rows % BLOCK or V % shard_rows:
        raise ValueError("shards must be whole 128-row blocks and tile V")
    maxes, idxs, offs = [], [], []
    for o in range(0, V, shard_rows):
        r = argmax(codes, scales, wq[o:o + shard_rows], ws[o // BLOCK:(o + shard_rows) // BLOCK], rows)
        maxes.append(r["max"])
        idxs.append(r["idx"])
        offs.append(o)
    return combine_shards(np.stack(maxes), np.stack(idxs), offs)
