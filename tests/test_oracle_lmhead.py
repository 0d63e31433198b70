"""Pins for the oracle's block-scaled FP8 LM head and greedy local argmax.

- logits against a float64 matmul of operands dequantized with torch's
  e4m3fn decode (a library routine, not the oracle's loop);
- exact rational brute force on a tiny case;
- one-hot activations, where every logit is one scaled weight element;
- argmax against numpy.argmax (first occurrence) on fp32 logits;
- planted exact ties, whose expected lower index is known by construction;
- the vocab-parallel view: per-shard local argmaxes combined by
  (max desc, global index asc) equal the full-vocab argmax ("[Spec
  Decode][Perf] Fuse the MTP trailing all-reduce; local-argmax draft
  tokens", Summary; the lowest global index resolves ties across shard
  boundaries).
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from mtp_draft_head_amd import inputs


def dec_torch(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def dequant(codes, scales, rows_per_scale):
    """codes [R, H], scales [R/rows_per_scale, H/128] -> fp64 [R, H]."""
    R, H = codes.shape
    s = np.repeat(np.repeat(scales.astype(np.float64), rows_per_scale, axis=0), 128, axis=1)
    return dec_torch(codes) * s


def small_case(seed, M, H, V):
    d = inputs.random_case(seed, M, H, V, outliers=True)
    nq = oracle.norm_quant(d["hidden"], d["residual"], d["norm_weight"], d["eps"])
    return nq["codes"], nq["scales"], d["w_codes"], d["w_scales"]


@pytest.mark.parametrize("M,H,V", [(3, 256, 384), (17, 640, 1152), (5, 128, 128)])
def test_logits_vs_float64_matmul(M, H, V):
    a, sa, w, sw = small_case(M * 1000 + H, M, H, V)
    z = oracle.logits(a, sa, w, sw)
    A = dequant(a, sa, 1)
    W = dequant(w, sw, 128)
    ref = A @ W.T
    mag = np.abs(A) @ np.abs(W).T
    assert np.all(np.abs(z - ref) <= 1e-13 * mag + 1e-300)


def test_logits_exact_rational_bruteforce():
    a, sa, w, sw = small_case(11, 2, 256, 256)
    z = oracle.logits(a, sa, w, sw)
    dec = {c: Fraction(float(v)) for c, v in enumerate(dec_torch(np.arange(256, dtype=np.uint8)))
           if np.isfinite(v)}
    for i in range(2):
        for v in range(0, 256, 37):
            exact = sum(
                Fraction(float(sa[i, b])) * Fraction(float(sw[v // 128, b])) *
                sum(dec[int(a[i, k])] * dec[int(w[v, k])] for k in range(b * 128, (b + 1) * 128))
                for b in range(2))
            assert abs(Fraction(z[i, v]) - exact) <= abs(exact) * Fraction(1, 2 ** 50)


def test_one_hot_activation_selects_one_scaled_weight_column():
    rng = np.random.default_rng(3)
    H, V = 512, 768                   # 4 K-blocks, 6 vocab blocks: a transposed scale index would show
    w = rng.integers(0, 256, size=(V, H), dtype=np.uint8)
    w[(w & 0x7F) == 0x7F] = 0x10      # no NaN codes
    sw = rng.uniform(1e-4, 1e-3, size=(V // 128, H // 128)).astype(np.float32)
    for k, code in [(0, 0x38), (200, 0xC0), (511, 0x05), (300, 0x7E)]:
        a = np.zeros((1, H), np.uint8)
        a[0, k] = code
        sa = rng.uniform(0.01, 0.1, size=(1, H // 128)).astype(np.float32)
        z = oracle.logits(a, sa, w, sw)[0]
        expect = (np.float64(sa[0, k // 128]) * sw[np.arange(V) // 128, k // 128].astype(np.float64)
                  * dec_torch(np.array([code], np.uint8))[0] * dec_torch(w[:, k]))
        assert np.array_equal(z, expect)


def test_argmax_matches_numpy_first_occurrence():
    a, sa, w, sw = small_case(21, 9, 384, 1280)
    r = oracle.argmax(a, sa, w, sw)
    z = oracle.logits(a, sa, w, sw)
    zf = z.astype(np.float32)
    assert np.array_equal(r["idx"], np.argmax(zf, axis=1))
    assert np.array_equal(r["max"], zf.max(axis=1))
    assert np.array_equal(r["z1"], z[np.arange(9), r["idx"]])
    zz = z.copy()
    zz[np.arange(9), r["idx"]] = -np.inf
    assert np.array_equal(r["z2"], zz.max(axis=1))


def test_argmax_row_subset_and_repeats():
    a, sa, w, sw = small_case(22, 6, 256, 512)
    full = oracle.argmax(a, sa, w, sw)
    rows = np.array([5, 0, 0, 3], np.int32)
    sub = oracle.argmax(a, sa, w, sw, rows=rows)
    assert np.array_equal(sub["idx"], full["idx"][rows])
    assert np.array_equal(sub["max"], full["max"][rows])


def test_zero_activation_row_argmax_is_index_zero():
    a, sa, w, sw = small_case(23, 3, 256, 512)
    a[1] = 0
    sa[1] = 0
    r = oracle.argmax(a, sa, w, sw)
    assert r["idx"][1] == 0 and r["max"][1] == 0.0


def test_planted_exact_ties_pick_lowest_index(workloads):
    d = workloads("tiny")
    nq = oracle.norm_quant(d["hidden"], d["residual"], d["norm_weight"], d["eps"])
    r = oracle.argmax(nq["codes"], nq["scales"], d["w_codes"], d["w_scales"])
    for row, lo, hi in d["meta"]["ties"]:
        assert r["idx"][row] == lo
        assert r["z1"][row] == r["z2"][row]          # an exact tie with the higher twin
        z = oracle.logits(nq["codes"], nq["scales"], d["w_codes"], d["w_scales"], rows=[row])[0]
        assert z[lo] == z[hi] == z.max()


@pytest.mark.parametrize("shard", [128, 256, 512])
def test_sharded_argmax_equals_full_vocab(shard, workloads):
    d = workloads("tiny")
    nq = oracle.norm_quant(d["hidden"], d["residual"], d["norm_weight"], d["eps"])
    full = oracle.argmax(nq["codes"], nq["scales"], d["w_codes"], d["w_scales"])
    m, i = oracle.argmax_sharded(nq["codes"], nq["scales"], d["w_codes"], d["w_scales"], shard)
    assert np.array_equal(i, full["idx"]) and np.array_equal(m, full["max"])


def test_combine_shards_prefers_lower_global_index_on_equal_max():
    m, i = oracle.combine_shards(np.array([[2.0, 1.0, -0.0], [2.0, 3.0, 0.0]], np.float32),
                                 np.array([[5, 1, 7], [0, 2, 3]]), [0, 128])
    assert list(i) == [5, 130, 7] and list(m) == [2.0, 3.0, 0.0]


@pytest.mark.slow
def test_mtp5_near_tie_rows_are_planted(workloads):
    d = workloads("mtp5_batch")
    nq = oracle.norm_quant(d["hidden"], d["residual"], d["norm_weight"], d["eps"])
    planted = d["meta"]["near_tie_rows"]
    rows = [p[0] for p in planted]
    r = oracle.argmax(nq["codes"], nq["scales"], d["w_codes"], d["w_scales"], rows=rows)
    gap = (r["z1"] - r["z2"]) / np.abs(r["z1"])
    assert len(rows) == 16
    assert np.all(gap > 1e-6) and np.all(gap < 1e-3)
    assert [int(x) for x in r["idx"]] == [p[1] for p in planted]


# --------------------------------------------------------------------------
# top-k ("feat(glm52): add checkpoint-native MTP speculative decoding",
# Accuracy: the top-8 and top-32 sets of draft and reference are compared)
# --------------------------------------------------------------------------

def test_topk_of_one_is_the_argmax():
    a, sa, w, sw = small_case(41, 6, 384, 640)
    v, i = oracle.topk(a, sa, w, sw, 1)
    ref = oracle.argmax(a, sa, w, sw)
    assert np.array_equal(i[:, 0], ref["idx"]) and np.array_equal(v[:, 0], ref["max"])


@pytest.mark.parametrize("k", [2, 8, 32])
def test_topk_matches_a_stable_sort_of_fp32_logits(k):
    """Against numpy's stable sort of the fp32 logits by descending value (a
    library ordering of the oracle's own logits, which are pinned above)."""
    a, sa, w, sw = small_case(42 + k, 5, 512, 1024)
    v, i = oracle.topk(a, sa, w, sw, k)
    z32 = oracle.logits(a, sa, w, sw).astype(np.float32)
    for r in range(5):
        order = np.argsort(-z32[r].astype(np.float64), kind="stable")[:k]
        assert np.array_equal(i[r], order)
        assert np.array_equal(v[r], z32[r][order])
        assert np.all(np.diff(v[r].astype(np.float64)) <= 0)


def test_topk_brute_force_on_python_tuples():
    """Pure-Python sort of (-value, index) pairs on a tiny case."""
    a, sa, w, sw = small_case(47, 2, 256, 256)
    z32 = oracle.logits(a, sa, w, sw).astype(np.float32)
    v, i = oracle.topk(a, sa, w, sw, 8)
    for r in range(2):
        pairs = sorted((-float(z32[r, c]), c) for c in range(256))[:8]
        assert [c for _, c in pairs] == list(i[r])


def test_topk_planted_ties_come_in_index_order():
    d = inputs.make("tiny")
    nq = oracle.norm_quant(d["hidden"], d["residual"], d["norm_weight"], d["eps"])
    v, i = oracle.topk(nq["codes"], nq["scales"], d["w_codes"], d["w_scales"], 4)
    for row, lo, hi in d["meta"]["ties"]:
        assert i[row, 0] == lo and i[row, 1] == hi and v[row, 0] == v[row, 1]


def test_topk_of_a_zero_row_is_the_lowest_indices():
    """A zero activation row makes every logit 0: the top-k are indices 0..k-1."""
    a, sa, w, sw = small_case(48, 3, 256, 384)
    a = a.copy(); sa = sa.copy()
    a[1] = 0; sa[1] = 0
    v, i = oracle.topk(a, sa, w, sw, 8)
    assert list(i[1]) == list(range(8)) and np.all(v[1] == 0)


# --------------------------------------------------------------------------
# vocab-shard combine of top-k lists
# --------------------------------------------------------------------------

@pytest.mark.parametrize("k,shard", [(1, 128), (8, 128), (8, 256), (32, 256)])
def test_combined_shard_topk_equals_full_vocab_topk(k, shard):
    """The k largest of the union of per-shard top-k lists are the k largest
    overall: shards of the oracle's own top-k, combined, equal its full-vocab
    top-k (values and indices)."""
    a, sa, w, sw = small_case(60 + k + shard, 4, 384, 1024)
    full_v, full_i = oracle.topk(a, sa, w, sw, k)
    vals, idxs, offs = [], [], []
    for o in range(0, 1024, shard):
        v, i = oracle.topk(a, sa, w[o:o + shard], sw[o // 128:(o + shard) // 128], k)
        vals.append(v)
        idxs.append(i)
        offs.append(o)
    cv, ci = oracle.combine_topk_shards(np.stack(vals), np.stack(idxs), offs, k)
    assert np.array_equal(ci, full_i) and np.array_equal(cv, full_v)


def test_combined_topk_of_one_is_the_argmax_combine():
    rng = np.random.default_rng(3)
    lv = rng.integers(-4, 4, (5, 7, 1)).astype(np.float32)
    li = rng.integers(0, 128, (5, 7, 1))
    offs = [0, 128, 256, 384, 512]
    cv, ci = oracle.combine_topk_shards(lv, li, offs, 1)
    m, i = oracle.combine_shards(lv[:, :, 0], li[:, :, 0], offs)
    assert np.array_equal(ci[:, 0], i) and np.array_equal(cv[:, 0], m)


def test_combined_topk_cross_shard_ties_and_signed_zeros():
    """Hand-built lists: equal values in different shards come out by global
    index; -0 and +0 are one value (returned as +0)."""
    lv = np.array([[[3.0, 1.0, -0.0]], [[3.0, 0.0, -2.0]]], np.float32)
    li = np.array([[[9, 4, 2]], [[1, 0, 5]]])
    cv, ci = oracle.combine_topk_shards(lv, li, [0, 100], 5)
    assert list(ci[0]) == [9, 101, 4, 2, 100]
    assert list(cv[0]) == [3.0, 3.0, 1.0, 0.0, 0.0] and not np.signbit(cv[0, 3])
