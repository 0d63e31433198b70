"""GPU parity of the LM head's top-k (k <= 32) against the oracle's top-k on
the same packed activation: the k largest fp32 logits per row, descending,
lowest index first among equal values ("feat(glm52): add checkpoint-native
MTP speculative decoding", Accuracy compares top-8 and top-32 sets).
"""
import numpy as np
import pytest
import torch

import oracle
import mtp_draft_head_amd as mtpd
from mtp_draft_head_amd import inputs
from tests import parity
from tests.test_gpu_parity import DEV, host, say, to_dev

pytestmark = pytest.mark.gpu


def _packed(d):
    h, r, g, wc, ws = to_dev(d)
    _, codes, scales = mtpd.norm_quant(h, r, g, d["eps"])
    return codes, scales, wc, ws


def _check(codes, scales, d, k, gv, gi, rows=None):
    c, s = host(codes), host(scales)
    ov, oi = oracle.topk(c, s, d["w_codes"], d["w_scales"], k, rows=rows)
    rr = rows if rows is not None else np.arange(ov.shape[0])
    return parity.check_topk(host(gv), host(gi), ov, oi,
                             logit_row=lambda i: oracle.logits(c, s, d["w_codes"], d["w_scales"],
                                                               rows=[int(rr[i])])[0])


# (M, H, V, k): one and several 64-row passes, both row-tile counts, ragged K,
# the largest k, k = 1
SHAPES = [(1, 1152, 2048, 8), (5, 640, 1152, 32), (16, 2048, 4096, 1), (17, 1024, 4096, 32), (33, 384, 2048, 8),
          (64, 1152, 4096, 16), (130, 256, 1024, 32), (3, 8192, 256, 4)]


@pytest.mark.parametrize("M,H,V,k", SHAPES)
def test_topk_small_shapes(M, H, V, k):
    say(f"topk M={M} H={H} V={V} k={k}")
    d = inputs.random_case(70 + M + k, M, H, V, outliers=True)
    codes, scales, wc, ws = _packed(d)
    gv, gi = mtpd.fp8_lmhead_topk(codes, scales, wc, ws, k)
    say(f"  {_check(codes, scales, d, k, gv, gi)}")


def test_topk_of_one_is_the_argmax():
    d = inputs.random_case(81, 40, 1536, 4096, outliers=True)
    codes, scales, wc, ws = _packed(d)
    gv, gi = mtpd.fp8_lmhead_topk(codes, scales, wc, ws, 1)
    m, i = mtpd.fp8_lmhead_argmax(codes, scales, wc, ws)
    # the same keys and rule; K-summation orders differ between the kernels, so
    # compare indices outside near-ties via the oracle and values to rounding
    c, s = host(codes), host(scales)
    ref = oracle.argmax(c, s, d["w_codes"], d["w_scales"])
    gap = (ref["z1"] - ref["z2"]) / np.abs(ref["z1"])
    clear = gap > 1e-5
    assert np.array_equal(host(gi)[clear, 0], host(i)[clear])
    assert np.allclose(host(gv)[:, 0], host(m), rtol=1e-5, atol=0)


def test_topk_row_index_and_planted_ties():
    d = inputs.make("tiny")
    codes, scales, wc, ws = _packed(d)
    idx = torch.tensor([1, 0, 3, 1], dtype=torch.int32, device=DEV)
    gv, gi = mtpd.fp8_lmhead_topk(codes, scales, wc, ws, 4, row_index=idx)
    _check(codes, scales, d, 4, gv, gi, rows=host(idx))
    full_v, full_i = mtpd.fp8_lmhead_topk(codes, scales, wc, ws, 4)
    assert torch.equal(gi, full_i[idx.long()]) and torch.equal(gv, full_v[idx.long()])
    hi = host(full_i)
    for row, lo, hi_idx in d["meta"]["ties"]:
        assert hi[row, 0] == lo and hi[row, 1] == hi_idx, (row, hi[row])


def test_topk_empty():
    d = inputs.random_case(82, 2, 256, 256)
    codes, scales, wc, ws = _packed(d)
    gv, gi = mtpd.fp8_lmhead_topk(codes[:0], scales[:0], wc, ws, 8)
    assert gv.shape == (0, 8)


@pytest.mark.parametrize("name,k", [("decode_c1_tp8_shard", 8), ("decode_c1_tp8_shard", 32), ("decode_c64_full", 8),
                                    ("decode_c64_full", 32)])
def test_topk_full_size(name, k, workloads):
    d = workloads(name)
    codes, scales, wc, ws = _packed(d)
    gv, gi = mtpd.fp8_lmhead_topk(codes, scales, wc, ws, k)
    say(f"topk {name} k={k}: {_check(codes, scales, d, k, gv, gi)}")


# (M, H, V, shards, k): vocab shards of 256, 512, 1024 and 128 rows, k from 1
# to 32, one and several rows per workgroup
COMBINE = [(5, 640, 2048, 8, 8), (64, 1152, 4096, 8, 32), (17, 384, 1024, 4, 1), (3, 256, 8192, 64, 4),
           (9, 512, 1024, 1, 16)]


@pytest.mark.parametrize("M,H,V,S,k", COMBINE)
def test_topk_vocab_shards_combine(M, H, V, S, k):
    """Per-shard top-k lists (one top-k launch per vocab shard) combined on
    the device: bit for bit the oracle's combine of the same lists, and the
    oracle's full-vocab top-k outside near ties."""
    say(f"topk combine M={M} H={H} V={V} shards={S} k={k}")
    d = inputs.random_case(90 + M + S, M, H, V, outliers=True)
    codes, scales, wc, ws = _packed(d)
    R = V // S
    vals, idxs = [], []
    for s in range(S):
        v, i = mtpd.fp8_lmhead_topk(codes, scales, wc[s * R:(s + 1) * R], ws[s * R // 128:(s + 1) * R // 128], k)
        vals.append(v)
        idxs.append(i)
    lv, li = torch.stack(vals), torch.stack(idxs)
    offs = [s * R for s in range(S)]
    gv, gi = mtpd.topk_combine(lv, li, offs)
    torch.cuda.synchronize()
    ev, ei = oracle.combine_topk_shards(host(lv), host(li), offs, k)
    assert np.array_equal(host(gi), ei.astype(np.int32))
    assert np.array_equal(host(gv), ev) and not np.any(np.signbit(host(gv)) & (host(gv) == 0))
    say(f"  against the full-vocab oracle: {_check(codes, scales, d, k, gv, gi)}")


def test_topk_combine_empty_and_planted_ties():
    """No rows launches nothing; the tiny workload's planted exact ties, split
    across two shards, still come out lowest global index first."""
    e = torch.empty((2, 0, 4), dtype=torch.float32, device=DEV)
    gv, gi = mtpd.topk_combine(e, e.to(torch.int32), [0, 512])
    assert gv.shape == (0, 4) and gi.shape == (0, 4)
    d = inputs.make("tiny")
    codes, scales, wc, ws = _packed(d)
    V = wc.shape[0]
    parts = [mtpd.fp8_lmhead_topk(codes, scales, wc[o:o + V // 2], ws[o // 128:(o + V // 2) // 128], 4)
             for o in (0, V // 2)]
    gv, gi = mtpd.topk_combine(torch.stack([p[0] for p in parts]), torch.stack([p[1] for p in parts]), [0, V // 2])
    full_v, full_i = mtpd.fp8_lmhead_topk(codes, scales, wc, ws, 4)
    assert torch.equal(gi, full_i) and torch.equal(gv, full_v)
    hi = host(gi)
    for row, lo, hi_idx in d["meta"]["ties"]:
        assert hi[row, 0] == lo and hi[row, 1] == hi_idx, (row, hi[row])


@pytest.mark.parametrize("k", [8, 32])
def test_topk_vocab_shards_full_size(k, workloads):
    """The c=64 full-vocab head as eight 18944-row shards (one GPU's TP8 share
    each), their top-k lists combined on the device: the oracle's combine of
    the same lists bit for bit, and the full-vocab top-k outside near ties."""
    d = workloads("decode_c64_full")
    codes, scales, wc, ws = _packed(d)
    S, R = 8, 18944
    parts = [mtpd.fp8_lmhead_topk(codes, scales, wc[s * R:(s + 1) * R], ws[s * R // 128:(s + 1) * R // 128], k)
             for s in range(S)]
    lv, li = torch.stack([p[0] for p in parts]), torch.stack([p[1] for p in parts])
    offs = [s * R for s in range(S)]
    gv, gi = mtpd.topk_combine(lv, li, offs)
    torch.cuda.synchronize()
    ev, ei = oracle.combine_topk_shards(host(lv), host(li), offs, k)
    assert np.array_equal(host(gi), ei.astype(np.int32)) and np.array_equal(host(gv), ev)
    say(f"topk shards c64 k={k} against the full-vocab oracle: {_check(codes, scales, d, k, gv, gi)}")
