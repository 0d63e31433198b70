"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Stagewise, as the tolerances require: norm_quant against the oracle's
residual add + RMSNorm + packing on the same inputs; then the LM head +
argmax against the oracle applied to the GPU's own packed activation (an
allowed one-code flip in the packing would otherwise be charged to the GEMM).
Full-size workloads run in the launch configuration the benchmark times;
the oracle covers every row where it finishes in seconds and a seeded sample
of rows (always including planted near-tie rows) elsewhere.
"""
import numpy as np
import pytest
import torch

import oracle
import mtp_draft_head_amd as mtpd
from mtp_draft_head_amd import inputs
from tests import parity

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)


def to_dev(d):
    h = torch.from_numpy(d["hidden"].view(np.int16)).to(DEV).view(torch.bfloat16)
    r = torch.from_numpy(d["residual"].view(np.int16)).to(DEV).view(torch.bfloat16)
    g = torch.from_numpy(d["norm_weight"]).to(DEV)
    wc = torch.from_numpy(d["w_codes"]).to(DEV)
    ws = torch.from_numpy(d["w_scales"]).to(DEV)
    return h, r, g, wc, ws


def host(t):
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def check_norm_quant(d, out_h, codes, scales, rows=None):
    hid, res = d["hidden"], d["residual"]
    if rows is not None:
        hid, res = hid[rows], res[rows]
    ref = oracle.norm_quant(hid, res, d["norm_weight"], d["eps"])
    gh, gc, gs = host(out_h), host(codes), host(scales)
    if rows is not None:
        gh, gc, gs = gh[rows], gc[rows], gs[rows]
    r1 = parity.check_bf16(gh, ref["hidden"])
    r2 = parity.check_codes(gc, ref["codes"])
    r3 = parity.check_scales(gs, ref["scales"])
    return r1, r2, r3


def check_self_consistent(codes, scales):
    """Every nonzero block holds a +-448 code and requantizing the exact
    dequantization reproduces codes and scales bit for bit."""
    c, s = host(codes), host(scales)
    M, H = c.shape
    mags = (c.reshape(M, H // 128, 128) & 0x7F).max(axis=2)
    assert np.all(mags[s > 0] == 0x7E)
    assert np.all(c.reshape(M, H // 128, 128)[s == 0] == 0)
    dq = (torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float64).numpy().reshape(M, H // 128, 128)
          * s.astype(np.float64)[:, :, None]).reshape(M, H)
    c2, s2 = oracle.block_quant(dq)
    assert np.array_equal(s2, s) and np.array_equal(c2, c)


def check_lmhead(codes, scales, d, gmax, gidx, rows=None):
    c, s = host(codes), host(scales)
    ref = oracle.argmax(c, s, d["w_codes"], d["w_scales"], rows=rows)
    gm, gi = host(gmax), host(gidx)
    if rows is not None:
        gm, gi = gm[rows], gi[rows]
    rr = rows if rows is not None else np.arange(len(gm))
    return parity.check_argmax(
        gm, gi, ref,
        logit_row=lambda i: oracle.logits(c, s, d["w_codes"], d["w_scales"], rows=[int(rr[i])])[0])


# --------------------------------------------------------------------------
# small and ragged shapes, edge cases
# --------------------------------------------------------------------------

SHAPES = [
    (1, 128, 128), (4, 256, 1024), (5, 384, 640), (17, 640, 1152), (33, 1024, 384),
    (64, 2048, 2048), (65, 768, 256), (130, 256, 512), (3, 16384, 256), (2, 6144, 2304), (1, 8320, 256),
]


@pytest.mark.parametrize("M,H,V", SHAPES)
def test_draft_tail_small_shapes(M, H, V):
    say(f"draft_tail M={M} H={H} V={V}")
    d = inputs.random_case(M * 7919 + H * 31 + V, M, H, V, outliers=True)
    h, r, g, wc, ws = to_dev(d)
    out = mtpd.draft_tail(h, r, g, d["eps"], wc, ws)
    check_norm_quant(d, *out[:3])
    check_self_consistent(out[1], out[2])
    check_lmhead(out[1], out[2], d, out[3], out[4])


def test_tiny_workload_planted_ties():
    d = inputs.make("tiny")
    h, r, g, wc, ws = to_dev(d)
    out_h, codes, scales, gmax, gidx = mtpd.draft_tail(h, r, g, d["eps"], wc, ws)
    check_norm_quant(d, out_h, codes, scales)
    check_lmhead(codes, scales, d, gmax, gidx)
    gi = host(gidx)
    for row, lo, hi in d["meta"]["ties"]:
        assert gi[row] == lo, (row, gi[row], lo, hi)


def test_zero_rows_and_zero_blocks():
    d = inputs.random_case(5, 6, 512, 256, zero_rows=(1, 4))
    h, r, g, wc, ws = to_dev(d)
    out_h, codes, scales, gmax, gidx = mtpd.draft_tail(h, r, g, d["eps"], wc, ws)
    c, s = host(codes), host(scales)
    assert np.all(c[[1, 4]] == 0) and np.all(s[[1, 4]] == 0) and np.all(host(out_h)[[1, 4]] == 0)
    gm, gi = host(gmax), host(gidx)
    assert gi[1] == 0 and gi[4] == 0 and gm[1] == 0 and gm[4] == 0
    check_lmhead(codes, scales, d, gmax, gidx)


def test_empty_batch_is_a_noop():
    d = inputs.random_case(6, 2, 256, 256)
    h, r, g, wc, ws = to_dev(d)
    out = mtpd.draft_tail(h[:0], r[:0], g, d["eps"], wc, ws)
    assert out[0].shape == (0, 256) and out[3].shape == (0,)
    m, i = mtpd.fp8_lmhead_argmax(out[1], out[2], wc, ws)
    assert m.shape == (0,)


def test_norm_quant_entry_point_matches_draft_tail():
    d = inputs.random_case(7, 9, 1024, 512, outliers=True)
    h, r, g, wc, ws = to_dev(d)
    a = mtpd.norm_quant(h, r, g, d["eps"])
    b = mtpd.draft_tail(h, r, g, d["eps"], wc, ws)
    for x, y in zip(a, b[:3]):
        assert torch.equal(x, y)
    m, i = mtpd.fp8_lmhead_argmax(a[1], a[2], wc, ws)
    assert torch.equal(m, b[3]) and torch.equal(i, b[4])


@pytest.mark.parametrize("M,H", [(1, 128), (3, 640), (9, 1024), (64, 6144), (67, 7168), (33, 8192), (320, 7168)])
def test_norm_quant_wavefront_per_row(M, H):
    """The wavefront-per-row norm_quant (a plan override, kept to measure the
    launch shape) meets the oracle to the same tolerances as the
    workgroup-per-row kernel, ragged row counts and an all-zero row included,
    and its packing is self-consistent."""
    d = inputs.random_case(41 + M, M, H, 256, outliers=True, zero_rows=(0,) if M > 2 else ())
    h, r, g, _, _ = to_dev(d)
    with mtpd.plan_override(norm_quant="wave"):
        assert mtpd.draft_tail_plan(max(M, 2), 256, H).startswith("norm_quant_wave_kernel")
        out_h, codes, scales = mtpd.norm_quant(h, r, g, d["eps"])
    torch.cuda.synchronize()
    r1, r2, r3 = check_norm_quant(d, out_h, codes, scales)
    say(f"  wave per row M={M} H={H}: bf16 {r1}  codes {r2}  scales {r3}")
    check_self_consistent(codes, scales)


@pytest.mark.parametrize("n_idx,cus", [(7, None), (24, None), (40, 8), (64, 8), (100, None)])
def test_row_index_gather(n_idx, cus):
    """Gathered rows (repeats included) give the same pairs as the ungathered
    call, through each kernel family: 7 rows (weight streaming), 24 (shared
    activation ring), 40 and 64 (K outermost, on a grid sized for 8 CUs so
    each workgroup takes several tiles), 100 (the LDS-tiled kernel)."""
    d = inputs.random_case(8 + n_idx, 20, 512, 4096, outliers=True)
    h, r, g, wc, ws = to_dev(d)
    _, codes, scales, gmax, gidx = mtpd.draft_tail(h, r, g, d["eps"], wc, ws)
    rng = np.random.default_rng(n_idx)
    sel = np.concatenate([[19, 0, 0, 7], rng.integers(0, 20, n_idx - 4)]).astype(np.int32)
    idx = torch.from_numpy(sel).to(DEV)
    with mtpd.plan_override(device_cus=cus):
        say(f"  plan: {mtpd.lmhead_plan(n_idx, 4096, 512)}")
        m, i = mtpd.fp8_lmhead_argmax(codes, scales, wc, ws, row_index=idx)
    torch.cuda.synchronize()
    assert torch.equal(m, gmax[idx.long()]) and torch.equal(i, gidx[idx.long()])


def test_poisoned_outputs_are_overwritten_and_workspace_left_zero():
    d = inputs.random_case(9, 37, 768, 640, outliers=True)
    h, r, g, wc, ws = to_dev(d)
    M, H = 37, 768
    out = (torch.full((M, H), -1, dtype=torch.int16, device=DEV).view(torch.bfloat16),
           torch.full((M, H), 0xFF, dtype=torch.uint8, device=DEV),
           torch.full((M, H // 128), float("nan"), dtype=torch.float32, device=DEV),
           torch.full((M,), float("nan"), dtype=torch.float32, device=DEV),
           torch.full((M,), -7, dtype=torch.int32, device=DEV))
    wsp = mtpd.Workspace(DEV)
    mtpd.draft_tail(h, r, g, d["eps"], wc, ws, workspace=wsp, out=out)
    check_norm_quant(d, *out[:3])
    check_lmhead(out[1], out[2], d, out[3], out[4])
    assert int(wsp.buf.count_nonzero().item()) == 0


def test_two_streams_in_flight_use_separate_workspaces():
    """Calls in flight together on two streams (no synchronization between
    them) give the results of separate runs: the default workspaces are kept
    per stream.  An explicit Workspace refuses a second stream."""
    ds = [inputs.random_case(41 + k, 64, 2048, 8192, outliers=True) for k in range(2)]
    devs = [to_dev(d) for d in ds]
    refs = [mtpd.draft_tail(h, r, g, d["eps"], wc, ws) for d, (h, r, g, wc, ws) in zip(ds, devs)]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(DEV), torch.cuda.Stream(DEV)]
    for st in streams:
        st.wait_stream(torch.cuda.current_stream(DEV))
    outs = [[], []]
    for _ in range(3):
        for k in range(2):
            h, r, g, wc, ws = devs[k]
            with torch.cuda.stream(streams[k]):
                outs[k].append(mtpd.draft_tail(h, r, g, ds[k]["eps"], wc, ws))
    torch.cuda.synchronize()
    for k in range(2):
        for o in outs[k]:
            assert torch.equal(o[3], refs[k][3]) and torch.equal(o[4], refs[k][4]) and torch.equal(o[1], refs[k][1])
    wsp = mtpd.Workspace(DEV)
    h, r, g, wc, ws = devs[0]
    mtpd.fp8_lmhead_argmax(refs[0][1], refs[0][2], wc, ws, workspace=wsp)
    with torch.cuda.stream(streams[0]):
        with pytest.raises(ValueError):
            mtpd.fp8_lmhead_argmax(refs[0][1], refs[0][2], wc, ws, workspace=wsp)
    torch.cuda.synchronize()


def test_repeated_calls_are_bit_identical():
    d = inputs.random_case(10, 64, 2048, 4096, outliers=True)
    h, r, g, wc, ws = to_dev(d)
    a = mtpd.draft_tail(h, r, g, d["eps"], wc, ws)
    for _ in range(3):
        b = mtpd.draft_tail(h, r, g, d["eps"], wc, ws)
        for x, y in zip(a, b):
            assert torch.equal(x.view(torch.uint8) if x.dtype == torch.bfloat16 else x,
                               y.view(torch.uint8) if y.dtype == torch.bfloat16 else y)


@pytest.mark.parametrize("tile", ["2,1,4", "2,2,4", "2,4,4", "4,1,2", "4,2,2", "4,4,2"])
def test_every_launch_shape_agrees(tile):
    """Every column-tile / split-K launch shape meets the oracle and picks the
    same indices (split-K changes only the fp32 summation order)."""
    d = inputs.random_case(11, 24, 1536, 2048, outliers=True)
    h, r, g, wc, ws = to_dev(d)
    _, codes, scales, m0, i0 = mtpd.draft_tail(h, r, g, d["eps"], wc, ws)
    with mtpd.plan_override(lmhead_kernel="generic", lmhead_tile=tile):
        plan = mtpd.lmhead_plan(24, 2048, 1536)
        say(f"  plan: {plan}")
        assert plan.startswith("lmhead_argmax_kernel<2," + tile + ">")
        m1, i1 = mtpd.fp8_lmhead_argmax(codes, scales, wc, ws)
    torch.cuda.synchronize()
    check_lmhead(codes, scales, d, m1, i1)
    assert torch.equal(i0, i1)


@pytest.mark.parametrize("shape", ["1,8", "1,4", "1,12", "2,8", "2,4"])
@pytest.mark.parametrize("M", [1, 8, 9, 16])
def test_stream_kernel_shapes(M, shape):
    """Up to 16 rows: every weight-streaming launch shape (tiles per wave, ring
    depth; K = 9 blocks is not a multiple of any depth) meets the oracle and
    picks the generic kernel's indices."""
    d = inputs.random_case(13 + M, M, 1152, 2048, outliers=True)
    h, r, g, wc, ws = to_dev(d)
    with mtpd.plan_override(lmhead_kernel="generic"):
        _, codes, scales, m0, i0 = mtpd.draft_tail(h, r, g, d["eps"], wc, ws)
    with mtpd.plan_override(lmhead_stream=shape):
        say(f"  plan: {mtpd.lmhead_plan(M, 2048, 1152)}")
        assert mtpd.lmhead_plan(M, 2048, 1152).startswith("lmhead_stream_kernel")
        m1, i1 = mtpd.fp8_lmhead_argmax(codes, scales, wc, ws)
    torch.cuda.synchronize()
    check_lmhead(codes, scales, d, m1, i1)
    assert torch.equal(i0, i1)


@pytest.mark.parametrize("shape", ["2,4,3", "2,4,4", "2,4,5", "1,8,4", "1,4,3", "1,4,4", "1,4,6", "2,4,6"])
@pytest.mark.parametrize("M", [17, 32, 33, 64])
def test_stream_rows_kernel_shapes(M, shape):
    """17..64 rows: every compiled shape of the streaming kernel with a shared
    activation ring (tiles per wave, waves, ring depth; K = 9 blocks) meets the
    oracle and picks the decode kernel's indices.  (Shapes not compiled for
    the row count fall back to the default shape.)"""
    d = inputs.random_case(29 + M, M, 1152, 4096, outliers=True)
    h, r, g, wc, ws = to_dev(d)
    with mtpd.plan_override(lmhead_kernel="decode"):
        _, codes, scales, m0, i0 = mtpd.draft_tail(h, r, g, d["eps"], wc, ws)
    with mtpd.plan_override(lmhead_rows=shape, lmhead_kouter="0"):
        plan = mtpd.lmhead_plan(M, 4096, 1152)
        say(f"  plan: {plan}")
        assert plan.startswith("lmhead_stream_rows_kernel")
        m1, i1 = mtpd.fp8_lmhead_argmax(codes, scales, wc, ws)
    torch.cuda.synchronize()
    check_lmhead(codes, scales, d, m1, i1)
    assert torch.equal(i0, i1)


# (M, H, V, CUs): the persistent grid sized for `cus` CUs gives every
# workgroup 4 tiles (4096 / 128 on 8, 3584 / 128 on 7), 3 to 4 (on 9, so
# some workgroups run dead tile slots), 5 (5120 on 8) or 4 to 5 (4608 on 8);
# ragged K (H = 2176) and M
@pytest.mark.parametrize("M,H,V,cus", [(64, 1024, 4096, 8), (33, 2176, 4096, 8), (48, 640, 3584, 7),
                                       (64, 1152, 4096, 9), (64, 1024, 5120, 8), (40, 2176, 4608, 8)])
def test_kouter_kernel_shapes(M, H, V, cus):
    """33..64 rows with K outermost (each workgroup's tiles share one copy of
    every activation block): meets the oracle and picks the decode kernel's
    indices."""
    d = inputs.random_case(31 + M + cus, M, H, V, outliers=True)
    h, r, g, wc, ws = to_dev(d)
    with mtpd.plan_override(lmhead_kernel="decode"):
        _, codes, scales, m0, i0 = mtpd.draft_tail(h, r, g, d["eps"], wc, ws)
    with mtpd.plan_override(device_cus=cus):
        plan = mtpd.lmhead_plan(M, V, H)
        say(f"  plan: {plan}")
        assert plan.startswith("lmhead_kouter_kernel")
        m1, i1 = mtpd.fp8_lmhead_argmax(codes, scales, wc, ws)
    torch.cuda.synchronize()
    check_lmhead(codes, scales, d, m1, i1)
    assert torch.equal(i0, i1)


def test_kouter_kernel_full_width():
    """64 rows, H = 6144, V = 131072 on the device's own CU count (1024
    tiles: four per workgroup on 256 CUs), sampled rows against the oracle."""
    M, H, V = 64, 6144, 131072
    d = inputs.random_case(77, M, H, V, outliers=True)
    h, r, g, wc, ws = to_dev(d)
    say(f"  plan: {mtpd.lmhead_plan(M, V, H)}")
    _, codes, scales, m, i = mtpd.draft_tail(h, r, g, d["eps"], wc, ws)
    check_lmhead(codes, scales, d, m, i, rows=np.array([0, 17, 40, 63]))


# the DeepSeek-V3 shape of the LM head (H = 7168, V = 129280) through every
# decode-regime family the dispatcher picks for it: the one-row tail on the
# full vocab (505 workgroups, more than the one-row workspace's key slots),
# the per-tile stream kernel, the rows kernel and the K-outer kernel's
# eight-wave shape
@pytest.mark.parametrize("M", [1, 5, 17, 64])
def test_deepseek_shape_full_vocab(M):
    H, V = 7168, 129280
    d = inputs.random_case(91 + M, M, H, V, outliers=True)
    h, r, g, wc, ws = to_dev(d)
    say(f"deepseek shape M={M}: {mtpd.draft_tail_plan(M, V, H)}")
    out_h, codes, scales, m, i = mtpd.draft_tail(h, r, g, d["eps"], wc, ws)
    check_norm_quant(d, out_h, codes, scales)
    say("  " + str(check_lmhead(codes, scales, d, m, i)))


def test_stream_rows_kernel_vocab_shard_shape(workloads):
    """64 rows on one GPU's 18944-row vocab shard (the decode c=64 weight's
    first 148 blocks): every row against the oracle."""
    d = workloads("decode_c64_full")
    h, r, g, wc, ws = to_dev(d)
    S = 18944
    say(f"  plan: {mtpd.lmhead_plan(64, S, 6144)}")
    _, codes, scales, _, _ = mtpd.draft_tail(h, r, g, d["eps"], wc, ws)
    m, i = mtpd.fp8_lmhead_argmax(codes, scales, wc[:S], ws[:S // 128])
    c, s = host(codes), host(scales)
    ref = oracle.argmax(c, s, d["w_codes"][:S], d["w_scales"][:S // 128])
    say("  " + str(parity.check_argmax(host(m), host(i), ref,
                                        logit_row=lambda k: oracle.logits(c, s, d["w_codes"][:S],
                                                                          d["w_scales"][:S // 128], rows=[k])[0])))


# 16-row tiles per workgroup: one (256, 2048, 4096), one or two (5120), four
# or five (18944), eight or nine (33152), sixteen on 592 workgroups (151552)
# H past 6144 runs the norm in four 2048-column steps (6272: a partial fourth
# step; 7168 x 16256: one GPU's eighth of a 129280-row vocab, padded to 128-row blocks)
@pytest.mark.parametrize("H,V", [(128, 256), (256, 512), (384, 640), (1152, 2048), (2304, 4096), (1152, 5120),
                                 (6144, 18944), (640, 33152), (2048, 151552), (6272, 2048), (7168, 16256),
                                 (8192, 4096)])
def test_fused_one_row_draft_tail_matches_split(H, V):
    """One row: the fused single-kernel tail reproduces the two-launch path's
    recycled hidden, codes and scales bit for bit (the same arithmetic), and
    both paths' argmax meets the oracle (their K summation orders differ)."""
    say(f"fused tail H={H} V={V}: {mtpd.draft_tail_plan(1, V, H)}")
    d = inputs.random_case(17 + H, 1, H, V, outliers=True)
    h, r, g, wc, ws = to_dev(d)
    fused = mtpd.draft_tail(h, r, g, d["eps"], wc, ws)
    with mtpd.plan_override(draft_tail="split"):
        split = mtpd.draft_tail(h, r, g, d["eps"], wc, ws)
    torch.cuda.synchronize()
    for x, y in zip(fused[:3], split[:3]):
        assert torch.equal(x.view(torch.uint8) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.uint8) if y.dtype == torch.bfloat16 else y)
    check_norm_quant(d, *fused[:3])
    check_lmhead(fused[1], fused[2], d, fused[3], fused[4])
    check_lmhead(split[1], split[2], d, split[3], split[4])


# H = 128 .. 384: fewer K blocks than waves (a wave with none must still
# read real data: a dead unit's zero factor times NaN would poison the row)
@pytest.mark.parametrize("H,V", [(128, 256), (256, 512), (384, 640), (1152, 5120), (6144, 18944), (2048, 151552),
                                 (7168, 16256), (8192, 2048)])
def test_one_row_lm_head_alone(H, V):
    """The LM head alone on one packed row runs the fused tail's persistent
    kernel: its (max, index) equal the fused tail's bit for bit, meet the
    oracle, and a gathered row (row_index into a 3-row activation) gives that
    row's pair."""
    say(f"one-row head H={H} V={V}: {mtpd.lmhead_plan(1, V, H)}")
    assert mtpd.lmhead_plan(1, V, H).startswith("draft_tail1_kernel")
    d = inputs.random_case(43 + H, 3, H, V, outliers=True)
    h, r, g, wc, ws = to_dev(d)
    _, codes, scales, _, _ = mtpd.draft_tail(h, r, g, d["eps"], wc, ws)
    fused = mtpd.draft_tail(h[2:3], r[2:3], g, d["eps"], wc, ws)
    m, i = mtpd.fp8_lmhead_argmax(codes[2:3].contiguous(), scales[2:3].contiguous(), wc, ws)
    idx = torch.tensor([2], dtype=torch.int32, device=DEV)
    mg, ig = mtpd.fp8_lmhead_argmax(codes, scales, wc, ws, row_index=idx)
    torch.cuda.synchronize()
    assert torch.equal(m, fused[3]) and torch.equal(i, fused[4])
    assert torch.equal(mg, m) and torch.equal(ig, i)
    check_lmhead(fused[1], fused[2], d, m, i)


# one shape per kernel family: fused one-row tail, per-tile stream, rows
# kernel, K-outer kernel, compute-regime tile
@pytest.mark.parametrize("M,H,V", [(1, 512, 2048), (8, 512, 2048), (40, 256, 4096), (64, 256, 151552),
                                   (300, 256, 1024)])
def test_workspace_canaries(M, H, V):
    """The kernels touch only the workspace they are given and leave it zero:
    4 KB guard regions of 0xA5 on both sides of it stay intact, twice."""
    import ctypes
    from mtp_draft_head_amd import FP8Weight, QAct

    d = inputs.random_case(47 + M, M, H, V)
    h, r, g, wc, ws = to_dev(d)
    L = mtpd.lib()
    need = L.mtpd_workspace_bytes(M)
    G = 4096
    buf = torch.zeros(G + need + G, dtype=torch.uint8, device=DEV)
    buf[:G] = 0xA5
    buf[G + need:] = 0xA5
    out_h = torch.empty((M, H), dtype=torch.bfloat16, device=DEV)
    codes = torch.empty((M, H), dtype=torch.uint8, device=DEV)
    scales = torch.empty((M, H // 128), dtype=torch.float32, device=DEV)
    om = torch.empty((M,), dtype=torch.float32, device=DEV)
    oi = torch.empty((M,), dtype=torch.int32, device=DEV)
    qa = QAct(codes.data_ptr(), scales.data_ptr(), M, H)
    w = FP8Weight(wc.data_ptr(), ws.data_ptr(), V, H)
    ref = mtpd.draft_tail(h, r, g, d["eps"], wc, ws)
    for _ in range(2):
        st = L.mtpd_draft_tail(h.data_ptr(), r.data_ptr(), g.data_ptr(), float(d["eps"]), M, H, ctypes.byref(w),
                               out_h.data_ptr(), ctypes.byref(qa), om.data_ptr(), oi.data_ptr(),
                               buf.data_ptr() + G, need, torch.cuda.current_stream(DEV).cuda_stream)
        assert st == 0, L.mtpd_last_error().decode()
        torch.cuda.synchronize()
        assert bool((buf[:G] == 0xA5).all()) and bool((buf[G + need:] == 0xA5).all())
        assert int(buf[G:G + need].count_nonzero()) == 0
        assert torch.equal(oi, ref[4]) and torch.equal(om, ref[3])
    say(f"  canaries M={M} H={H} V={V}: {mtpd.draft_tail_plan(M, V, H)}")


def _scaled_case(seed, M, H, V, row_mag, small_blocks=()):
    """random_case with row m of hidden and residual scaled by row_mag[m], and
    the listed (row, 128-column block) pairs 1e-30 times smaller still."""
    d = inputs.random_case(seed, M, H, V)
    for key in ("hidden", "residual"):
        x = torch.from_numpy(d[key].view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
        x *= np.asarray(row_mag, np.float32)[:, None]
        for m, kb in small_blocks:
            x[m, kb * 128:(kb + 1) * 128] *= np.float32(1e-30)
        d[key] = inputs.to_bf16_bits(x)
    return d


def test_block_scales_across_the_exponent_range():
    """Block scales from about 2^-107 to 2^-6: a row so small that eps
    dominates its norm (scales below 2^-60, where the packing divides in full
    rather than through the block's reciprocal), rows just above that, and a
    normal row with blocks 1e-30 times smaller than the rest.  Hidden, codes
    and scales against the oracle, the packing self-consistent, and every row
    through the fused one-row tail bit for bit equal to the two-launch path."""
    M, H, V = 4, 1024, 512
    d = _scaled_case(31, M, H, V, [1e-20, 3e-18, 1e-16, 1.0], small_blocks=[(3, 1), (3, 5)])
    h, r, g, wc, ws = to_dev(d)
    out = mtpd.draft_tail(h, r, g, d["eps"], wc, ws)
    r1, r2, r3 = check_norm_quant(d, *out[:3])
    s = host(out[2])
    say(f"  scales {s[s > 0].min():.3e} .. {s.max():.3e}; bf16 {r1}  codes {r2}")
    assert s.min() > 0 and s.min() < 2.0 ** -100 and s[0].max() < 2.0 ** -60 and s[1].min() > 2.0 ** -60
    check_self_consistent(out[1], out[2])
    check_lmhead(out[1], out[2], d, out[3], out[4])
    for m in range(M):
        fused = mtpd.draft_tail(h[m:m + 1], r[m:m + 1], g, d["eps"], wc, ws)
        with mtpd.plan_override(draft_tail="split"):
            split = mtpd.draft_tail(h[m:m + 1], r[m:m + 1], g, d["eps"], wc, ws)
        torch.cuda.synchronize()
        for x, y in zip(fused[:3], split[:3]):
            assert torch.equal(x.view(torch.uint8) if x.dtype == torch.bfloat16 else x,
                               y.view(torch.uint8) if y.dtype == torch.bfloat16 else y), m


# compute-regime kernel variants (plan override lmhead_gemm): 1 the
# single-wait kernel, 2-4 pipelined 256-row tiles (row-tile groups 4, 8, 16),
# 5-6 pipelined 160-row tiles, 7-8 pipelined 320-row tiles; ragged M and odd
# K block counts (including fewer blocks than a scale chunk)
@pytest.mark.parametrize("variant", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("M,H,V", [(300, 1152, 1536), (65, 128, 512), (517, 2176, 2304), (160, 640, 768),
                                   (700, 1664, 1024)])
def test_gemm_variants(variant, M, H, V):
    """Every compute-regime variant meets the oracle on every row and picks the
    same indices as the generic kernel outside near ties (all variants sum the
    128-wide K blocks in the same order, so they agree bit for bit)."""
    d = inputs.random_case(19 + M + H, M, H, V, outliers=True)
    h, r, g, wc, ws = to_dev(d)
    with mtpd.plan_override(lmhead_gemm=1):
        _, codes, scales, m1, i1 = mtpd.draft_tail(h, r, g, d["eps"], wc, ws)
    with mtpd.plan_override(lmhead_gemm=variant):
        m, i = mtpd.fp8_lmhead_argmax(codes, scales, wc, ws)
    torch.cuda.synchronize()
    say(f"  variant {variant}: {check_lmhead(codes, scales, d, m, i)}")
    assert torch.equal(i, i1) and torch.equal(m, m1)


@pytest.mark.parametrize("variant", [2, 5, 7])
def test_gemm_variants_row_index(variant):
    """Gathered rows (repeats included) through the pipelined kernels give the
    ungathered call's pairs."""
    d = inputs.random_case(23, 200, 1024, 2048, outliers=True)
    h, r, g, wc, ws = to_dev(d)
    _, codes, scales, gmax, gidx = mtpd.draft_tail(h, r, g, d["eps"], wc, ws)
    sel = np.concatenate([[199, 0, 0, 7], np.random.default_rng(5).integers(0, 200, 296)]).astype(np.int32)
    idx = torch.from_numpy(sel).to(DEV)
    with mtpd.plan_override(lmhead_gemm=variant):
        m, i = mtpd.fp8_lmhead_argmax(codes, scales, wc, ws, row_index=idx)
    torch.cuda.synchronize()
    assert torch.equal(m, gmax[idx.long()]) and torch.equal(i, gidx[idx.long()])


@pytest.mark.parametrize("kernel", ["generic", "default"])
def test_many_rows_both_kernels(kernel):
    """More than 64 rows: the LDS-tiled 256x256 kernel by default, the generic
    tiled kernel when forced; both meet the oracle and pick the same indices."""
    d = inputs.random_case(12, 300, 1024, 1536, outliers=True)
    h, r, g, wc, ws = to_dev(d)
    with mtpd.plan_override(lmhead_kernel="generic" if kernel == "generic" else None):
        say(f"  plan: {mtpd.lmhead_plan(300, 1536, 1024)}")
        out_h, codes, scales, gmax, gidx = mtpd.draft_tail(h, r, g, d["eps"], wc, ws)
    check_norm_quant(d, out_h, codes, scales)
    check_lmhead(codes, scales, d, gmax, gidx)


# --------------------------------------------------------------------------
# the five workloads at full size
# --------------------------------------------------------------------------

def _sample(M, n, must, seed):
    rng = np.random.default_rng(seed)
    rows = set(int(x) for x in must)
    rest = [x for x in range(M) if x not in rows]
    rows |= set(int(x) for x in rng.choice(rest, size=min(len(rest), max(0, n - len(rows))), replace=False))
    return np.array(sorted(rows), np.int32)


def _sweep_cases(n=28, seed=20261202, cap=1.5e9):
    """Seeded shapes across every kernel family the dispatcher holds: row
    counts on both sides of each boundary (1, 16/17, 64/65, 256/257), H up to
    past the streaming kernels' limit, V a multiple of 128 or of 256, and
    sometimes a small CU count (which turns small vocabularies into several
    tiles per workgroup)."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        M = int(rng.choice([1, 2, 5, 9, 16, 17, 31, 33, 48, 64, 65, 100, 129, 200, 257, 300]))
        H = 128 * int(rng.integers(1, 73))
        V = (256 if rng.random() < 0.5 else 128) * int(rng.integers(1, 33))
        cus = [None, None, 8, 37][int(rng.integers(0, 4))]
        gather = bool(rng.random() < 0.5)
        if M * H * V <= cap:
            out.append((M, H, V, cus, gather, int(rng.integers(0, 2 ** 31))))
    # and the families a random draw may miss: the one-row tail and the
    # K-outer kernel (several tiles per workgroup) in both of its shapes
    out += [(1, 2048, 4096, None, True, 11), (1, 6144, 2560, 8, False, 12),
            (48, 1024, 4608, 8, True, 13), (40, 768, 4096, 8, False, 14), (64, 2304, 5120, 8, True, 15)]
    return out


SWEEP = _sweep_cases()


@pytest.mark.parametrize("M,H,V,cus,gather,seed", SWEEP)
def test_dispatcher_sweep(M, H, V, cus, gather, seed):
    """Whatever kernel the dispatcher picks: the norm step on every row, the
    packed activation self-consistent, every row's argmax against the oracle;
    half the cases also run the LM head alone on a gathered, repeating row
    list and check that against the oracle."""
    with mtpd.plan_override(**({"device_cus": cus} if cus else {})):
        say(f"sweep M={M} H={H} V={V} cus={cus} gather={gather}: {mtpd.lmhead_plan(M, V, H)}")
        d = inputs.random_case(seed, M, H, V, outliers=True)
        h, r, g, wc, ws = to_dev(d)
        out_h, codes, scales, gmax, gidx = mtpd.draft_tail(h, r, g, d["eps"], wc, ws)
        if gather:
            n = int(np.random.default_rng(seed).integers(1, M + 6))
            sel = np.random.default_rng(seed + 1).integers(0, M, n).astype(np.int32)
            idx = torch.from_numpy(sel).to(DEV)
            say(f"  gathered {n} rows: {mtpd.lmhead_plan(n, V, H)}")
            mg, ig = mtpd.fp8_lmhead_argmax(codes, scales, wc, ws, row_index=idx)
    check_norm_quant(d, out_h, codes, scales)
    check_self_consistent(codes, scales)
    say("  " + str(check_lmhead(codes, scales, d, gmax, gidx)))
    if gather:
        il = idx.long()
        say("  gathered " + str(check_lmhead(codes[il], scales[il], d, mg, ig)))


@pytest.mark.parametrize("name", ["decode_c1_tp8_shard", "decode_c64_full", "mtp5_batch", "compute_stress"])
def test_workload_full_size(name, workloads):
    d = workloads(name)
    w = d["workload"]
    say(f"workload {name}: M={w.M} H={w.H} V={w.V}")
    h, r, g, wc, ws = to_dev(d)
    out_h, codes, scales, gmax, gidx = mtpd.draft_tail(h, r, g, d["eps"], wc, ws)
    torch.cuda.synchronize()
    # every row of the 1-, 64- and 320-row workloads; a seeded 128-row subset
    # (always holding the planted near-tie rows) of the 8192-row one
    rows = None
    if w.M > 320:
        must = [p[0] for p in d["meta"]["near_tie_rows"]]
        rows = _sample(w.M, 128, must, 1234)
    # the norm step is cheap on the CPU: check every row
    r1, r2, r3 = check_norm_quant(d, out_h, codes, scales)
    say(f"  bf16 {r1}  codes {r2}  scales {r3}")
    check_self_consistent(codes, scales)
    rep = check_lmhead(codes, scales, d, gmax, gidx, rows=rows)
    say(f"  argmax over {w.M if rows is None else len(rows)} of {w.M} rows: {rep}")
    if name == "mtp5_batch":
        gi = host(gidx)
        for row, best, runner in d["meta"]["near_tie_rows"]:
            assert gi[row] in (best, runner)
    # determinism at full size
    o2 = mtpd.draft_tail(h, r, g, d["eps"], wc, ws)
    assert torch.equal(o2[4], gidx) and torch.equal(o2[3], gmax) and torch.equal(o2[1], codes)


def test_vocab_shards_combine_to_full_vocab(workloads):
    """The decode c=64 weight cut into 8 vocab shards of 18944 rows: each shard's
    local (max, idx) pairs, combined by largest max then lowest global index,
    give the full-vocab argmax (checked against the oracle, and index for index
    against the single full-vocab launch outside near-ties; shard and full
    launches may split K differently, so max values agree to rounding)."""
    d = workloads("decode_c64_full")
    h, r, g, wc, ws = to_dev(d)
    _, codes, scales, gmax, gidx = mtpd.draft_tail(h, r, g, d["eps"], wc, ws)
    S = 18944
    maxes, idxs = [], []
    for k in range(8):
        m, i = mtpd.fp8_lmhead_argmax(codes, scales, wc[k * S:(k + 1) * S], ws[k * S // 128:(k + 1) * S // 128])
        maxes.append(host(m))
        idxs.append(host(i))
    cm, ci = oracle.combine_shards(np.stack(maxes), np.stack(idxs), [k * S for k in range(8)])
    c, s = host(codes), host(scales)
    ref = oracle.argmax(c, s, d["w_codes"], d["w_scales"])
    rep = parity.check_argmax(cm, ci, ref,
                              logit_row=lambda i: oracle.logits(c, s, d["w_codes"], d["w_scales"], rows=[i])[0])
    say(f"  shards vs oracle {rep}")
    gap = (ref["z1"] - ref["z2"]) / np.abs(ref["z1"])
    clear = gap > 1e-5
    assert np.array_equal(ci[clear], host(gidx).astype(np.int64)[clear])
    assert np.allclose(cm, host(gmax), rtol=1e-5, atol=0)
