"""Chained MTP positions on the GPU: successive draft_tail calls in which each
position's hidden input is the previous position's recycled bf16 hidden
("[Quant][MTP] Reuse packed FP8 logits inputs", Purpose: the post-norm bf16
hidden is recycled into the next MTP position).  The layer body between
positions needs real weights, so an identity stands in for it (the residual
is kept).

Checked stagewise against the oracle on the GPU's own inputs (position p's
input is the GPU's output of position p - 1, so an allowed one-ulp difference
does not compound), and a HIP graph holding the whole chain is replayed
several times, with eager work in between, against the eager chain bit for
bit.
"""
import numpy as np
import pytest
import torch

import mtp_draft_head_amd as mtpd
from mtp_draft_head_amd import inputs
from tests.test_gpu_parity import DEV, check_lmhead, check_norm_quant, host, say, to_dev

pytestmark = pytest.mark.gpu


def _bufs(M, H):
    return (torch.empty((M, H), dtype=torch.bfloat16, device=DEV),
            torch.empty((M, H), dtype=torch.uint8, device=DEV),
            torch.empty((M, H // 128), dtype=torch.float32, device=DEV),
            torch.empty((M,), dtype=torch.float32, device=DEV),
            torch.empty((M,), dtype=torch.int32, device=DEV))


def _chain(h, r, g, eps, wc, ws, outs, wsp):
    hin = h
    for o in outs:
        mtpd.draft_tail(hin, r, g, eps, wc, ws, workspace=wsp, out=o)
        hin = o[0]


def _same(a, b):
    return all(torch.equal(x.view(torch.uint8) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.uint8) if y.dtype == torch.bfloat16 else y) for x, y in zip(a, b))


@pytest.mark.parametrize("name,K", [("decode_c1_tp8_shard", 5), ("decode_c1_tp8_shard", 3), ("tiny", 5)])
def test_chained_positions_stagewise_and_graph(name, K, workloads):
    d = workloads(name)
    w = d["workload"]
    say(f"chain {name}: K={K} M={w.M} H={w.H} V={w.V}")
    h, r, g, wc, ws = to_dev(d)
    wsp = mtpd.Workspace(DEV, any_stream=True)   # eager calls and a graph captured on a side stream
    wsp.get(w.M)
    outs = [_bufs(w.M, w.H) for _ in range(K)]
    _chain(h, r, g, d["eps"], wc, ws, outs, wsp)
    torch.cuda.synchronize()
    eager = [tuple(x.clone() for x in o) for o in outs]

    # stagewise parity: position p against the oracle on the GPU's own input
    for p in range(K):
        dp = dict(d)
        if p > 0:
            dp["hidden"] = host(eager[p - 1][0])
        r1, r2, r3 = check_norm_quant(dp, *eager[p][:3])
        rep = check_lmhead(eager[p][1], eager[p][2], dp, eager[p][3], eager[p][4])
        say(f"  position {p}: bf16 {r1}  codes {r2}  argmax {rep}")
    # the positions really differ (the recycled hidden moves the norm input)
    assert not torch.equal(eager[0][0].view(torch.int16), eager[1][0].view(torch.int16))

    # the whole chain in one graph, replayed with eager work in between
    s = torch.cuda.Stream(device=DEV)
    s.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(s):
        _chain(h, r, g, d["eps"], wc, ws, outs, wsp)
    torch.cuda.current_stream(DEV).wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _chain(h, r, g, d["eps"], wc, ws, outs, wsp)
    for rep in range(3):
        for o in outs:
            for x in o:
                x.view(torch.uint8).fill_(0xA5)      # poison between replays
        graph.replay()
        torch.cuda.synchronize()
        for p in range(K):
            assert _same(outs[p], eager[p]), (rep, p)
        mtpd.draft_tail(h, r, g, d["eps"], wc, ws, workspace=wsp)   # eager work between replays
        torch.cuda.synchronize()
    assert int(wsp.buf.count_nonzero().item()) == 0
