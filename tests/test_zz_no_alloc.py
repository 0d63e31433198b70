"""The allocation-free draft tail (mtpd_draft_tail_noalloc, called through the
C ABI) against mtpd_draft_tail on the same inputs: two calls in a row, the
second with fewer rows, and a one-row call (the fused tail), each bit for bit
(the same kernels run; only the scratch differs)."""
import ctypes

import numpy as np
import pytest
import torch

import mtp_draft_head_amd as mtpd
from mtp_draft_head_amd import FP8Weight, QAct, inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _dev(d):
    h = torch.from_numpy(d["hidden"].view(np.int16)).to(DEV).view(torch.bfloat16)
    r = torch.from_numpy(d["residual"].view(np.int16)).to(DEV).view(torch.bfloat16)
    g = torch.from_numpy(d["norm_weight"]).to(DEV)
    wc = torch.from_numpy(d["w_codes"]).to(DEV)
    ws = torch.from_numpy(d["w_scales"]).to(DEV)
    return h, r, g, wc, ws


def _noalloc(h, r, g, eps, wc, ws):
    M, H = h.shape
    V = wc.shape[0]
    out = (torch.full((M, H), -1, dtype=torch.int16, device=DEV).view(torch.bfloat16),
           torch.full((M, H), 0xFF, dtype=torch.uint8, device=DEV),
           torch.full((M, H // 128), float("nan"), dtype=torch.float32, device=DEV),
           torch.full((M,), float("nan"), dtype=torch.float32, device=DEV),
           torch.full((M,), -7, dtype=torch.int32, device=DEV))
    qa = QAct(out[1].data_ptr(), out[2].data_ptr(), M, H)
    w = FP8Weight(wc.data_ptr(), ws.data_ptr(), V, H)
    st = mtpd.lib().mtpd_draft_tail_noalloc(h.data_ptr(), r.data_ptr(), g.data_ptr(), float(eps), M, H,
                                            ctypes.byref(w), out[0].data_ptr(), ctypes.byref(qa),
                                            out[3].data_ptr(), out[4].data_ptr(),
                                            torch.cuda.current_stream(DEV).cuda_stream)
    assert st == 0, mtpd.lib().mtpd_last_error().decode()
    return out


def _same(a, b):
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.uint8) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.uint8) if y.dtype == torch.bfloat16 else y)


@pytest.mark.parametrize("first,second", [((300, 1024, 2048), (40, 1024, 2048)), ((64, 6144, 4096), (1, 6144, 4096))])
def test_noalloc_matches_draft_tail_twice(first, second):
    for k, (M, H, V) in enumerate((first, second)):
        d = inputs.random_case(61 + k + M, M, H, V, outliers=True)
        h, r, g, wc, ws = _dev(d)
        ref = mtpd.draft_tail(h, r, g, d["eps"], wc, ws)
        got = _noalloc(h, r, g, d["eps"], wc, ws)
        torch.cuda.synchronize()
        print(f"  no-alloc M={M} H={H} V={V}: idx {got[4][:4].tolist()}", flush=True)
        _same(got, ref)

