"""The C ABI without a GPU: the library loads, exports every symbol the header
declares, and rejects invalid arguments with typed statuses before any HIP
call (so nothing here launches a kernel)."""
import ctypes
import os
import re

import pytest

import mtp_draft_head_amd as m
from mtp_draft_head_amd import FP8Weight, QAct

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mtpd.h")

OK, NULL, SHAPE, ALIGN, ALIAS, WORKSPACE, HIP = range(7)
A = 0x10000000          # fake, never dereferenced device addresses (validation fails first)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mtpd_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(m.library_path()):
        from mtp_draft_head_amd import build
        build.build()
    return m.lib()


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert {"mtpd_norm_quant", "mtpd_fp8_lmhead_argmax", "mtpd_draft_tail", "mtpd_workspace_bytes",
            "mtpd_status_name", "mtpd_last_error", "mtpd_clear_error", "mtpd_abi_version",
            "mtpd_lmhead_plan", "mtpd_draft_tail_plan", "mtpd_allreduce_norm_quant",
            "mtpd_argmax_combine", "mtpd_topk_combine", "mtpd_fp8_lmhead_topk", "mtpd_topk_workspace_bytes",
            "mtpd_set_plan_override"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_status_names_and_version(L):
    assert [L.mtpd_status_name(i).decode() for i in range(7)] == [
        "MTPD_OK", "MTPD_ERR_NULL", "MTPD_ERR_SHAPE", "MTPD_ERR_ALIGN", "MTPD_ERR_ALIAS",
        "MTPD_ERR_WORKSPACE", "MTPD_ERR_HIP"]
    assert L.mtpd_status_name(99).decode() == "MTPD_UNKNOWN"
    assert L.mtpd_abi_version() == 7


def test_workspace_bytes(L):
    # P key partitions (256 halved until P * n_rows <= 4096, at least 1); while
    # P * n_rows <= 4096 each key has its own 128-byte line, else keys are dense;
    # padded to 256 bytes, then 33 counters on 128-byte lines (4352 bytes)
    def expect(n):
        P = 256
        while P > 1 and P * n > 4096:
            P //= 2
        stride = 16 if P * n <= 4096 else 1
        return -(-P * n * stride * 8 // 256) * 256 + 4352
    assert L.mtpd_workspace_bytes(0) == 0
    assert L.mtpd_workspace_bytes(-3) == 0
    for n in (1, 7, 30, 31, 64, 65, 320, 4096, 4097, 8192, 1 << 24):
        assert L.mtpd_workspace_bytes(n) == expect(n), n
        assert L.mtpd_workspace_bytes(n) % 256 == 0
    assert L.mtpd_workspace_bytes(1) == 32768 + 4352
    assert L.mtpd_workspace_bytes(8192) == 65536 + 4352


def nq(L, hidden=A, residual=A + 0x1000000, g=A + 0x2000000, M=4, H=256, out_h=A + 0x3000000,
       codes=A + 0x4000000, scales=A + 0x5000000, rows=None, cols=None):
    qa = QAct(codes, scales, M if rows is None else rows, H if cols is None else cols)
    L.mtpd_clear_error()
    return L.mtpd_norm_quant(hidden, residual, g, 1e-6, M, H, out_h, ctypes.byref(qa), None)


def test_norm_quant_validation(L):
    assert nq(L, hidden=None) == NULL
    assert "NULL" in L.mtpd_last_error().decode()
    assert nq(L, H=200) == SHAPE
    assert nq(L, H=0) == SHAPE
    assert nq(L, H=16384 + 128, cols=16384 + 128) == SHAPE
    assert nq(L, M=-1) == SHAPE
    assert nq(L, rows=3) == SHAPE
    assert nq(L, cols=128) == SHAPE
    assert nq(L, hidden=A + 8) == ALIGN
    assert nq(L, codes=A + 0x4000000 + 4) == ALIGN
    assert nq(L, scales=A + 0x5000000 + 2) == ALIGN
    assert nq(L, out_h=A) == ALIAS                       # output over the hidden input
    assert nq(L, codes=A + 0x3000000 + 512) == ALIAS     # codes inside out_hidden
    assert nq(L, M=0) == OK                              # empty call: nothing to do, nothing launched
    assert L.mtpd_norm_quant(A, A, A, 1e-6, 4, 256, A, None, None) == NULL


def test_first_error_is_kept_until_cleared(L):
    L.mtpd_clear_error()
    qa = QAct(A + 0x4000000, A + 0x5000000, 4, 256)
    assert L.mtpd_norm_quant(None, A, A, 1e-6, 4, 256, A, ctypes.byref(qa), None) == NULL
    first = L.mtpd_last_error().decode()
    assert L.mtpd_norm_quant(A, A, A, 1e-6, 4, 200, A, ctypes.byref(qa), None) == SHAPE
    assert L.mtpd_last_error().decode() == first
    L.mtpd_clear_error()
    assert L.mtpd_last_error().decode() == ""


def lm(L, M=4, H=256, V=1024, act_rows=None, act_codes=A, act_scales=A + 0x100000, row_index=None,
       w_codes=A + 0x1000000, w_scales=A + 0x2000000, wV=None, wH=None, out_max=A + 0x3000000,
       out_idx=A + 0x3100000, ws=A + 0x4000000, ws_bytes=None):
    qa = QAct(act_codes, act_scales, M if act_rows is None else act_rows, H)
    w = FP8Weight(w_codes, w_scales, V if wV is None else wV, H if wH is None else wH)
    if ws_bytes is None:
        ws_bytes = L.mtpd_workspace_bytes(M)
    L.mtpd_clear_error()
    return L.mtpd_fp8_lmhead_argmax(ctypes.byref(qa), row_index, M, ctypes.byref(w), out_max, out_idx,
                                    ws, ws_bytes, None)


def test_lmhead_validation(L):
    assert lm(L, act_codes=None) == NULL
    assert lm(L, w_codes=None) == NULL
    assert lm(L, out_idx=None) == NULL
    assert lm(L, V=1000) == SHAPE
    assert lm(L, V=1 << 31, wV=1 << 31) == SHAPE
    assert lm(L, wH=512) == SHAPE
    assert lm(L, M=5, act_rows=4) == SHAPE               # more rows than the activation, no row_index
    assert lm(L, M=-2) == SHAPE
    assert lm(L, w_codes=A + 0x1000000 + 1) == ALIGN
    assert lm(L, ws=A + 0x4000000 + 64) == ALIGN
    assert lm(L, ws=None) == WORKSPACE
    assert lm(L, ws_bytes=16) == WORKSPACE
    assert lm(L, ws_bytes=L.mtpd_workspace_bytes(4) - 256) == WORKSPACE
    assert lm(L, out_max=A + 0x1000000 + 64) == ALIAS     # output inside the weight codes
    assert lm(L, out_idx=A + 0x3000000) == ALIAS          # two outputs overlap
    assert lm(L, ws=A + 0x100000) == ALIAS                # workspace over the activation scales
    assert lm(L, M=0) == OK


def test_draft_tail_validation(L):
    def dt(M=4, H=256, V=1024, wH=None, ws_bytes=None, out_max=A + 0x6000000, hidden=A):
        qa = QAct(A + 0x4000000, A + 0x5000000, M, H)
        w = FP8Weight(A + 0x7000000, A + 0x8000000, V, H if wH is None else wH)
        L.mtpd_clear_error()
        return L.mtpd_draft_tail(hidden, A + 0x1000000, A + 0x2000000, 1e-6, M, H, ctypes.byref(w),
                                 A + 0x3000000, ctypes.byref(qa), out_max, A + 0x6100000, A + 0x9000000,
                                 L.mtpd_workspace_bytes(M) if ws_bytes is None else ws_bytes, None)
    assert dt(hidden=None) == NULL
    assert dt(wH=512) == SHAPE
    assert dt(V=100) == SHAPE
    assert dt(ws_bytes=8) == WORKSPACE
    assert dt(out_max=A + 0x7000000) == ALIAS
    assert dt(M=0) == OK


def test_allreduce_norm_quant_validation(L):
    def ar(ptrs=(A, A + 0x400000), n=None, residual=A + 0x1000000, M=4, H=256, out_h=A + 0x3000000,
           codes=A + 0x4000000):
        n = len(ptrs) if n is None else n
        arr = (ctypes.c_void_p * max(1, len(ptrs)))(*ptrs) if ptrs is not None else None
        qa = QAct(codes, A + 0x5000000, M, H)
        L.mtpd_clear_error()
        return L.mtpd_allreduce_norm_quant(arr, n, residual, A + 0x2000000, 1e-6,
                                           M, H, out_h, ctypes.byref(qa), None)
    assert ar(n=0) == SHAPE
    assert ar(n=17, ptrs=[A + i * 0x10000 for i in range(17)]) == SHAPE
    assert ar(ptrs=None, n=2) == NULL
    assert ar(ptrs=(A, None)) == NULL
    assert ar(ptrs=(A, A + 0x400000 + 8)) == ALIGN
    assert ar(H=200) == SHAPE
    assert ar(residual=None) == NULL
    assert ar(out_h=A + 0x400000) == ALIAS                # output over the second partial
    assert ar(codes=A + 0x400000 + 256) == ALIAS
    assert ar(M=0) == OK


def test_argmax_combine_validation(L):
    def cb(offs=(0, 1024), n=None, rows=4, lmax=A, lidx=A + 0x1000, omax=A + 0x2000, oidx=A + 0x3000):
        n = len(offs) if n is None else n
        arr = (ctypes.c_int64 * max(1, len(offs)))(*offs) if offs is not None else None
        L.mtpd_clear_error()
        return L.mtpd_argmax_combine(lmax, lidx, arr, n, rows, omax, oidx, None)
    assert cb(n=0) == SHAPE
    assert cb(offs=list(range(65))) == SHAPE
    assert cb(offs=(0, -128)) == SHAPE
    assert cb(offs=(0, 1 << 31)) == SHAPE
    assert cb(offs=None, n=2) == NULL
    assert cb(rows=-1) == SHAPE
    assert cb(rows=(1 << 24) + 1) == SHAPE
    assert cb(lmax=None) == NULL
    assert cb(oidx=A + 0x3002) == ALIGN
    assert cb(omax=A + 8) == ALIAS                        # output inside local_max ([2][4] f32)
    assert cb(oidx=A + 0x2008) == ALIAS                   # the two outputs overlap
    assert cb(rows=0, lmax=None, lidx=None, omax=None, oidx=None) == OK


def test_topk_combine_validation(L):
    def cb(offs=(0, 1024), n=None, rows=4, k=8, lval=A, lidx=A + 0x1000, oval=A + 0x2000, oidx=A + 0x3000):
        n = len(offs) if n is None else n
        arr = (ctypes.c_int64 * max(1, len(offs)))(*offs) if offs is not None else None
        L.mtpd_clear_error()
        return L.mtpd_topk_combine(lval, lidx, arr, n, rows, k, oval, oidx, None)
    assert cb(n=0) == SHAPE
    assert cb(offs=list(range(65))) == SHAPE
    assert cb(offs=(0, -128)) == SHAPE
    assert cb(offs=(0, 1 << 31)) == SHAPE
    assert cb(offs=None, n=2) == NULL
    assert cb(rows=-1) == SHAPE
    assert cb(rows=(1 << 24) + 1) == SHAPE
    assert cb(k=0) == SHAPE
    assert cb(k=33) == SHAPE
    assert cb(lval=None) == NULL
    assert cb(oval=A + 0x2002) == ALIGN
    assert cb(oval=A + 0x80) == ALIAS                      # output inside local_val ([2][4][8] f32)
    assert cb(oidx=A + 0x2040) == ALIAS                    # the two outputs ([4][8] each) overlap
    assert cb(rows=0, lval=None, lidx=None, oval=None, oidx=None) == OK


def test_topk_workspace_bytes(L):
    # one pass of at most 64 rows: rows x (V / 32 lists) x k keys x 8 bytes, padded to 256
    assert L.mtpd_topk_workspace_bytes(1, 18944, 8) == -(-1 * (18944 // 32) * 8 * 8 // 256) * 256
    assert L.mtpd_topk_workspace_bytes(64, 151552, 32) == 64 * (151552 // 32) * 32 * 8
    assert L.mtpd_topk_workspace_bytes(300, 1024, 4) == L.mtpd_topk_workspace_bytes(64, 1024, 4)
    assert L.mtpd_topk_workspace_bytes(0, 1024, 4) == 0
    assert L.mtpd_topk_workspace_bytes(4, 1024, 0) == 0
    assert L.mtpd_topk_workspace_bytes(4, 1024, 33) == 0
    assert L.mtpd_topk_workspace_bytes(4, 1000, 4) == 0


def test_topk_validation(L):
    def tk(M=4, H=256, V=1024, k=8, act_codes=A, w_codes=A + 0x1000000, ws=A + 0x4000000, ws_bytes=None,
           out_val=A + 0x3000000, out_idx=A + 0x3100000):
        qa = QAct(act_codes, A + 0x100000, M, H)
        w = FP8Weight(w_codes, A + 0x2000000, V, H)
        if ws_bytes is None:
            ws_bytes = max(L.mtpd_topk_workspace_bytes(M, V, k), 256)
        L.mtpd_clear_error()
        return L.mtpd_fp8_lmhead_topk(ctypes.byref(qa), None, M, ctypes.byref(w), k, out_val, out_idx, ws,
                                      ws_bytes, None)
    assert tk(k=0) == SHAPE
    assert tk(k=33) == SHAPE
    assert tk(H=16384) == SHAPE                          # beyond the streaming kernel's H
    assert tk(V=1000) == SHAPE
    assert tk(act_codes=None) == NULL
    assert tk(out_val=None) == NULL
    assert tk(ws=None) == WORKSPACE
    assert tk(ws_bytes=256) == WORKSPACE
    assert tk(ws=A + 0x4000000 + 64) == ALIGN
    assert tk(out_idx=A + 0x3000000 + 16) == ALIAS       # the two outputs overlap
    assert tk(out_val=A + 0x1000000) == ALIAS            # output over the weight codes
    assert tk(M=0) == OK


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros((4, 256), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        m.norm_quant(x, x, torch.ones(256), 1e-6)


def test_plan_override_parsing(L):
    """The override setter rejects unknown keys and malformed values (changing
    nothing), and the plan strings follow what it pins (host-only)."""
    L.mtpd_set_plan_override(None, None)
    auto = L.mtpd_lmhead_plan(24, 2048, 1536).decode()
    for key, bad in [(b"nonsense", b"1"), (b"lmhead_kernel", b"fast"), (b"lmhead_tile", b"2,2"),
                     (b"lmhead_tile", b"2,x,4"), (b"lmhead_stream", b"0,4"), (b"lmhead_kouter", b"1,2,3"),
                     (b"draft_tail", b"fused"), (b"device_cus", b"-3"), (b"lmhead_rows", b"1,2,3,4"),
                     (b"norm_quant", b"warp")]:
        L.mtpd_clear_error()
        assert L.mtpd_set_plan_override(key, bad) == SHAPE, (key, bad)
        assert L.mtpd_last_error().decode().startswith("MTPD_ERR_SHAPE")
        assert L.mtpd_lmhead_plan(24, 2048, 1536).decode() == auto
    try:
        assert L.mtpd_set_plan_override(b"lmhead_kernel", b"generic") == OK
        assert L.mtpd_set_plan_override(b"lmhead_tile", b"2,4,4") == OK
        assert L.mtpd_lmhead_plan(24, 2048, 1536).decode().startswith("lmhead_argmax_kernel<2,2,4,4>")
        assert L.mtpd_set_plan_override(b"lmhead_tile", None) == OK      # one key cleared
        assert L.mtpd_lmhead_plan(24, 2048, 1536).decode().startswith("lmhead_argmax_kernel<")
        assert L.mtpd_set_plan_override(b"draft_tail", b"split") == OK
        assert L.mtpd_draft_tail_plan(1, 2048, 1024).decode().startswith("norm_quant_kernel")
        assert L.mtpd_set_plan_override(b"norm_quant", b"wave") == OK
        assert L.mtpd_draft_tail_plan(9, 2048, 1024).decode().startswith("norm_quant_wave_kernel<2> grid=3x256")
        assert L.mtpd_draft_tail_plan(9, 2048, 16384).decode().startswith("norm_quant_kernel<8> grid=9x256")
        assert L.mtpd_set_plan_override(b"norm_quant", b"workgroup") == OK
        assert L.mtpd_draft_tail_plan(9, 2048, 1024).decode().startswith("norm_quant_kernel<1> grid=9x256")
    finally:
        assert L.mtpd_set_plan_override(None, None) == OK
    assert L.mtpd_lmhead_plan(24, 2048, 1536).decode() == auto
    assert L.mtpd_draft_tail_plan(1, 2048, 1024).decode().startswith("draft_tail1_kernel")
    with m.plan_override(device_cus=8, lmhead_kouter="0"):
        assert not L.mtpd_lmhead_plan(64, 4096, 1024).decode().startswith("lmhead_kouter")
    with pytest.raises(KeyError):
        m.plan_override(bogus=1)


def test_noalloc_rejects_too_many_rows(L):
    """The allocation-free tail refuses M beyond its scratch before any HIP call;
    its scratch covers the workspace of the largest M it accepts."""
    assert L.mtpd_workspace_bytes(65536) <= 528640
    qa = QAct(0x10000000, 0x20000000, 65537, 256)
    w = FP8Weight(0x30000000, 0x40000000, 256, 256)
    L.mtpd_clear_error()
    st = L.mtpd_draft_tail_noalloc(0x50000000, 0x60000000, 0x70000000, 1e-6, 65537, 256, ctypes.byref(w),
                                   0x80000000, ctypes.byref(qa), 0x90000000, 0xA0000000, None)
    assert st == 5, st   # MTPD_ERR_WORKSPACE, before any HIP call
    assert "65536" in L.mtpd_last_error().decode()
    L.mtpd_clear_error()


def test_dispatcher_sweep_reaches_every_kernel_family():
    """The GPU dispatcher sweep is only as good as the kernels it reaches
    (the plan is decided on the host, so this runs without a GPU)."""
    from tests.test_gpu_parity import SWEEP
    fams = set()
    for M, H, V, cus, _, _ in SWEEP:
        with m.plan_override(**({"device_cus": cus} if cus else {})):
            fams.add(m.lmhead_plan(M, V, H).split("<")[0].split(" ")[0])
    assert {"draft_tail1_kernel", "lmhead_stream_kernel", "lmhead_stream_rows_kernel", "lmhead_kouter_kernel",
            "lmhead_gemm2_kernel", "lmhead_argmax_kernel"} <= fams, fams
