"""MTP draft-layer tail on one AMD MI355X (gfx950).

Thin Python binding over libmtpd's C ABI (``include/mtpd.h``): it checks
tensor dtypes, devices and contiguity, then passes raw device pointers and
the current HIP stream.  Every step of the path runs in the HIP kernels of
libmtpd; this module only marshals arguments.  PyTorch supplies device memory
and streams.

The library is loaded on first use from ``mtp_draft_head_amd/_build``; if it
is missing, calls raise ``MtpdLibraryMissing`` -- there is no fallback.
Build it with ``python -m mtp_draft_head_amd.build`` (or the repository's
``__graft_entry__.build()``).

Entry points (same names as the C ABI):
  norm_quant(hidden, residual, norm_weight, eps)
      -> (out_hidden bf16 [M,H], codes uint8 [M,H], scales f32 [M,H/128])
  fp8_lmhead_argmax(codes, scales, w_codes, w_scales, row_index=None)
      -> (max f32 [n], idx int32 [n])
  draft_tail(hidden, residual, norm_weight, eps, w_codes, w_scales)
      -> (out_hidden, codes, scales, max, idx)
  allreduce_norm_quant(partials, residual, norm_weight, eps)
      -> norm_quant's outputs for the norm input sum(partials) + residual
  argmax_combine(local_max, local_idx, shard_offsets)
      -> (max f32 [n], global idx int32 [n]) from per-shard pairs [P, n]
  fp8_lmhead_topk(codes, scales, w_codes, w_scales, k, row_index=None)
      -> (values f32 [n, k], idx int32 [n, k]), descending
  topk_combine(local_val, local_idx, shard_offsets)
      -> (values f32 [n, k], global idx int32 [n, k]) from per-shard lists [P, n, k]
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

__all__ = [
    "MtpdError", "MtpdLibraryMissing", "norm_quant", "fp8_lmhead_argmax", "draft_tail",
    "workspace_bytes", "Workspace", "library_path", "lib", "lmhead_plan", "draft_tail_plan",
    "allreduce_norm_quant", "argmax_combine", "topk_combine", "fp8_lmhead_topk", "topk_workspace_bytes",
    "plan_override",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
BLOCK = 128


def library_path() -> str:
    return os.path.join(_HERE, "_build", "libmtpd.so")


class MtpdLibraryMissing(RuntimeError):
    pass


class MtpdError(RuntimeError):
    def __init__(self, status: int, name: str, detail: str):
        super().__init__(f"{name} ({status}): {detail}")
        self.status = status
        self.name = name
        self.detail = detail


class QAct(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64)]


class FP8Weight(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("V", ctypes.c_int64), ("H", ctypes.c_int64)]


_lib = None
_lib_lock = threading.Lock()


def lib():
    """The loaded libmtpd (ctypes.CDLL), with argument types declared."""
    global _lib
    if _lib is not None:
        return _lib
    with _lib_lock:
        if _lib is not None:
            return _lib
        path = library_path()
        if not os.path.exists(path):
            raise MtpdLibraryMissing(
                f"{path} is not built; run `python -m mtp_draft_head_amd.build` (no CPU fallback exists)")
        L = ctypes.CDLL(path)
        P, I64, F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float
        L.mtpd_norm_quant.restype = ctypes.c_int
        L.mtpd_norm_quant.argtypes = [P, P, P, F, I64, I64, P, ctypes.POINTER(QAct), P]
        L.mtpd_fp8_lmhead_argmax.restype = ctypes.c_int
        L.mtpd_fp8_lmhead_argmax.argtypes = [ctypes.POINTER(QAct), P, I64, ctypes.POINTER(FP8Weight),
                                             P, P, P, ctypes.c_size_t, P]
        L.mtpd_draft_tail.restype = ctypes.c_int
        L.mtpd_draft_tail.argtypes = [P, P, P, F, I64, I64, ctypes.POINTER(FP8Weight), P,
                                      ctypes.POINTER(QAct), P, P, P, ctypes.c_size_t, P]
        L.mtpd_allreduce_norm_quant.restype = ctypes.c_int
        L.mtpd_allreduce_norm_quant.argtypes = [ctypes.POINTER(ctypes.c_void_p), I64, P, P, F, I64, I64, P,
                                                ctypes.POINTER(QAct), P]
        L.mtpd_argmax_combine.restype = ctypes.c_int
        L.mtpd_argmax_combine.argtypes = [P, P, ctypes.POINTER(ctypes.c_int64), I64, I64, P, P, P]
        L.mtpd_topk_combine.restype = ctypes.c_int
        L.mtpd_topk_combine.argtypes = [P, P, ctypes.POINTER(ctypes.c_int64), I64, I64, I64, P, P, P]
        L.mtpd_fp8_lmhead_topk.restype = ctypes.c_int
        L.mtpd_fp8_lmhead_topk.argtypes = [ctypes.POINTER(QAct), P, I64, ctypes.POINTER(FP8Weight), I64, P, P, P,
                                           ctypes.c_size_t, P]
        L.mtpd_topk_workspace_bytes.restype = ctypes.c_size_t
        L.mtpd_topk_workspace_bytes.argtypes = [I64, I64, I64]
        L.mtpd_workspace_bytes.restype = ctypes.c_size_t
        L.mtpd_workspace_bytes.argtypes = [I64]
        L.mtpd_status_name.restype = ctypes.c_char_p
        L.mtpd_status_name.argtypes = [ctypes.c_int]
        L.mtpd_last_error.restype = ctypes.c_char_p
        L.mtpd_last_error.argtypes = []
        L.mtpd_clear_error.restype = None
        L.mtpd_clear_error.argtypes = []
        L.mtpd_lmhead_plan.restype = ctypes.c_char_p
        L.mtpd_lmhead_plan.argtypes = [I64, I64, I64]
        L.mtpd_draft_tail_plan.restype = ctypes.c_char_p
        L.mtpd_draft_tail_plan.argtypes = [I64, I64, I64]
        L.mtpd_abi_version.restype = ctypes.c_int
        L.mtpd_abi_version.argtypes = []
        L.mtpd_draft_tail_noalloc.restype = ctypes.c_int
        L.mtpd_draft_tail_noalloc.argtypes = [P, P, P, F, I64, I64, ctypes.POINTER(FP8Weight), P,
                                              ctypes.POINTER(QAct), P, P, P]
        L.mtpd_set_plan_override.restype = ctypes.c_int
        L.mtpd_set_plan_override.argtypes = [ctypes.c_char_p, ctypes.c_char_p]
        _lib = L
        return L


def _check(status: int):
    if status != 0:
        L = lib()
        name = L.mtpd_status_name(status).decode()
        detail = L.mtpd_last_error().decode()
        L.mtpd_clear_error()
        raise MtpdError(status, name, detail)


def lmhead_plan(n_rows: int, V: int, H: int) -> str:
    """The LM-head kernel and launch shape the library picks for these sizes."""
    return lib().mtpd_lmhead_plan(int(n_rows), int(V), int(H)).decode()


def draft_tail_plan(M: int, V: int, H: int) -> str:
    """The kernel launches draft_tail makes for these sizes."""
    return lib().mtpd_draft_tail_plan(int(M), int(V), int(H)).decode()


def workspace_bytes(n_rows: int) -> int:
    return int(lib().mtpd_workspace_bytes(int(n_rows)))


class Workspace:
    """A zero-filled device workspace, grown on demand and reused.

    The library leaves the workspace zero-filled after every completed call,
    so one buffer serves any number of calls issued in order on ONE stream:
    calls in flight together on two streams would merge their argmax keys and
    arrival counters.  The workspace therefore binds to the stream of its
    first call and raises ValueError if a later call runs on another stream
    (the default workspaces are kept per device and stream, so they never
    do).  ``any_stream=True`` lifts the check for callers that order every
    use themselves, e.g. a HIP graph captured on torch's capture stream and
    replayed on the stream of the eager calls.  When the buffer grows, the
    old one is released only after the work already queued on the stream of
    its last use (``record_stream``).
    """

    def __init__(self, device=None, any_stream: bool = False):
        self.device = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
        self.buf = None
        self.stream = None
        self.any_stream = bool(any_stream)

    def get(self, n_rows: int) -> torch.Tensor:
        return self.get_bytes(workspace_bytes(n_rows))

    def get_bytes(self, need: int) -> torch.Tensor:
        stream = torch.cuda.current_stream(self.device)
        if self.stream is None or self.any_stream:
            if self.buf is not None and self.stream is not None and self.stream.cuda_stream != stream.cuda_stream:
                self.buf.record_stream(stream)
            self.stream = stream
        elif self.stream.cuda_stream != stream.cuda_stream:
            raise ValueError("this Workspace is bound to another stream; calls that may overlap in time "
                             "need separate workspaces")
        if self.buf is None or self.buf.numel() < need:
            if self.buf is not None:
                self.buf.record_stream(self.stream)
            with torch.cuda.stream(self.stream):
                self.buf = torch.zeros(max(need, 256), dtype=torch.uint8, device=self.device)
        return self.buf


_default_ws: dict = {}


def _workspace_for(device: torch.device) -> Workspace:
    key = (device.type, device.index, torch.cuda.current_stream(device).cuda_stream)
    if key not in _default_ws:
        _default_ws[key] = Workspace(device)
    return _default_ws[key]


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


_OVERRIDE_KEYS = ("lmhead_kernel", "lmhead_tile", "lmhead_stream", "lmhead_rows", "lmhead_decode",
                  "lmhead_kouter", "lmhead_gemm", "draft_tail", "device_cus", "norm_quant")


class plan_override:
    """Context manager pinning the library's launch plan (tuning and tests only).

    ``with plan_override(lmhead_kernel="generic", device_cus=8): ...`` sets the
    given keys of ``mtpd_set_plan_override`` (values as strings, tuples or
    ints; None leaves a key automatic) and clears every key on exit.  The
    setting is process-wide: use it only while no other thread calls the
    library.
    """

    def __init__(self, **keys):
        for k in keys:
            if k not in _OVERRIDE_KEYS:
                raise KeyError(f"unknown plan-override key {k!r}")
        self.keys = keys

    def __enter__(self):
        L = lib()
        L.mtpd_set_plan_override(None, None)
        for k, v in self.keys.items():
            if v is None:
                continue
            if isinstance(v, (tuple, list)):
                v = ",".join(str(int(x)) for x in v)
            _check(L.mtpd_set_plan_override(k.encode(), str(v).encode()))
        return self

    def __exit__(self, *exc):
        lib().mtpd_set_plan_override(None, None)
        return False


def _dev(t: torch.Tensor, name: str, dtypes, dim: int):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU (got {t.device}); there is no CPU path")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if t.dim() != dim:
        raise ValueError(f"{name} must be {dim}-D, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)
_U8 = (torch.uint8, torch.float8_e4m3fn)


def _weight(w_codes, w_scales) -> FP8Weight:
    _dev(w_codes, "w_codes", _U8, 2)
    _dev(w_scales, "w_scales", (torch.float32,), 2)
    V, H = w_codes.shape
    return FP8Weight(w_codes.data_ptr(), w_scales.data_ptr(), V, H)


def norm_quant(hidden, residual, norm_weight, eps: float = 1e-6, out=None):
    """Residual add + RMSNorm -> (bf16 recycled hidden, E4M3 codes, fp32 block scales)."""
    _dev(hidden, "hidden", _BF16, 2)
    _dev(residual, "residual", _BF16, 2)
    _dev(norm_weight, "norm_weight", (torch.float32,), 1)
    M, H = hidden.shape
    dev = hidden.device
    if out is None:
        out_h = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
        codes = torch.empty((M, H), dtype=torch.uint8, device=dev)
        scales = torch.empty((M, H // BLOCK if H % BLOCK == 0 else 0), dtype=torch.float32, device=dev)
    else:
        out_h, codes, scales = out
    qa = QAct(codes.data_ptr(), scales.data_ptr(), M, H)
    with torch.cuda.device(dev):
        _check(lib().mtpd_norm_quant(hidden.data_ptr(), residual.data_ptr(), norm_weight.data_ptr(),
                                     float(eps), M, H, out_h.data_ptr(), ctypes.byref(qa), _stream(dev)))
    return out_h, codes, scales


def fp8_lmhead_argmax(codes, scales, w_codes, w_scales, row_index=None, workspace: Workspace | None = None,
                      out=None):
    """Greedy local argmax of the block-scaled FP8 LM head over a packed activation.

    Returns (max float32 [n], idx int32 [n]); idx is local to this weight.
    row_index (int32 [n]) selects activation rows; None means all rows.
    """
    _dev(codes, "codes", _U8, 2)
    _dev(scales, "scales", (torch.float32,), 2)
    w = _weight(w_codes, w_scales)
    dev = codes.device
    A, H = codes.shape
    if row_index is not None:
        _dev(row_index, "row_index", (torch.int32,), 1)
        n = row_index.shape[0]
        ri = row_index.data_ptr()
    else:
        n, ri = A, None
    if out is None:
        out_max = torch.empty((n,), dtype=torch.float32, device=dev)
        out_idx = torch.empty((n,), dtype=torch.int32, device=dev)
    else:
        out_max, out_idx = out
    ws = (workspace or _workspace_for(dev)).get(n)
    qa = QAct(codes.data_ptr(), scales.data_ptr(), A, H)
    with torch.cuda.device(dev):
        _check(lib().mtpd_fp8_lmhead_argmax(ctypes.byref(qa), ri, n, ctypes.byref(w), out_max.data_ptr(),
                                            out_idx.data_ptr(), ws.data_ptr(), ws.numel(), _stream(dev)))
    return out_max, out_idx


def draft_tail(hidden, residual, norm_weight, eps, w_codes, w_scales, workspace: Workspace | None = None,
               out=None):
    """The whole tail: (out_hidden, codes, scales, max, idx) for every row."""
    _dev(hidden, "hidden", _BF16, 2)
    _dev(residual, "residual", _BF16, 2)
    _dev(norm_weight, "norm_weight", (torch.float32,), 1)
    w = _weight(w_codes, w_scales)
    M, H = hidden.shape
    dev = hidden.device
    if out is None:
        out_h = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
        codes = torch.empty((M, H), dtype=torch.uint8, device=dev)
        scales = torch.empty((M, H // BLOCK if H % BLOCK == 0 else 0), dtype=torch.float32, device=dev)
        out_max = torch.empty((M,), dtype=torch.float32, device=dev)
        out_idx = torch.empty((M,), dtype=torch.int32, device=dev)
    else:
        out_h, codes, scales, out_max, out_idx = out
    ws = (workspace or _workspace_for(dev)).get(M)
    qa = QAct(codes.data_ptr(), scales.data_ptr(), M, H)
    with torch.cuda.device(dev):
        _check(lib().mtpd_draft_tail(hidden.data_ptr(), residual.data_ptr(), norm_weight.data_ptr(), float(eps),
                                     M, H, ctypes.byref(w), out_h.data_ptr(), ctypes.byref(qa),
                                     out_max.data_ptr(), out_idx.data_ptr(), ws.data_ptr(), ws.numel(),
                                     _stream(dev)))
    return out_h, codes, scales, out_max, out_idx


def allreduce_norm_quant(partials, residual, norm_weight, eps: float = 1e-6, out=None):
    """norm_quant whose norm input is sum(partials) + residual (fp32, in list order).

    partials: a sequence of 1..16 bf16 [M,H] device tensors (the row-parallel
    partial outputs an all-reduce would sum).  Returns (out_hidden, codes, scales).
    """
    parts = list(partials)
    if not parts:
        raise ValueError("at least one partial is required")
    for i, p in enumerate(parts):
        _dev(p, f"partials[{i}]", _BF16, 2)
        if p.shape != parts[0].shape or p.device != parts[0].device:
            raise ValueError("partials must share shape and device")
    _dev(residual, "residual", _BF16, 2)
    _dev(norm_weight, "norm_weight", (torch.float32,), 1)
    M, H = residual.shape
    dev = residual.device
    if out is None:
        out_h = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
        codes = torch.empty((M, H), dtype=torch.uint8, device=dev)
        scales = torch.empty((M, H // BLOCK if H % BLOCK == 0 else 0), dtype=torch.float32, device=dev)
    else:
        out_h, codes, scales = out
    ptrs = (ctypes.c_void_p * len(parts))(*[p.data_ptr() for p in parts])
    qa = QAct(codes.data_ptr(), scales.data_ptr(), M, H)
    with torch.cuda.device(dev):
        _check(lib().mtpd_allreduce_norm_quant(ptrs, len(parts), residual.data_ptr(), norm_weight.data_ptr(),
                                               float(eps), M, H, out_h.data_ptr(), ctypes.byref(qa), _stream(dev)))
    return out_h, codes, scales


def argmax_combine(local_max, local_idx, shard_offsets, out=None):
    """Global greedy argmax from per-shard local pairs.

    local_max float32 [P, n], local_idx int32 [P, n] (device); shard_offsets:
    P ints, the first global vocab row of each shard.  Returns (max float32 [n],
    idx int32 [n]) with global indices.
    """
    _dev(local_max, "local_max", (torch.float32,), 2)
    _dev(local_idx, "local_idx", (torch.int32,), 2)
    if local_max.shape != local_idx.shape:
        raise ValueError("local_max and local_idx differ in shape")
    P, n = local_max.shape
    offs = [int(o) for o in shard_offsets]
    if len(offs) != P:
        raise ValueError(f"{len(offs)} shard offsets for {P} shards")
    dev = local_max.device
    if out is None:
        out_max = torch.empty((n,), dtype=torch.float32, device=dev)
        out_idx = torch.empty((n,), dtype=torch.int32, device=dev)
    else:
        out_max, out_idx = out
    arr = (ctypes.c_int64 * max(P, 1))(*offs)
    with torch.cuda.device(dev):
        _check(lib().mtpd_argmax_combine(local_max.data_ptr(), local_idx.data_ptr(), arr, P, n,
                                         out_max.data_ptr(), out_idx.data_ptr(), _stream(dev)))
    return out_max, out_idx


def topk_combine(local_val, local_idx, shard_offsets, out=None):
    """Global top-k from per-shard top-k lists.

    local_val float32 [P, n, k], local_idx int32 [P, n, k] (device), each list
    as fp8_lmhead_topk returns it (descending, equal values in index order);
    shard_offsets: P ints, the first global vocab row of each shard.  Returns
    (values float32 [n, k], idx int32 [n, k]) with global indices.
    """
    _dev(local_val, "local_val", (torch.float32,), 3)
    _dev(local_idx, "local_idx", (torch.int32,), 3)
    if local_val.shape != local_idx.shape:
        raise ValueError("local_val and local_idx differ in shape")
    P, n, k = local_val.shape
    offs = [int(o) for o in shard_offsets]
    if len(offs) != P:
        raise ValueError(f"{len(offs)} shard offsets for {P} shards")
    dev = local_val.device
    if out is None:
        out_val = torch.empty((n, k), dtype=torch.float32, device=dev)
        out_idx = torch.empty((n, k), dtype=torch.int32, device=dev)
    else:
        out_val, out_idx = out
    arr = (ctypes.c_int64 * max(P, 1))(*offs)
    with torch.cuda.device(dev):
        _check(lib().mtpd_topk_combine(local_val.data_ptr(), local_idx.data_ptr(), arr, P, n, k,
                                       out_val.data_ptr(), out_idx.data_ptr(), _stream(dev)))
    return out_val, out_idx


def topk_workspace_bytes(n_rows: int, V: int, k: int) -> int:
    return int(lib().mtpd_topk_workspace_bytes(int(n_rows), int(V), int(k)))


_topk_ws: dict = {}


def fp8_lmhead_topk(codes, scales, w_codes, w_scales, k: int, row_index=None, workspace: Workspace | None = None,
                    out=None):
    """Greedy local top-k of the block-scaled FP8 LM head over a packed activation.

    Returns (values float32 [n, k], idx int32 [n, k]), each row in descending
    order of the fp32 logit, equal values in ascending index order.  The
    workspace holds candidate lists and needs no zeroing; by default one
    buffer per device and stream (separate from the argmax workspace) is reused.
    """
    _dev(codes, "codes", _U8, 2)
    _dev(scales, "scales", (torch.float32,), 2)
    w = _weight(w_codes, w_scales)
    dev = codes.device
    A, H = codes.shape
    if row_index is not None:
        _dev(row_index, "row_index", (torch.int32,), 1)
        n = row_index.shape[0]
        ri = row_index.data_ptr()
    else:
        n, ri = A, None
    k = int(k)
    if out is None:
        out_val = torch.empty((n, k), dtype=torch.float32, device=dev)
        out_idx = torch.empty((n, k), dtype=torch.int32, device=dev)
    else:
        out_val, out_idx = out
    if workspace is None:
        key = (dev.type, dev.index, torch.cuda.current_stream(dev).cuda_stream)
        if key not in _topk_ws:
            _topk_ws[key] = Workspace(dev)
        workspace = _topk_ws[key]
    ws = workspace.get_bytes(topk_workspace_bytes(n, w.V, k))
    qa = QAct(codes.data_ptr(), scales.data_ptr(), A, H)
    with torch.cuda.device(dev):
        _check(lib().mtpd_fp8_lmhead_topk(ctypes.byref(qa), ri, n, ctypes.byref(w), k, out_val.data_ptr(),
                                          out_idx.data_ptr(), ws.data_ptr(), ws.numel(), _stream(dev)))
    return out_val, out_idx
