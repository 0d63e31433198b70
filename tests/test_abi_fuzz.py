"""Randomized calls of the C ABI's host side (CPU only; hypothesis).

- The plan and sizing queries take any integers, valid or not, without
  crashing; the workspace size is zero exactly where no launch can use one.
- The compute entry points, given random shapes and random pointer choices
  (NULL, misaligned, aliased, or distinct aligned addresses that are never
  dereferenced), always return one of the typed statuses and keep the first
  error's detail.  With no GPU present any call that passes validation stops
  at its first HIP call (MTPD_ERR_HIP), so nothing runs on a device; the test
  is skipped where a GPU is visible.
"""
import ctypes

import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import mtp_draft_head_amd as m
from mtp_draft_head_amd import FP8Weight, QAct

SETTINGS = settings(max_examples=300, deadline=None, suppress_health_check=[HealthCheck.too_slow])
STATUSES = set(range(7))
A = 0x10000000   # fake device addresses, 16 MiB apart

ints = st.one_of(st.integers(min_value=-3, max_value=300), st.sampled_from([128, 256, 6144, 8192, 8320, 18944,
                                                                           151552, 1 << 31, (1 << 31) + 128,
                                                                           1 << 40, -(1 << 40)]))


@pytest.fixture(scope="module")
def L():
    return m.lib()


@SETTINGS
@given(ints, ints, ints, st.integers(min_value=-2, max_value=40))
def test_plan_and_size_queries_take_any_integers(L, n, V, H, k):
    assert isinstance(L.mtpd_lmhead_plan(n, V, H), bytes)
    assert isinstance(L.mtpd_draft_tail_plan(n, V, H), bytes)
    wb = L.mtpd_workspace_bytes(n)
    assert wb == 0 if n <= 0 or n > (1 << 24) else wb > 0   # no workspace beyond 2^24 rows
    assert L.mtpd_topk_workspace_bytes(n, V, k) >= 0


def _ptr(choice, slot):
    # 0: NULL, 1: misaligned, 2: slot 0 (aliases every other slot-0 pointer), 3: a slot of its own
    return [None, A + (slot << 24) + 4, A, A + (slot << 24)][choice]


ptr_choice = st.integers(min_value=0, max_value=3)


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="fake device pointers must never reach a GPU")
@SETTINGS
@given(st.integers(min_value=-2, max_value=70), st.sampled_from([0, 64, 128, 256, 384, 8192, 8320]),
       st.sampled_from([0, 128, 256, 1000, 18944]), st.lists(ptr_choice, min_size=12, max_size=12),
       st.sampled_from([0, 1, 1 << 20]))
def test_entry_points_return_typed_statuses(L, M, H, V, p, ws_bytes):
    L.mtpd_clear_error()
    act = QAct(_ptr(p[0], 1), _ptr(p[1], 2), max(M, 0), H)
    w = FP8Weight(_ptr(p[2], 3), _ptr(p[3], 4), V, H)
    s1 = L.mtpd_draft_tail(_ptr(p[4], 5), _ptr(p[5], 6), _ptr(p[6], 7), 1e-6, M, H, ctypes.byref(w),
                           _ptr(p[7], 8), ctypes.byref(act), _ptr(p[8], 9), _ptr(p[9], 10), _ptr(p[10], 11),
                           ws_bytes, None)
    assert s1 in STATUSES
    first = L.mtpd_last_error()
    assert (first == b"") == (s1 == 0)
    s2 = L.mtpd_fp8_lmhead_argmax(ctypes.byref(act), _ptr(p[11], 12), M, ctypes.byref(w), _ptr(p[8], 9),
                                  _ptr(p[9], 10), _ptr(p[10], 11), ws_bytes, None)
    assert s2 in STATUSES
    s3 = L.mtpd_norm_quant(_ptr(p[4], 5), _ptr(p[5], 6), _ptr(p[6], 7), 1e-6, M, H, _ptr(p[7], 8),
                           ctypes.byref(act), None)
    assert s3 in STATUSES
    if s1 != 0:
        assert L.mtpd_last_error() == first   # the first failure's detail is kept
    if M == 0 and s1 == 0:
        assert s2 in (0, 1, 2, 3, 4, 5)       # nothing to launch: never a HIP error


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="fake device pointers must never reach a GPU")
@SETTINGS
@given(st.integers(min_value=-2, max_value=70), st.integers(min_value=-2, max_value=300),
       st.integers(min_value=-2, max_value=40),
       st.lists(st.sampled_from([0, 128, 18944, (1 << 31) - 128, 1 << 31, -128]), min_size=0, max_size=70),
       st.lists(ptr_choice, min_size=4, max_size=4))
def test_combine_entry_points_return_typed_statuses(L, S, n, k, offs, p):
    """Both vocab-shard combines, under random shard counts, row counts, k,
    host offsets (short arrays included) and pointer choices."""
    L.mtpd_clear_error()
    arr = (ctypes.c_int64 * max(S, len(offs), 1))(*(offs + [0] * max(0, S - len(offs))))
    s1 = L.mtpd_argmax_combine(_ptr(p[0], 1), _ptr(p[1], 2), arr, S, n, _ptr(p[2], 3), _ptr(p[3], 4), None)
    assert s1 in STATUSES
    s2 = L.mtpd_topk_combine(_ptr(p[0], 1), _ptr(p[1], 2), arr, S, n, k, _ptr(p[2], 3), _ptr(p[3], 4), None)
    assert s2 in STATUSES
    if not 1 <= S <= 64 or not 0 <= n <= (1 << 24):
        assert s1 == 2 and s2 == 2
    if not 1 <= k <= 32 and 1 <= S <= 64 and 0 <= n <= (1 << 24):
        assert s2 == 2
