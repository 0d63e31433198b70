"""Pins for the oracle's E4M3FN and bfloat16 codecs.

The oracle's codecs are written from the format definitions; here they are
checked against torch's own float8_e4m3fn / bfloat16 casts (an independent
library routine), exhaustively where the space is small, on every rounding
boundary, and on a strided sweep of fp32 bit patterns.  torch's e4m3fn cast
maps overflow to NaN instead of saturating, so inputs are clamped to +-448
before it is called and saturation is pinned separately.
"""
import numpy as np
import pytest
import torch

import oracle


def torch_e4m3(x32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.clip(x32, -448.0, 448.0).astype(np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def torch_bf16(x32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(x32.astype(np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_e4m3_decode_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_e4m3_format_constants(tmp_path):
    # closed forms of the OCP E4M3FN layout (1-4-3, bias 7, no infinities)
    dec = oracle.e4m3_decode
    assert dec(np.uint8(0x7E)) == 448.0
    assert dec(np.uint8(0x01)) == 2.0 ** -9          # smallest subnormal
    assert dec(np.uint8(0x07)) == 7 * 2.0 ** -9      # largest subnormal
    assert dec(np.uint8(0x08)) == 2.0 ** -6          # smallest normal
    assert dec(np.uint8(0x38)) == 1.0
    assert dec(np.uint8(0xFE)) == -448.0


def _finite_e4m3_values():
    codes = np.arange(0x7F, dtype=np.uint8)          # 0x00 .. 0x7E, the non-negative finite codes
    vals = oracle.e4m3_decode(codes)
    return codes, vals


def test_e4m3_encode_exact_values_roundtrip():
    codes, vals = _finite_e4m3_values()
    assert np.array_equal(oracle.e4m3_encode(vals), codes)
    assert np.array_equal(oracle.e4m3_encode(-vals[1:]), codes[1:] | 0x80)


def test_e4m3_encode_rounding_boundaries_f64():
    """At, just below and just above every midpoint, in fp64 (not representable in fp32)."""
    codes, vals = _finite_e4m3_values()
    lo, hi = vals[:-1], vals[1:]
    mid = (lo + hi) / 2                      # exact in fp64
    even = np.where(codes[:-1] % 2 == 0, codes[:-1], codes[1:])
    assert np.array_equal(oracle.e4m3_encode(mid), even)
    below = mid - (hi - lo) * 2.0 ** -30
    above = mid + (hi - lo) * 2.0 ** -30
    assert np.array_equal(oracle.e4m3_encode(below), codes[:-1])
    assert np.array_equal(oracle.e4m3_encode(above), codes[1:])
    # negative side mirrors
    assert np.array_equal(oracle.e4m3_encode(-mid), even | 0x80)


def test_e4m3_encode_boundaries_vs_torch():
    codes, vals = _finite_e4m3_values()
    mid = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)      # midpoints are fp32-exact
    pts = np.concatenate([mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(np.inf)),
                          vals.astype(np.float32)])
    pts = np.concatenate([pts, -pts])
    assert np.array_equal(oracle.e4m3_encode(pts.astype(np.float64)), torch_e4m3(pts))


def test_e4m3_encode_fp32_sweep_vs_torch():
    # every 61st fp32 bit pattern with magnitude in [0, 448] (about 18M per sign)
    top = np.float32(448.0).view(np.uint32)
    bits = np.arange(0, int(top) + 1, 61, dtype=np.uint32)
    x = bits.view(np.float32)
    x = np.concatenate([x, -x])
    assert np.array_equal(oracle.e4m3_encode(x.astype(np.float64)), torch_e4m3(x))


def test_e4m3_encode_saturates_and_keeps_sign():
    big = np.array([448.0, 463.99, 464.0, 465.0, 480.0, 1e6, 1e300, np.inf])
    assert np.all(oracle.e4m3_encode(big) == 0x7E)
    assert np.all(oracle.e4m3_encode(-big) == 0xFE)
    assert oracle.e4m3_encode(np.array([-1e-9]))[0] == 0x80
    assert oracle.e4m3_encode(np.array([-0.0]))[0] == 0x80
    assert oracle.e4m3_encode(np.array([0.5 * 2.0 ** -9]))[0] == 0x00      # tie to even (0)
    assert oracle.e4m3_encode(np.array([1.5 * 2.0 ** -9]))[0] == 0x02      # tie to even (2)
    assert oracle.e4m3_encode(np.array([np.nan]))[0] == 0x7F


def test_bf16_decode_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.bf16_decode(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_bf16_encode_fp32_sweep_vs_torch():
    rng = np.random.default_rng(7)
    # strided sweep over all finite fp32 patterns, plus every pattern whose low
    # half is at or next to the rounding midpoint 0x8000
    bits = np.arange(0, 0x7F800000, 4099, dtype=np.uint32)
    hi = rng.integers(0, 0x7F80, size=200000, dtype=np.uint32) << 16
    ties = np.concatenate([hi | 0x8000, hi | 0x7FFF, hi | 0x8001])
    x = np.concatenate([bits, ties]).view(np.float32)
    x = np.concatenate([x, -x])
    assert np.array_equal(oracle.bf16_encode(x.astype(np.float64)), torch_bf16(x))


def test_bf16_encode_f64_midpoints():
    rng = np.random.default_rng(8)
    hi = rng.integers(0x0080, 0x7F7F, size=100000, dtype=np.uint32)   # normal, finite
    lo_v = (hi << 16).view(np.float32).astype(np.float64)
    up_v = ((hi + 1) << 16).view(np.float32).astype(np.float64)
    mid = (lo_v + up_v) / 2
    even = np.where(hi % 2 == 0, hi, hi + 1).astype(np.uint16)
    assert np.array_equal(oracle.bf16_encode(mid), even)
    assert np.array_equal(oracle.bf16_encode(mid - (up_v - lo_v) * 2.0 ** -40), hi.astype(np.uint16))
    assert np.array_equal(oracle.bf16_encode(mid + (up_v - lo_v) * 2.0 ** -40), (hi + 1).astype(np.uint16))
