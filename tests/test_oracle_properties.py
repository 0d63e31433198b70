"""Property tests of the oracle (hypothesis; CPU only).

Randomized checks of what the format definitions and the algebra fix, each
against a method other than the oracle's own:
  - E4M3 packing is the nearest finite E4M3 value of the clamped input, ties
    to the even code, found here by searching the 254 finite values torch's
    float8_e4m3fn decodes (OCP E4M3FN; "[Quant][MTP] Reuse packed FP8 logits
    inputs", Purpose: the packed activation);
  - bf16 rounding is the nearer of the two bf16 neighbours, ties to even,
    found from float32 bit patterns;
  - the RMSNorm with eps = 0 is invariant under scaling the row by a power of
    two (codes, scales and the bf16 hidden unchanged);
  - the logits are linear in the weight scales and follow a permutation of
    the weight rows; the argmax is the first maximum of the fp32 logits.
"""
import numpy as np
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle

SETTINGS = settings(max_examples=60, deadline=None, suppress_health_check=[HealthCheck.too_slow])

# the finite E4M3FN values by code, from torch (not from the oracle)
_CODES = np.arange(256, dtype=np.uint8)
_VALUES = torch.from_numpy(_CODES.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
_FINITE = [(int(c), float(v)) for c, v in zip(_CODES, _VALUES) if np.isfinite(v)]


def _nearest_e4m3(x: float) -> float:
    x = min(max(x, -448.0), 448.0)
    best = None
    for c, v in _FINITE:
        d = abs(v - x)
        if best is None or d < best[0] or (d == best[0] and (c & 1) == 0 and (best[1] & 1) == 1):
            best = (d, c, v)
    return best[2]


finite_doubles = st.one_of(
    st.floats(min_value=-1000.0, max_value=1000.0, allow_nan=False, allow_infinity=False),
    st.floats(min_value=-2.0 ** -5, max_value=2.0 ** -5, allow_nan=False, allow_infinity=False),
    st.integers(min_value=-460 * 64, max_value=460 * 64).map(lambda k: k / 64.0),
)


@SETTINGS
@given(st.lists(finite_doubles, min_size=1, max_size=64))
def test_e4m3_is_nearest_even(xs):
    codes = oracle.e4m3_encode(np.array(xs, np.float64))
    got = _VALUES[codes]
    want = np.array([_nearest_e4m3(x) for x in xs])
    assert np.array_equal(got, want), (xs, got, want)


def _bf16_nearest_even(x: float) -> float:
    """The bf16 value nearest x, ties to the even pattern: x's float32 rounding
    truncated to bf16 and its two bf16 neighbours bracket x; pick among them."""
    t = int(np.array([np.float32(x)]).view(np.uint32)[0]) & 0xFFFF0000
    best = None
    for b in (t - 0x10000, t, t + 0x10000):
        if not 0 <= b <= 0xFFFFFFFF:
            continue
        v = float(np.array([b], np.uint32).view(np.float32)[0])
        if not np.isfinite(v):
            continue
        key = (abs(v - x), (b >> 16) & 1)
        if best is None or key < best[0]:
            best = (key, v)
    return best[1]


@SETTINGS
@given(st.lists(st.floats(min_value=-1e30, max_value=1e30, allow_nan=False, allow_infinity=False)
                .filter(lambda v: v == 0.0 or abs(v) > 1e-30), min_size=1, max_size=32))
def test_bf16_is_nearest_even(xs):
    got = oracle.bf16_decode(oracle.bf16_encode(np.array(xs, np.float64)))
    for x, g in zip(xs, got):
        assert g == _bf16_nearest_even(x), (x, g)


def _bf16_bits(a):
    return oracle.bf16_encode(np.asarray(a, np.float64))


@SETTINGS
@given(st.integers(min_value=1, max_value=3), st.integers(min_value=1, max_value=4),
       st.integers(min_value=-6, max_value=6), st.integers(min_value=0, max_value=2 ** 31 - 1))
def test_norm_invariant_under_power_of_two_scaling(M, nb, k, seed):
    """eps = 0: rstd(2^k s) = 2^-k rstd(s) exactly, so y, and with it the bf16
    hidden, the codes and the scales, do not change."""
    H = 128 * nb
    rng = np.random.default_rng(seed)
    h = _bf16_bits(rng.normal(0, 1, (M, H)))
    r = _bf16_bits(rng.normal(0, 1, (M, H)))
    g = rng.uniform(0.5, 1.5, H).astype(np.float32)
    h2 = _bf16_bits(oracle.bf16_decode(h) * 2.0 ** k)
    r2 = _bf16_bits(oracle.bf16_decode(r) * 2.0 ** k)
    a = oracle.norm_quant(h, r, g, 0.0)
    b = oracle.norm_quant(h2, r2, g, 0.0)
    assert np.array_equal(a["hidden"], b["hidden"])
    assert np.array_equal(a["codes"], b["codes"])
    assert np.array_equal(a["scales"], b["scales"])


@SETTINGS
@given(st.integers(min_value=1, max_value=3), st.integers(min_value=1, max_value=3),
       st.integers(min_value=1, max_value=3), st.integers(min_value=0, max_value=2 ** 31 - 1))
def test_logits_linear_in_weight_scales_and_follow_row_permutations(M, nb, vb, seed):
    H, V = 128 * nb, 128 * vb
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, (M, H), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0   # no NaN codes
    scales = rng.uniform(0.01, 1.0, (M, nb)).astype(np.float32)
    wq = rng.integers(0, 256, (V, H), dtype=np.uint8)
    wq[(wq & 0x7F) == 0x7F] = 0
    ws = rng.uniform(0.01, 1.0, (vb, nb)).astype(np.float32)
    z = oracle.logits(codes, scales, wq, ws)
    assert np.array_equal(oracle.logits(codes, scales, wq, ws * np.float32(2.0)), 2.0 * z)
    perm = np.concatenate([rng.permutation(128) + 128 * j for j in range(vb)])   # rows stay in their scale block
    assert np.array_equal(oracle.logits(codes, scales, wq[perm], ws), z[:, perm])
    am = oracle.argmax(codes, scales, wq, ws)
    z32 = z.astype(np.float32)
    assert np.array_equal(am["idx"], np.argmax(z32, axis=1).astype(np.int32))
    assert np.array_equal(am["max"], z32.max(axis=1))
