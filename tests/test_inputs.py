"""The seeded workload generator: determinism, shapes and the documented recipe."""
import numpy as np

from mtp_draft_head_amd import inputs


def test_tiny_is_deterministic_and_shaped():
    a = inputs.make("tiny")
    b = inputs.make("tiny")
    for k in ("hidden", "residual", "norm_weight", "w_codes", "w_scales"):
        assert np.array_equal(a[k], b[k])
    assert a["hidden"].shape == (4, 256) and a["hidden"].dtype == np.uint16
    assert a["w_codes"].shape == (1024, 256) and a["w_scales"].shape == (8, 2)
    assert a["eps"] == 1e-6
    assert len(a["meta"]["ties"]) == 2


def test_shard_weight_is_prefix_of_full_vocab_weight():
    c2, s2 = inputs.weight_family(6144, 151552, n_blocks=3)
    c1, s1 = inputs.weight_family(6144, 151552, n_blocks=1)
    assert np.array_equal(c2[:128], c1) and np.array_equal(s2[:1], s1)
    # no NaN codes, scales = amax/448 of an N(0, 0.02) draw (~4.5 sigma / 448)
    assert not np.any((c2 & 0x7F) == 0x7F)
    assert np.all((s2 > 0.05 / 448) & (s2 < 0.2 / 448))
    # every block holds a +-448 code
    blk = (c2.reshape(3, 128, 48, 128) & 0x7F).max(axis=(1, 3))
    assert np.all(blk == 0x7E)


def test_outlier_channels():
    d = inputs.make("decode_c1_tp8_shard")
    outl = d["meta"]["outliers"]
    assert len(outl) == 61 and len(set(outl.tolist())) == 61
    h = d["hidden"].view(np.int16).astype(np.int32) << 16
    hv = h.astype(np.uint32).view(np.float32)[0]
    assert np.abs(hv[outl]).mean() > 10 * np.abs(np.delete(hv, outl)).mean()
    assert d["w_codes"].shape == (18944, 6144)
