"""Seeded input generators: determinism and the stated recipe."""
import hashlib

import numpy as np

from bit_prefill_gemm_amd import synth


def _h(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()[:16]


def test_seeded_determinism():
    a = synth.make("tiny")
    b = synth.make("tiny")
    assert _h(a["x"]) == _h(b["x"]) and _h(a["w"]) == _h(b["w"])
    c = synth.make("tiny", seed=1)
    assert _h(a["x"]) != _h(c["x"])


def test_tiny_recipe():
    t = synth.make("tiny")
    assert t["x"].dtype == np.float32 and t["x"].shape == (16, 256)
    assert len(t["outlier_channels"]) == 5               # round(0.02 * 256)
    assert t["w"].shape == (128, 8, 18)
    d = t["w"][..., 0:2].copy().view("<f2").astype(np.float64)
    assert d.min() >= 0.005 - 1e-5 and d.max() <= 0.05 + 1e-4
    # outlier channels are 20x wider than the rest
    x = t["x"].astype(np.float64)
    ch = t["outlier_channels"]
    rest = np.setdiff1d(np.arange(256), ch)
    assert np.abs(x[:, ch]).mean() > 8 * np.abs(x[:, rest]).mean()


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -9, 1.0 + 2 ** -9, -2.5, 3.0e38],
                 dtype=np.float32)
    got = synth.bf16_to_f32(synth.bf16_bits(x))
    expect = np.array([1.0, 1.0, 1.0 + 2 ** -7, 1.0, -2.5, np.float32(3.0e38)],  # 1+2^-8 is a tie -> even
                      dtype=np.float32)
    assert np.array_equal(got[:5], expect[:5])
    assert abs(got[5] - x[5]) <= 2 ** -8 * x[5]


def test_weight_codes_are_uniform():
    w = synth.draw_q4_0(np.random.default_rng(0), (256,), 1024, 0.002, 0.02)
    qs = w[..., 2:].reshape(-1)
    nib = np.concatenate([qs & 15, qs >> 4])
    counts = np.bincount(nib, minlength=16)
    assert counts.min() > 0.9 * counts.mean()


def test_moe_routing():
    rng = np.random.default_rng(0)
    tok, exp, off = synth.draw_routing(rng, 512, 128, 8)
    assert off[0] == 0 and off[-1] == 4096 and np.all(np.diff(off) >= 0)
    assert np.array_equal(np.bincount(tok, minlength=512), np.full(512, 8))
    for t in range(0, 512, 37):
        assert len(set(exp[tok == t])) == 8
    for e in range(128):
        seg = slice(off[e], off[e + 1])
        assert np.all(exp[seg] == e)
        assert np.all(np.diff(tok[seg]) > 0)        # stable: tokens ascending
    counts = np.diff(off)
    assert abs(counts.mean() - 32) < 1e-9 and 3 < counts.std() < 9
