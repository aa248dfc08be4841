"""Pins of the oracle's MoE glue (the expert layer around the grouped product):
the fp32 exponential and SwiGLU of the reading, the SwiGLU -> rotate ->
quantize step, the expert sort and the weighted combine."""
import math

import numpy as np
import pytest

import oracle


def test_exp_f32_matches_libm_within_a_few_ulp():
    xs = np.linspace(-87.0, 88.0, 20001, dtype=np.float64).astype(np.float32)
    got = oracle.exp_f32(xs).astype(np.float64)
    ref = np.exp(xs.astype(np.float64))
    rel = np.abs(got / ref - 1.0)
    assert rel.max() < 3e-7, rel.max()


def test_exp_f32_special_values():
    assert oracle.exp_f32(np.float32([0.0]))[0] == 1.0
    # arguments that reduce to r = 0 (x = n ln2 in fp32): a power of two up to
    # the rounding of x itself
    for n in (-60, -3, 1, 5, 90):
        x = float(np.float32(n * math.log(2.0)))
        v = float(oracle.exp_f32(np.float32([x]))[0])
        assert abs(v / math.exp(x) - 1.0) < 2e-7
        assert abs(v / 2.0 ** n - 1.0) < abs(n) * 1e-7
    # clamping keeps the extremes finite and positive
    big = oracle.exp_f32(np.float32([1000.0, -1000.0]))
    assert np.all(np.isfinite(big)) and np.all(big > 0)


def test_silu_against_formula_and_identity():
    g = np.linspace(-30.0, 30.0, 6001, dtype=np.float64).astype(np.float32)
    s = oracle.silu_f32(g).astype(np.float64)
    g64 = g.astype(np.float64)
    ref = g64 / (1.0 + np.exp(-g64))
    assert np.all(np.abs(s - ref) <= 1e-6 * np.abs(ref) + 1e-30)
    # silu(g) - silu(-g) = g
    sn = oracle.silu_f32(-g).astype(np.float64)
    assert np.allclose(s - sn, g64, rtol=1e-6, atol=1e-6)
    assert oracle.silu_f32(np.float32([0.0]))[0] == 0.0


def _gu(rng, rows, inter, gate_scale=2.0):
    g = (rng.standard_normal((rows, inter)) * gate_scale).astype(np.float32)
    u = rng.standard_normal((rows, inter)).astype(np.float32)
    return np.concatenate([g, u], axis=1), g, u


@pytest.mark.parametrize("bits", [4, 8])
def test_swiglu_quantize_reduces_to_quantize_when_gate_saturates(bits):
    """For gate >= 20, e^-g < 3e-9 and 1 + e^-g rounds to 1, so silu(g) = g
    exactly: the step is the activation quantizer applied to g * u."""
    rng = np.random.default_rng(3)
    rows, inter = 5, 96
    gu, g, u = _gu(rng, rows, inter)
    gu[:, :inter] = 20.0 + np.abs(g)
    h = (gu[:, :inter] * gu[:, inter:]).astype(np.float32)
    q, d, _ = oracle.swiglu_quantize(gu, inter, bits)
    q2, d2, _ = oracle.quantize(h, bits)
    assert np.array_equal(q, q2) and np.array_equal(d.view(np.uint32), d2.view(np.uint32))


def test_swiglu_quantize_matches_its_definition_step_by_step():
    rng = np.random.default_rng(4)
    rows, inter = 3, 64
    gu, g, u = _gu(rng, rows, inter)
    h = (oracle.silu_f32(g) * u).astype(np.float32)
    q, d, _ = oracle.swiglu_quantize(gu, inter, 4)
    q2, d2, _ = oracle.quantize(h, 4)
    assert np.array_equal(q, q2) and np.array_equal(d.view(np.uint32), d2.view(np.uint32))
    # zero up projection: all codes 0, scale 0
    gu0 = gu.copy()
    gu0[:, inter:] = 0.0
    q0, d0, _ = oracle.swiglu_quantize(gu0, inter, 4)
    assert not q0.any() and not d0.any()
    # gate and up are not interchangeable
    qs, _, _ = oracle.swiglu_quantize(np.concatenate([gu[:, inter:], gu[:, :inter]], axis=1),
                                      inter, 4)
    assert not np.array_equal(qs, q)


def test_swiglu_quantize_leading_dimension():
    rng = np.random.default_rng(5)
    rows, inter = 4, 32
    gu, _, _ = _gu(rng, rows, inter)
    wide = np.zeros((rows, 2 * inter + 32), dtype=np.float32)
    wide[:, :2 * inter] = gu
    wide[:, 2 * inter:] = 1e30   # past the two projections: never read
    assert np.array_equal(oracle.swiglu_quantize(wide, inter, 4)[0],
                          oracle.swiglu_quantize(gu, inter, 4)[0])


def test_route_sort_invariants():
    rng = np.random.default_rng(6)
    tokens, topk, experts = 37, 4, 9
    e = np.stack([rng.choice(experts, topk, replace=False) for _ in range(tokens)]).ravel()
    off, row_entry, slot_of = oracle.route_sort(e, experts)
    assert np.array_equal(np.diff(off), np.bincount(e, minlength=experts))
    assert off[0] == 0 and off[-1] == e.size
    se = e[row_entry]
    assert np.all(np.diff(se) >= 0)
    for x in range(experts):   # stable: entries ascend inside an expert
        seg = row_entry[off[x]:off[x + 1]]
        assert np.all(np.diff(seg) > 0)
        assert np.all(e[seg] == x)
    assert np.array_equal(slot_of[row_entry], np.arange(e.size))
    assert np.array_equal(np.sort(row_entry), np.arange(e.size))


def test_combine_one_hot_and_sum():
    rng = np.random.default_rng(7)
    tokens, topk, hidden = 6, 3, 40
    n = tokens * topk
    dn = rng.standard_normal((n, hidden)).astype(np.float32)
    slot = rng.permutation(n).astype(np.int32)
    w = np.zeros(n, dtype=np.float32)
    w[::topk] = 1.0                         # choice 0 only
    out = oracle.moe_combine(dn, slot, w, tokens, topk)
    assert np.array_equal(out, dn[slot[::topk]])
    w = rng.random(n).astype(np.float32)
    out = oracle.moe_combine(dn, slot, w, tokens, topk)
    ref = (w.reshape(tokens, topk, 1).astype(np.float64) *
           dn[slot].reshape(tokens, topk, hidden).astype(np.float64)).sum(axis=1)
    assert np.allclose(out, ref, rtol=1e-5, atol=1e-6)


def test_combine_accumulates_in_fp32_in_choice_order():
    """1e8 + 1 rounds back to 1e8 in fp32: the fma chain in choice order gives
    0 where an fp64 sum gives 1."""
    dn = np.array([[1e8], [1.0], [-1e8]], dtype=np.float32)
    slot = np.array([0, 1, 2], dtype=np.int32)
    w = np.array([1.0, 1.0, 1.0], dtype=np.float32)
    assert oracle.moe_combine(dn, slot, w, 1, 3)[0, 0] == 0.0
    slot = np.array([0, 2, 1], dtype=np.int32)   # 1e8 - 1e8 first: the 1 survives
    assert oracle.moe_combine(dn, slot, w, 1, 3)[0, 0] == 1.0
