"""Pins of the oracle's longer rotations (H64, H128 over spans of 64 or 128
values, per-32 quantization unchanged)."""
import numpy as np
import pytest

import oracle


def sylvester(n):
    h = np.array([[1.0]])
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


@pytest.mark.parametrize("n", [32, 64, 128])
def test_rotation_is_the_sylvester_matrix(n):
    rng = np.random.default_rng(n)
    x = rng.standard_normal((5, 2 * n))
    v = oracle.rotate_n_f64(x, n)
    ref = (x.reshape(-1, n) @ sylvester(n).T / np.sqrt(n)).reshape(x.shape)
    assert np.allclose(v, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("n", [64, 128])
def test_rotation_f32_close_to_f64(n):
    rng = np.random.default_rng(n + 1)
    x = rng.standard_normal((7, 4 * n)).astype(np.float32)
    v32 = oracle.rotate_n_f32(x, n).astype(np.float64)
    v64 = oracle.rotate_n_f64(x.astype(np.float64), n)
    assert np.abs(v32 - v64).max() <= 1e-5 * np.abs(v64).max()


@pytest.mark.parametrize("n", [64, 128])
def test_rotation_preserves_dot_products_and_is_an_involution(n):
    rng = np.random.default_rng(n + 2)
    x = rng.standard_normal((3, 2 * n))
    w = rng.standard_normal((3, 2 * n))
    hx, hw = oracle.rotate_n_f64(x, n), oracle.rotate_n_f64(w, n)
    assert np.allclose((x * w).sum(axis=1), (hx * hw).sum(axis=1), rtol=1e-12)
    assert np.allclose(oracle.rotate_n_f64(hx, n), x, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("n", [32, 64, 128])
def test_one_outlier_spreads_evenly(n):
    """A span holding a single value c becomes +-c/sqrt(n) everywhere."""
    x = np.zeros((1, n))
    x[0, 5] = 3.0
    v = oracle.rotate_n_f64(x, n)
    assert np.allclose(np.abs(v), 3.0 / np.sqrt(n))


def test_n64_is_h2_kron_h32():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((1, 64))
    a, b = oracle.rotate_n_f64(x[:, :32], 32), oracle.rotate_n_f64(x[:, 32:], 32)
    ref = np.concatenate([a + b, a - b], axis=1) / np.sqrt(2.0)
    assert np.allclose(oracle.rotate_n_f64(x, 64), ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("bits", [4, 8])
def test_quantize_rot_reduces_to_the_route_and_to_no_rotation(bits):
    rng = np.random.default_rng(10 + bits)
    x = rng.standard_normal((6, 256)).astype(np.float32)
    q, d, _ = oracle.quantize_rot(x, 32, bits)
    q2, d2, _ = oracle.quantize(x, bits)
    assert np.array_equal(q, q2) and np.array_equal(d.view(np.uint32), d2.view(np.uint32))
    q, d, _ = oracle.quantize_rot(x, 0, bits)
    q2, d2, _ = oracle.quantize(x, bits, rotate=False)
    assert np.array_equal(q, q2) and np.array_equal(d.view(np.uint32), d2.view(np.uint32))


@pytest.mark.parametrize("n", [64, 128])
def test_quantize_rot_is_rotation_then_per_32_quantization(n):
    rng = np.random.default_rng(n + 11)
    x = rng.standard_normal((4, 2 * n)).astype(np.float32)
    v = oracle.rotate_n_f32(x, n)
    q, d, _ = oracle.quantize_rot(x, n, 4)
    q2, d2, _ = oracle.quantize(v, 4, rotate=False)
    assert np.array_equal(q, q2) and np.array_equal(d.view(np.uint32), d2.view(np.uint32))


def test_weight_quantizer_rot():
    rng = np.random.default_rng(12)
    w = (rng.standard_normal((8, 256)) * 0.03).astype(np.float32)
    assert np.array_equal(oracle.quantize_weights_q4_0_rot(w, 32),
                          oracle.quantize_weights_q4_0(w, rotate=True))
    assert np.array_equal(oracle.quantize_weights_q4_0_rot(w, 0),
                          oracle.quantize_weights_q4_0(w, rotate=False))
    for n in (64, 128):
        blocks = oracle.quantize_weights_q4_0_rot(w, n)
        wq, dw = oracle.q4_0_decode(blocks, 256)
        deq = wq * np.repeat(dw, 32, axis=1)
        # the blocks hold H_n w / sqrt(n) to within half a step per value
        ref = oracle.rotate_n_f64(w.astype(np.float64), n)
        assert np.all(np.abs(deq - ref) <= 0.5 * np.repeat(dw, 32, axis=1) + 1e-12)
