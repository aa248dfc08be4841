"""Pins for the CPU oracle: each check ties it to something other than itself.

Pins used: closed forms, the invariants the pages state, reductions to numpy
library routines, IEEE reference conversions, brute force with the dense
Hadamard matrix, and hand-written fixtures under tests/golden/.  A plausible
slip anywhere in the oracle (wrong butterfly pairing or sign, a transposed
operand, a wrong block index, a dropped scale, a wrong tie rule) fails at
least one of them.
"""
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

import oracle
from bit_prefill_gemm_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def sylvester_h32() -> np.ndarray:
    """Dense Sylvester Hadamard matrix from its definition (-1)^popcount(i & j)."""
    i = np.arange(32)[:, None]
    j = np.arange(32)[None, :]
    bits = np.vectorize(lambda v: bin(int(v)).count("1"))(i & j)
    return np.where(bits % 2 == 0, 1.0, -1.0)


H = sylvester_h32()


def rotate_dense_f64(x: np.ndarray) -> np.ndarray:
    xb = x.reshape(-1, 32).astype(np.float64)
    return (xb @ H.T / np.sqrt(32.0)).reshape(x.shape)


# ----------------------------------------------------------------- constants

def test_h32_is_hadamard():
    assert np.array_equal(H @ H, 32 * np.eye(32))
    assert np.array_equal(H, H.T)
    assert np.all(H[0] == 1)


def test_inv_sqrt32_is_correctly_rounded():
    getcontext().prec = 80
    exact = Fraction(Decimal(2).sqrt() / Decimal(8))
    c = oracle.inv_sqrt32_f32()
    lo = np.nextafter(c, np.float32(0))
    hi = np.nextafter(c, np.float32(1))
    err = abs(Fraction(float(c)) - exact)
    assert err <= abs(Fraction(float(lo)) - exact)
    assert err <= abs(Fraction(float(hi)) - exact)
    assert int(np.float32(c).view(np.uint32)) == 0x3E3504F3


# ----------------------------------------------------------------- rotation

def test_rotation_of_unit_vectors_is_sylvester_column():
    """Butterflies on e_j produce only sums of +-1 and 0, so the result is exact."""
    c = oracle.inv_sqrt32_f32()
    for j in range(32):
        e = np.zeros(32, dtype=np.float32)
        e[j] = 1.0
        v = oracle.rotate_f32(e)
        expect = (H[:, j] * np.float64(c)).astype(np.float32)
        assert np.array_equal(v, expect), j


def test_rotation_f32_close_to_dense_matrix():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((4000, 32)).astype(np.float32) * 3
    v = oracle.rotate_f32(x).astype(np.float64)
    ref = rotate_dense_f64(x)
    # five butterfly stages and one scaling, each one fp32 rounding
    bound = 6 * 2.0 ** -24 * np.abs(x).astype(np.float64).sum(axis=1, keepdims=True)
    assert np.all(np.abs(v - ref) <= bound)


def test_rotation_f64_matches_dense_matrix():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((500, 32))
    assert np.allclose(oracle.rotate_f64(x), rotate_dense_f64(x), rtol=0, atol=1e-14)


@pytest.mark.parametrize("k", [32, 256, 5120, 17408])
def test_rotation_preserves_dot_products(k):
    """x . w = (Hx) . (Hw), from "The rotation" section of the H32 post."""
    rng = np.random.default_rng(k)
    x = rng.standard_normal(k)
    w = rng.standard_normal(k)
    lhs = float(x @ w)
    rhs = float(oracle.rotate_f64(x) @ oracle.rotate_f64(w))
    assert abs(lhs - rhs) <= 1e-12 * np.linalg.norm(x) * np.linalg.norm(w)


def test_rotation_is_an_involution():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((64, 32))
    assert np.allclose(oracle.rotate_f64(oracle.rotate_f64(x)), x, rtol=0, atol=1e-14)


# ----------------------------------------------------------------- fp16

def test_fp16_conversions_match_ieee():
    rng = np.random.default_rng(4)
    vals = np.concatenate([
        rng.uniform(-70000, 70000, 3000),
        rng.uniform(-1, 1, 3000) * 1e-4,
        rng.uniform(-1, 1, 3000) * 1e-7,           # subnormal range
        np.array([0.0, -0.0, 65504.0, 65520.0, 65519.99, 1e6, 2.0 ** -24, 2.0 ** -25,
                  3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -25, 1.0 + 2.0 ** -11,
                  1.0 + 3 * 2.0 ** -11, 2047.0, 2049.0, 0.1, 0.002, 0.02, 0.005]),
    ])
    for v in vals:
        with np.errstate(over="ignore"):
            ref = int(np.float16(v).view(np.uint16))   # numpy casts double->half with RNE
        got = oracle.f64_to_f16(v)
        assert got == ref, (v, hex(got), hex(ref))
    for h in range(0, 0x7C00, 7):
        assert oracle.f16_to_f64(h) == float(np.uint16(h).view(np.float16))
        assert oracle.f16_to_f64(h | 0x8000) == float(np.uint16(h | 0x8000).view(np.float16))


# ----------------------------------------------------------------- Q4_0

def test_q4_0_code_flip_table():
    rows = [ln.split() for ln in open(os.path.join(GOLDEN, "q4_0_flip.txt"))
            if ln.strip() and not ln.startswith("#")]
    assert len(rows) == 16
    blk = np.zeros((1, 1, 18), dtype=np.uint8)
    blk[0, 0, 0:2] = np.array([1.0], dtype="<f2").view(np.uint8)
    for j in range(16):
        blk[0, 0, 2 + j] = j | ((15 - j) << 4)
    w, dw = oracle.q4_0_decode(blk, 32)
    assert dw[0, 0] == 1.0
    for code, value, nib in rows:
        code, value = int(code), int(value)
        twos = int(nib, 2)
        sext = twos - 16 if twos & 8 else twos
        assert sext == value
        assert (code ^ 8) == twos
        assert w[0, code] == value            # low nibble of byte `code`
        assert w[0, 16 + 15 - code] == value  # high nibble of byte 15-code
        # the same value scaled by 16 sits in the top nibble of an int8
        assert np.int8(np.uint8(((code ^ 8) << 4) & 0xFF)) == 16 * value


def test_q4_0_decode_layout_and_scale():
    d = synth.draw_q4_0(np.random.default_rng(5), (3,), 64, 0.01, 0.02)
    w, dw = oracle.q4_0_decode(d, 64)
    for r in range(3):
        for b in range(2):
            blk = d[r, b]
            assert dw[r, b] == float(blk[0:2].view("<f2")[0])
            for j in range(16):
                assert w[r, 32 * b + j] == (int(blk[2 + j]) & 15) - 8
                assert w[r, 32 * b + 16 + j] == (int(blk[2 + j]) >> 4) - 8


# ----------------------------------------------------------------- quantizer

def test_quantize_constant_block_closed_form():
    c = oracle.inv_sqrt32_f32()
    for a in [1.0, -3.25, 0.0078125, 1000.0, -1e-20]:
        x = np.full((1, 32), a, dtype=np.float32)
        q, d, _ = oracle.quantize(x, 4)
        v0 = np.float32(np.float32(32 * a) * c)
        expect = np.zeros(32, dtype=np.int8)
        expect[0] = 7 if a > 0 else -7
        assert np.array_equal(q[0], expect), a
        assert d[0, 0] == np.float32(np.abs(v0) / np.float32(7.0))


def test_quantize_spike_closed_form():
    """x = a e_j: all rotated values have equal magnitude, codes are 7 sign(a) H[i][j]."""
    c = oracle.inv_sqrt32_f32()
    for j in [0, 1, 5, 16, 31]:
        for a in [2.0, -0.75]:
            x = np.zeros((1, 32), dtype=np.float32)
            x[0, j] = a
            q, d, _ = oracle.quantize(x, 4)
            assert np.array_equal(q[0], (7 * np.sign(a) * H[:, j]).astype(np.int8))
            assert d[0, 0] == np.float32(np.float32(abs(a) * c) / np.float32(7.0))
            q8, d8, _ = oracle.quantize(x, 8)
            assert np.array_equal(q8[0], (127 * np.sign(a) * H[:, j]).astype(np.int8))


def test_quantize_zero_block():
    x = np.zeros((2, 64), dtype=np.float32)
    x[1, 40] = 1.0
    q, d, _ = oracle.quantize(x, 4)
    assert np.all(q[0] == 0) and np.all(d[0] == 0)
    assert np.all(q[1, :32] == 0) and d[1, 0] == 0 and d[1, 1] > 0


def test_quantize_subnormal_blocks():
    """Blocks of subnormal values, against numpy's own IEEE float32 arithmetic
    (subnormals kept): a constant block of the smallest subnormal rotates to
    fp32(32 a * c) in element 0, whose scale fp32(v0 / 7) is still nonzero; a
    spike of 7 times it rotates to +-2^-149 everywhere, whose amax / 7 underflows
    to 0, and a zero scale gives codes 0 (both widths)."""
    tiny = np.float32(2.0 ** -149)
    c = np.float32(oracle.inv_sqrt32_f32())
    x = np.full((1, 32), tiny, dtype=np.float32)
    q, d, _ = oracle.quantize(x, 4)
    v0 = np.float32(np.float32(32 * tiny) * c)
    d0 = np.float32(v0 / np.float32(7.0))
    assert v0 > 0 and d0 > 0 and d[0, 0] == d0
    expect = np.zeros(32, dtype=np.int8)
    expect[0] = np.rint(np.float32(v0 / d0))
    assert np.array_equal(q[0], expect)
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, 8] = np.float32(-7.0) * tiny
    for bits in (4, 8):
        q, d, _ = oracle.quantize(x, bits)
        assert np.float32(np.float32(7.0 * tiny) * c) == tiny   # every |v| = 2^-149
        assert np.float32(tiny / np.float32(7.0)) == 0.0        # the scale underflows
        assert d[0, 0] == 0.0 and np.all(q[0] == 0)


def test_rint_ties_to_even():
    rows = [ln.split() for ln in open(os.path.join(GOLDEN, "rint_ties.txt"))
            if ln.strip() and not ln.startswith("#")]
    quot = [float(a) for a, _ in rows]
    code = [int(b) for _, b in rows]
    # without the transform, amax = 7 makes d = 1 exactly, so v/d = v
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, 0] = 7.0
    x[0, 1:1 + len(quot)] = quot
    q, d, ties = oracle.quantize(x, 4, rotate=False)
    assert d[0, 0] == 1.0
    assert list(q[0, 1:1 + len(quot)]) == code
    assert ties == len(quot)


def test_quantize_error_bound_and_range():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((64, 512)).astype(np.float32)
    x[:, rng.choice(512, 10, replace=False)] *= 25
    v = oracle.rotate_f32(x).astype(np.float64)
    for bits, qmax in [(4, 7), (8, 127)]:
        q, d, _ = oracle.quantize(x, bits)
        dd = np.repeat(d.astype(np.float64), 32, axis=1)
        assert np.all(np.abs(q) <= qmax)
        assert np.all(np.abs(v - dd * q) <= dd / 2 * (1 + 1e-6))
        # the largest value of every block takes the extreme code
        assert np.all(np.abs(q).reshape(64, -1, 32).max(axis=2) == qmax)


def test_quantize_matches_bruteforce_dense():
    """Codes from the dense fp64 transform agree away from .5 boundaries."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal((200, 64)).astype(np.float32)
    q, d, _ = oracle.quantize(x, 4)
    v = rotate_dense_f64(x)
    amax = np.abs(v).reshape(200, 2, 32).max(axis=2)
    dref = amax / 7.0
    assert np.allclose(d, dref, rtol=1e-6, atol=0)
    r = v / np.repeat(dref, 32, axis=1)
    safe = np.abs(r - np.floor(r) - 0.5) > 1e-4
    assert safe.mean() > 0.99
    assert np.array_equal(q[safe], np.rint(r[safe]).astype(np.int8))


def test_quantize_unrotated_route_bruteforce():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((50, 96)).astype(np.float32)
    q, d, _ = oracle.quantize(x, 4, rotate=False)
    amax = np.abs(x.astype(np.float64)).reshape(50, 3, 32).max(axis=2)
    assert np.allclose(d, amax / 7.0, rtol=1e-6, atol=0)
    r = x / np.repeat(amax / 7.0, 32, axis=1)
    safe = np.abs(r - np.floor(r) - 0.5) > 1e-4
    assert np.array_equal(q[safe], np.rint(r[safe]).astype(np.int8))


def test_bf16_input_is_widened_exactly():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((8, 128)).astype(np.float32)
    xb = synth.bf16_bits(x)
    q1, d1, _ = oracle.quantize(xb, 4)
    q2, d2, _ = oracle.quantize(synth.bf16_to_f32(xb), 4)
    assert np.array_equal(q1, q2) and np.array_equal(d1.view(np.uint32), d2.view(np.uint32))


def test_pack_int4_layout_fixture():
    lines = {ln.split()[0]: ln.split()[1:] for ln in open(os.path.join(GOLDEN,
             "int4_block_layout.txt")) if ln.strip() and not ln.startswith("#")}
    codes = np.array([int(t) for t in lines["codes"]], dtype=np.int8)[None, :]
    expect = np.array([int(t, 16) for t in lines["bytes"]], dtype=np.uint8)
    assert np.array_equal(oracle.pack_int4(codes)[0], expect)


# ----------------------------------------------------------------- products

def _small_case(m, k, n, seed):
    case = synth.small_dense(m, k, n, seed=seed)
    q, da, _ = oracle.quantize(case["x"], 4)
    w, dw = oracle.q4_0_decode(case["w"], k)
    return case, q, da, w, dw


def test_block_sums_match_numpy_matmul():
    case, q, da, w, dw = _small_case(9, 160, 33, 10)
    S = oracle.block_sums(q, w, 0, 9, 0, 33)
    qb = q.reshape(9, 5, 32).astype(np.int64)
    wb = w.reshape(33, 5, 32).astype(np.int64)
    ref = np.stack([qb[:, b, :] @ wb[:, b, :].T for b in range(5)], axis=2)
    assert np.array_equal(S, ref)
    S2 = oracle.block_sums(q, w, 3, 7, 10, 30)
    assert np.array_equal(S2, ref[3:7, 10:30])


def test_gemm_with_unit_scales_is_integer_matmul():
    case, q, da, w, dw = _small_case(7, 96, 20, 11)
    y = oracle.gemm_rect(q, np.ones_like(da), w, np.ones_like(dw), 0, 7, 0, 20)
    assert np.array_equal(y, (q.astype(np.int64) @ w.astype(np.int64).T).astype(np.float64))


def test_gemm_matches_numpy_formula():
    case, q, da, w, dw = _small_case(12, 256, 40, 12)
    y = oracle.gemm_rect(q, da, w, dw, 0, 12, 0, 40)
    S = np.stack([q.reshape(12, 8, 32)[:, b].astype(np.float64)
                  @ w.reshape(40, 8, 32)[:, b].astype(np.float64).T for b in range(8)], axis=2)
    ref = np.einsum("mb,nb,mnb->mn", da.astype(np.float64), dw, S)
    assert np.allclose(y, ref, rtol=1e-13, atol=1e-13 * np.abs(ref).max())
    pts = oracle.gemm_points(q, da, w, dw, [0, 11, 5], [39, 0, 17])
    assert np.array_equal(pts, y[[0, 11, 5], [39, 0, 17]])


def test_abs_sum_matches_numpy_and_bounds_output():
    """sum_b |da dw S|: numpy from integer block products; it bounds |y|, and
    it equals y where every term is non-negative (all codes and scales >= 0)."""
    case, q, da, w, dw = _small_case(8, 192, 24, 19)
    a = oracle.gemm_abs_rect(q, da, w, dw, 0, 8, 0, 24)
    S = np.stack([q.reshape(8, 6, 32)[:, b].astype(np.int64)
                  @ w.reshape(24, 6, 32)[:, b].astype(np.int64).T for b in range(6)], axis=2)
    ref = np.abs(da.astype(np.float64)[:, None, :] * dw[None, :, :] * S).sum(axis=2)
    assert np.allclose(a, ref, rtol=1e-14, atol=0)
    y = oracle.gemm_rect(q, da, w, dw, 0, 8, 0, 24)
    assert np.all(np.abs(y) <= a * (1 + 1e-14))
    assert np.array_equal(oracle.gemm_abs_rect(q, da, w, dw, 2, 5, 3, 20), a[2:5, 3:20])
    qp, wp = np.abs(q), np.abs(w)
    assert np.array_equal(oracle.gemm_abs_rect(qp, da, wp, dw, 0, 8, 0, 24),
                          oracle.gemm_rect(qp, da, wp, dw, 0, 8, 0, 24))
    # the grouped form selects the row's expert like grouped_points
    off = np.array([0, 5, 8], dtype=np.int32)
    wg = np.stack([w[:12], w[12:]])
    dwg = np.stack([dw[:12], dw[12:]])
    rows, cols = np.repeat(np.arange(9), 12), np.tile(np.arange(12), 9)
    ag = oracle.grouped_abs_points(q, da, off, wg, dwg, rows[:96], cols[:96]).reshape(8, 12)
    assert np.allclose(ag[:5], a[:5, :12], rtol=1e-14, atol=0)
    assert np.allclose(ag[5:], a[5:, 12:], rtol=1e-14, atol=0)
    assert np.isnan(oracle.grouped_abs_points(q, da, off, wg, dwg, [8], [0])[0])


def test_bruteforce_2x32x2():
    """Literal loops from the dense matrix: one block, so y = da dw S exactly."""
    rng = np.random.default_rng(13)
    x = rng.standard_normal((2, 32)).astype(np.float32)
    wblk = synth.draw_q4_0(rng, (2,), 32, 0.01, 0.05)
    q, da, _ = oracle.quantize(x, 4)
    w, dw = oracle.q4_0_decode(wblk, 32)
    for m in range(2):
        v = [sum(H[i][j] * float(x[m, j]) for j in range(32)) / np.sqrt(32.0) for i in range(32)]
        dref = max(abs(t) for t in v) / 7.0
        assert abs(da[m, 0] - dref) <= 1e-6 * dref
        for i in range(32):
            r = v[i] / dref
            if abs(r - np.floor(r) - 0.5) > 1e-4:
                assert q[m, i] == int(np.rint(r))
        for n in range(2):
            u = [((int(wblk[n, 0, 2 + (i % 16)]) >> (4 * (i // 16))) & 15) for i in range(32)]
            s = sum(int(q[m, i]) * (u[i] - 8) for i in range(32))
            dwn = float(wblk[n, 0, 0:2].view("<f2")[0])
            y = oracle.gemm_rect(q, da, w, dw, m, m + 1, n, n + 1)[0, 0]
            assert oracle.block_sums(q, w, m, m + 1, n, n + 1)[0, 0, 0] == s
            assert y == float(da[m, 0]) * dwn * s


def test_end_to_end_within_quantization_bound():
    """The whole route approximates the plain unrotated product x . w.

    Weights are stored rotated: w_rot = dw (u - 8); the unrotated weights are
    H w_rot / sqrt(32) per block.  The only error of the route is rounding the
    rotated activations to codes, |v - d q| <= d/2 per value, plus fp32
    rounding in the transform.
    """
    m, k, n = 6, 256, 24
    case, q, da, w, dw = _small_case(m, k, n, 14)
    x = case["x"].astype(np.float64)
    wrot = (w.reshape(n, -1, 32) * dw[:, :, None]).reshape(n, k)
    wun = rotate_dense_f64(wrot)
    y_plain = x @ wun.T
    y = oracle.gemm_rect(q, da, w, dw, 0, m, 0, n)
    absw = np.abs(wrot).reshape(n, -1, 32).sum(axis=2)            # [n, B]
    bound = (da.astype(np.float64) / 2) @ absw.T                  # [m, n]
    rot_err = 6 * 2.0 ** -24 * np.abs(x).reshape(m, -1, 32).sum(axis=2) @ absw.T
    assert np.all(np.abs(y - y_plain) <= bound * (1 + 1e-6) + rot_err + 1e-12)
    # and it is a real approximation, not a vacuous bound
    rel = np.linalg.norm(y - y_plain) / np.linalg.norm(y_plain)
    assert rel < 0.2
    # the unquantized reference equals the plain product
    rows, cols = np.meshgrid(np.arange(m), np.arange(n), indexing="ij")
    yr = oracle.ref_points(case["x"], w, dw, rows.ravel(), cols.ravel()).reshape(m, n)
    assert np.allclose(yr, y_plain, rtol=0, atol=1e-12 * np.abs(y_plain).max())


def test_rotation_reduces_block_error_with_outliers():
    """The reason for the rotation: with outlier channels, 4-bit error drops."""
    rng = np.random.default_rng(15)
    x, _ = synth.draw_activations(rng, 64, 1024, "normal", 0.01, 50.0)
    v = oracle.rotate_f32(x).astype(np.float64)
    qr, dr, _ = oracle.quantize(x, 4, rotate=True)
    qu, du, _ = oracle.quantize(x, 4, rotate=False)
    err_rot = np.linalg.norm(v - np.repeat(dr, 32, axis=1) * qr)
    err_un = np.linalg.norm(x - np.repeat(du, 32, axis=1) * qu)
    assert err_rot < 0.8 * err_un


def test_grouped_points_select_expert_weights():
    rng = np.random.default_rng(16)
    E, n, k, T = 5, 16, 64, 9
    x = rng.standard_normal((T * 2, k)).astype(np.float32)
    off = np.array([0, 3, 3, 10, 11, 18], dtype=np.int32)   # one empty expert
    blocks = synth.draw_q4_0(rng, (E, n), k, 0.01, 0.02)
    q, da, _ = oracle.quantize(x, 4)
    w, dw = oracle.q4_0_decode(blocks, k)
    w = w.reshape(E, n, k)
    dw = dw.reshape(E, n, k // 32)
    rows = np.repeat(np.arange(18), n)
    cols = np.tile(np.arange(n), 18)
    y = oracle.grouped_points(q, da, off, w, dw, rows, cols).reshape(18, n)
    for e in range(E):
        for r in range(off[e], off[e + 1]):
            S = np.array([q[r, 32 * b:32 * b + 32].astype(np.int64) @
                          w[e, :, 32 * b:32 * b + 32].astype(np.int64).T for b in range(2)])
            ref = (float(da[r, 0]) * dw[e, :, 0] * S[0] + float(da[r, 1]) * dw[e, :, 1] * S[1])
            assert np.allclose(y[r], ref, rtol=1e-14, atol=0)
    nan = oracle.grouped_points(q, da, off, w, dw, [18], [0])
    assert np.isnan(nan[0])


# ----------------------------------------------------------------- float weights

def test_weight_quantizer_roundtrip_without_rotation():
    rng = np.random.default_rng(17)
    u = rng.integers(1, 16, size=(10, 64))   # values -7..7 (amax/7 gives back dw)
    u[:, 0] = 15        # makes amax = 7 dw in block 0
    u[:, 32] = 15       # and in block 1
    dwv = np.float16(rng.uniform(0.01, 0.05, size=(10, 2))).astype(np.float64)
    wf = ((u - 8) * np.repeat(dwv, 32, axis=1)).astype(np.float32)
    blocks = oracle.quantize_weights_q4_0(wf, rotate=False)
    w, dw = oracle.q4_0_decode(blocks, 64)
    assert np.array_equal(w, (u - 8).astype(np.int8))
    assert np.array_equal(dw, dwv)


def test_weight_quantizer_with_rotation_reconstructs():
    rng = np.random.default_rng(18)
    wf = rng.standard_normal((20, 128)).astype(np.float32) * 0.05
    blocks = oracle.quantize_weights_q4_0(wf, rotate=True)
    w, dw = oracle.q4_0_decode(blocks, 128)
    wrot = (w.reshape(20, 4, 32) * dw[:, :, None]).reshape(20, 128)
    back = rotate_dense_f64(wrot)             # H/sqrt(32) is its own inverse
    err = np.abs(back - wf).reshape(20, 4, 32)
    # per block, the rotated-domain error is at most dw/2 per value (plus the
    # fp16 rounding of dw), and the inverse transform preserves the 2-norm
    blk_norm = np.sqrt((err ** 2).sum(axis=2))
    assert np.all(blk_norm <= np.sqrt(32) * dw * 0.5 * (1 + 1e-3) + 1e-12)
