"""GPU parity of the longer rotations (spans of 64 and 128 values, per-32
scales) and their accuracy against the unquantized fp64 product.

Bar: codes and scales bit-exact against the oracle; fp32 outputs within 1e-3
row-L2 of the oracle's fp64 output (and within the fp32 accumulation error).
"""
import numpy as np
import pytest

import oracle
from bit_prefill_gemm_amd import binding as bb
from bit_prefill_gemm_amd import synth

from gpu_util import (act_to_device, assert_within_bound, oracle_codes, row_rel_err, sample_rows,
                      torch_mod)

pytestmark = pytest.mark.gpu

TOL = 1e-3


@pytest.fixture(scope="module")
def torch():
    t = torch_mod()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    return t


def quantize_rot_and_check(x, rot, bits):
    torch = torch_mod()
    codes, scales = bb.quantize_act_rot(act_to_device(x), rot, bits)
    torch.cuda.synchronize()
    q, d, _ = oracle.quantize_rot(x, rot, bits)
    got = codes.cpu().numpy()
    bad = np.argwhere(got != oracle_codes(q, bits))
    assert bad.size == 0, "codes differ at %s (of %d)" % (bad[:5].tolist(), len(bad))
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), d.view(np.uint32))
    return codes, scales, q, d


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("rot", [32, 64, 128])
@pytest.mark.parametrize("name", ["tiny", "attn512", "m16_down"])
def test_quantize_rot_parity(torch, name, rot, bits):
    print("quantize rot", name, rot, bits, flush=True)
    quantize_rot_and_check(synth.make(name)["x"], rot, bits)


@pytest.mark.parametrize("rot", [64, 128])
def test_quantize_rot_ragged_and_edge(torch, rot):
    rng = np.random.default_rng(rot)
    x = rng.standard_normal((37, 3 * rot)).astype(np.float32)
    x[0] = 0.0
    x[1, :rot] = 1e-30
    x[2, 5] = 80.0
    x[3, :] = -2.0
    tiny = np.float32(2.0 ** -149)
    x[4, :rot] = tiny                 # subnormal inputs
    x[5, :rot] = 0.0
    x[5, 3] = -7 * tiny               # a scale that underflows to 0
    quantize_rot_and_check(x, rot, 4)
    quantize_rot_and_check(x, rot, 8)
    quantize_rot_and_check(np.ascontiguousarray(x[:1]), rot, 4)
    # ldx > k: the left part of a wider matrix
    wide = synth.bf16_bits(rng.standard_normal((9, 4 * rot)).astype(np.float32))
    xd = act_to_device(wide)[:, :2 * rot]
    codes, scales = bb.quantize_act_rot(xd, rot, 4)
    torch.cuda.synchronize()
    q, d, _ = oracle.quantize_rot(np.ascontiguousarray(wide[:, :2 * rot]), rot, 4)
    assert np.array_equal(codes.cpu().numpy(), oracle_codes(q, 4))


@pytest.mark.parametrize("rot", [64, 128])
@pytest.mark.parametrize("m,k,n", [(5, 256, 64), (100, 1024, 96), (512, 5120, 5120)])
def test_gemm_rot_parity(torch, rot, m, k, n):
    rng = np.random.default_rng(m + k + rot)
    x, _ = synth.draw_activations(rng, m, k, "normal", 0.01, 30.0)
    w = synth.draw_weights_f32(rng, n, k, 0.02)
    codes, scales, q, d = quantize_rot_and_check(x, rot, 4)
    W = bb.rotate_pack_weights_rot(w, bb.SRC_F32, n, k, rot).to("cuda")
    print("gemm rot", rot, m, k, n, flush=True)
    y = bb.w4a4_gemm_rot(codes, scales, 4, rot, W)
    torch.cuda.synchronize()
    wq, dw = oracle.q4_0_decode(oracle.quantize_weights_q4_0_rot(w, rot), k)
    rows = sample_rows(m, 8, seed=rot)
    ref = np.concatenate([oracle.gemm_rect(q, d, wq, dw, r, r + 1, 0, n) for r in rows])
    a = np.concatenate([oracle.gemm_abs_rect(q, d, wq, dw, r, r + 1, 0, n) for r in rows])
    err = row_rel_err(y.cpu().numpy()[rows], ref)
    assert err <= TOL, err
    assert_within_bound(y.cpu().numpy()[rows], ref, a, k, "rot %d" % rot)


def span_errors(name, seed=0, sample=6):
    """Route error against the fp64 x . W^T for spans 0 (unrotated), 32, 64,
    128 (4-bit activations, Q4_0 weights quantized from the same floats)."""
    torch = torch_mod()
    t = synth.make(name, seed)
    c = t["cfg"]
    m, k, n = c["m"], c["k"], c["n"]
    w = synth.draw_weights_f32(np.random.default_rng(1000 + seed), n, k, 0.02)
    rows = sample_rows(m, sample, seed=5)
    exact = synth.bf16_to_f32(t["x"][rows]).astype(np.float64) @ w.astype(np.float64).T
    xd = act_to_device(t["x"])
    out = {}
    for rot in (0, 32, 64, 128):
        if rot == 0:
            W = bb.pack_weights_unrotated(w, bb.SRC_F32, n, k).to("cuda")
            codes, scales = bb.quantize_act_unrotated(xd, 4)
            y = bb.w4a4_gemm_unrotated(codes, scales, 4, W)
        else:
            W = bb.rotate_pack_weights_rot(w, bb.SRC_F32, n, k, rot).to("cuda")
            codes, scales = bb.quantize_act_rot(xd, rot, 4)
            y = bb.w4a4_gemm_rot(codes, scales, 4, rot, W)
        torch.cuda.synchronize()
        yr = y.cpu().numpy()[rows]
        rel = np.linalg.norm(yr - exact, axis=1) / np.linalg.norm(exact, axis=1)
        out[rot] = float(rel.mean())
        del W, codes, scales, y
    print("%s error vs fp64 x.W by rotation span: none %.4f, 32 %.4f, 64 %.4f, 128 %.4f"
          % (name, out[0], out[32], out[64], out[128]), flush=True)
    return out


@pytest.mark.parametrize("name", ["attn512", "long1024"])
def test_span_accuracy(torch, name):
    e = span_errors(name)
    # every rotation beats none; the spans are reported, not ordered
    assert max(e[32], e[64], e[128]) < e[0]
