"""GPU parity of the unrotated W4A4 route (plain Q4_0 weights, 4-bit
activations with no rotation), and the accuracy of the three routes against
the unquantized fp64 product on the dense prompt workloads.

Bar: codes and scales bit-exact against the oracle's unrotated quantizer;
fp32 outputs within 1e-3 row-L2 of the oracle's fp64 output (and within the
fp32 accumulation error).
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


def quantize_unrotated_and_check(x, bits):
    torch = torch_mod()
    codes, scales = bb.quantize_act_unrotated(act_to_device(x), bits)
    torch.cuda.synchronize()
    q, d, _ = oracle.quantize(x, bits, rotate=False)
    got = codes.cpu().numpy()
    bad = np.argwhere(got != oracle_codes(q, bits))
    assert bad.size == 0, "codes differ at %s (of %d)" % (bad[:5].tolist(), len(bad))
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), d.view(np.uint32))
    return codes, scales, q, d


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("name", ["tiny", "attn512", "m16_attn"])
def test_quantize_unrotated_parity(torch, name, bits):
    print("quantize unrotated", name, bits, flush=True)
    quantize_unrotated_and_check(synth.make(name)["x"], bits)


def test_quantize_unrotated_edge_cases(torch):
    rng = np.random.default_rng(41)
    x = rng.standard_normal((5, 96)).astype(np.float32)
    x[0] = 0.0
    x[1, :32] = -3.0
    x[2, 32:64] = 1e-30
    x[3, 40] = 55.0
    tiny = np.float32(2.0 ** -149)
    x[4, :32] = 0.0
    x[4, 7] = 3 * tiny                # the scale underflows to 0 (no rotation)
    x[4, 32:64] = 7 * tiny            # subnormal scale, codes 7
    for bits in (4, 8):
        quantize_unrotated_and_check(x, bits)
        quantize_unrotated_and_check(np.ascontiguousarray(x[:1, :32]), bits)


def check_unrotated_gemm(x, blocks, n, k, bits, rows=None, label=""):
    torch = torch_mod()
    codes, scales, q, d = quantize_unrotated_and_check(x, bits)
    W = bb.pack_weights_unrotated(blocks, bb.SRC_Q4_0, n, k, 1).to("cuda")
    print("gemm unrotated", label, x.shape, n, bits, flush=True)
    y = bb.w4a4_gemm_unrotated(codes, scales, bits, W)
    torch.cuda.synchronize()
    w, dw = oracle.q4_0_decode(blocks, k)
    rows = np.arange(x.shape[0]) if rows is None else rows
    ref = np.concatenate([oracle.gemm_rect(q, d, w, dw, r, r + 1, 0, n) for r in rows])
    a = np.concatenate([oracle.gemm_abs_rect(q, d, w, dw, r, r + 1, 0, n) for r in rows])
    err = row_rel_err(y.cpu().numpy()[rows], ref)
    assert err <= TOL, err
    assert_within_bound(y.cpu().numpy()[rows], ref, a, k, label)
    return y


@pytest.mark.parametrize("m,k,n", [(1, 64, 32), (17, 1056, 96), (100, 320, 96),
                                   (257, 160, 224)])
@pytest.mark.parametrize("bits", [4, 8])
def test_gemm_unrotated_ragged(torch, m, k, n, bits):
    case = synth.small_dense(m, k, n, seed=7 * m + k + n)
    check_unrotated_gemm(case["x"], case["w"], n, k, bits, label="ragged")


@pytest.mark.parametrize("name", ["attn512", "m16_attn"])
def test_gemm_unrotated_full_size(torch, name):
    t = synth.make(name)
    c = t["cfg"]
    rows = sample_rows(c["m"], 8, seed=9)
    check_unrotated_gemm(t["x"], t["w"], c["n"], c["k"], 4, rows=rows, label=name)


def test_unrotated_image_refused_by_rotated_gemm(torch):
    case = synth.small_dense(16, 64, 32, seed=2)
    codes, scales = bb.quantize_act_h32(act_to_device(case["x"]), 4)
    W = bb.pack_weights_unrotated(case["w"], bb.SRC_Q4_0, 32, 64, 1).to("cuda")
    with pytest.raises(bb.BpgError) as ei:
        bb.w4a4_gemm(codes, scales, 4, W)
    assert ei.value.status == 5


# ------------------------------------------------------------ route accuracy

def route_errors(name, seed=0, sample=6):
    """Float weights W (normal, std 0.02) are packed by both offline packers;
    activations are the workload's (outlier channels included).  Every route's
    GPU output is checked against the oracle, then compared with the fp64
    product x . W^T on sampled rows."""
    torch = torch_mod()
    t = synth.make(name, seed)
    c = t["cfg"]
    m, k, n = c["m"], c["k"], c["n"]
    w = synth.draw_weights_f32(np.random.default_rng(1000 + seed), n, k, 0.02)
    rows = sample_rows(m, sample, seed=5)
    xs = synth.bf16_to_f32(t["x"][rows]).astype(np.float64)
    exact = xs @ w.astype(np.float64).T
    xd = act_to_device(t["x"])
    out = {}
    for rotate in (False, True):
        pack = bb.rotate_pack_weights if rotate else bb.pack_weights_unrotated
        W = pack(w, bb.SRC_F32, n, k, 1).to("cuda")
        wq, dw = oracle.q4_0_decode(oracle.quantize_weights_q4_0(w, rotate=rotate), k)
        for bits in (4, 8):
            print("route", name, "rotated" if rotate else "unrotated", bits, flush=True)
            if rotate:
                codes, scales = bb.quantize_act_h32(xd, bits)
                y = bb.w4a4_gemm(codes, scales, bits, W)
            else:
                codes, scales = bb.quantize_act_unrotated(xd, bits)
                y = bb.w4a4_gemm_unrotated(codes, scales, bits, W)
            torch.cuda.synchronize()
            yr = y.cpu().numpy()[rows]
            q, d, _ = oracle.quantize(t["x"][rows], bits, rotate=rotate)
            ref = oracle.gemm_rect(q, d, wq, dw, 0, len(rows), 0, n)
            a = oracle.gemm_abs_rect(q, d, wq, dw, 0, len(rows), 0, n)
            err = row_rel_err(yr, ref)
            assert err <= TOL, err
            assert_within_bound(yr, ref, a, k, "route %s %d" % (rotate, bits))
            rel = np.linalg.norm(yr - exact, axis=1) / np.linalg.norm(exact, axis=1)
            out[(rotate, bits)] = float(rel.mean())
            del y, codes, scales
        del W
    print("%s error vs fp64 x.W (mean row-L2): unrotated int4 %.4f, rotated int4 %.4f, "
          "rotated q8 %.4f, unrotated q8 %.4f" % (name, out[(False, 4)], out[(True, 4)],
                                                   out[(True, 8)], out[(False, 8)]), flush=True)
    return out


@pytest.mark.parametrize("name", ["attn512", "long1024"])
def test_route_accuracy(torch, name):
    e = route_errors(name)
    # the pages' ordering: exact 8-bit < rotated 4-bit < unrotated 4-bit
    assert e[(True, 8)] < e[(True, 4)] < e[(False, 4)]
