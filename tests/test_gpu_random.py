"""Seeded random shapes through every routed product, against the oracle.

The hand-picked cases of the other files pin each kernel's edges; these draw
shapes at random:
  - (M, K, N, code width, input dtype) over the shapes the routing sends to the
    weight-stream, tiled, strip and wide kernels;
  - ragged expert counts (empty experts included) for the grouped product with
    4- and 8-bit codes;
  - token, expert and width counts through the expert layer's sort, gathered
    product, SwiGLU-quantize and combine;
  - the unrotated route, the longer rotations and the bf16 output.
All at sizes the oracle computes in well under a second.  Codes, scales, sort
indices and combines are compared bit for bit; every product output checked
lies within the fp32 accumulation bound of the oracle's exact value.
"""
import numpy as np
import pytest

import oracle
from bit_prefill_gemm_amd import binding as bb
from bit_prefill_gemm_amd import synth

from gpu_util import (act_to_device, assert_within_bound, check_grouped_rows, oracle_codes,
                      quantize_and_check, row_rel_err, sample_rows, torch_mod, weights_to_device)

pytestmark = pytest.mark.gpu

SEED = 20260
DENSE_CASES = 80
GROUPED_CASES = 24
TOL = 1e-3  # row-L2 relative error, the contract


@pytest.fixture(scope="module")
def torch():
    t = torch_mod()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    return t


def dense_shape(rng, i):
    """(m, k, n, bits, dtype): few rows, medium and many rows; N any multiple
    of 32, of 128 (strips) or of 160 (wide tiles); every fourth case a wide-
    tile shape (many 64 x 160 tiles, short K)."""
    bits = int(rng.choice([4, 8]))
    kind = int(rng.integers(3))
    m = (int(rng.integers(1, 33)) if kind == 0 else
         int(rng.integers(33, 160)) if kind == 1 else int(rng.integers(160, 700)))
    k = 32 * int(rng.integers(1, 97))
    nk = int(rng.integers(3))
    n = (32 * int(rng.integers(1, 49)) if nk == 0 else
         128 * int(rng.integers(1, 13)) if nk == 1 else 160 * int(rng.integers(1, 11)))
    if i % 4 == 3:
        m, n, k, bits = (int(rng.integers(65, 400)), 160 * int(rng.integers(32, 128)),
                         32 * int(rng.integers(1, 8)), 4)
    while m * k * n > 4e8:
        m = max(1, m // 2)
    return m, k, n, bits, str(rng.choice(["f32", "bf16"]))


def test_random_dense_shapes(torch):
    rng = np.random.default_rng(SEED)
    seen = set()
    for i in range(DENSE_CASES):
        m, k, n, bits, dt = dense_shape(rng, i)
        sd = int(rng.integers(1 << 30))
        case = synth.small_dense(m, k, n, seed=sd, dtype=dt)
        codes, scales, q, d = quantize_and_check(case["x"], bits)
        W = weights_to_device(case["w"], n, k)
        kname = bb.w4a4_gemm_kernel_name(bits, m, W)
        print("random dense", i, (m, k, n), bits, dt, kname, flush=True)
        seen.add(kname)
        y = bb.w4a4_gemm(codes, scales, bits, W)
        torch.cuda.synchronize()
        w, dw = oracle.q4_0_decode(case["w"], k)
        rows = np.arange(m) if m <= 64 else sample_rows(m, 24, sd)
        ref = np.concatenate([oracle.gemm_rect(q, d, w, dw, r, r + 1, 0, n) for r in rows])
        a = np.concatenate([oracle.gemm_abs_rect(q, d, w, dw, r, r + 1, 0, n) for r in rows])
        yg = y.cpu().numpy()[rows]
        assert row_rel_err(yg, ref) <= TOL
        assert_within_bound(yg, ref, a, k, "random dense %d %s" % (i, (m, k, n, bits)))
    # the draw reaches every dense kernel family
    assert {"weight-stream", "strip 32x128", "wide 64x160"} <= seen, seen
    assert any(s.startswith("tiled") for s in seen), seen


def test_random_grouped_shapes(torch):
    rng = np.random.default_rng(SEED + 1)
    seen = set()
    for i in range(GROUPED_CASES):
        E = int(rng.integers(1, 80))
        counts = rng.integers(0, 90, size=E)
        counts[rng.random(E) < 0.2] = 0
        if counts.sum() == 0:
            counts[0] = 5
        n = int(rng.choice([64, 96, 128, 256, 384, 512, 768]))
        k = 32 * int(rng.integers(1, 65))
        if counts.sum() * k * n > 4e8:
            k = 32 * max(1, int(4e8 / (counts.sum() * n * 32)))
        bits = int(rng.choice([4, 4, 8]))
        sd = int(rng.integers(1 << 30))
        off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
        total = int(off[-1])
        r2 = np.random.default_rng(sd)
        x, _ = synth.draw_activations(r2, total, k, "normal", 0.02, 20.0)
        blocks = synth.draw_q4_0(r2, (E, n), k, 0.005, 0.05)
        codes, scales = bb.quantize_act_h32(act_to_device(x), bits)
        q, d, _ = oracle.quantize(x, bits)
        torch.cuda.synchronize()
        assert np.array_equal(codes.cpu().numpy(), oracle_codes(q, bits))
        W = bb.rotate_pack_weights(blocks, bb.SRC_Q4_0_ROTATED, n, k, E).to("cuda")
        wq, dwq = oracle.q4_0_decode(blocks.reshape(E * n, k // 32, 18), k)
        kname = bb.w4a4_grouped_gemm_kernel_name(bits, total, W)
        print("random grouped", i, E, total, n, k, bits, kname, flush=True)
        seen.add(kname)
        y = torch.full((total, n), float("nan"), device="cuda")
        bb.w4a4_grouped_gemm(codes, scales, bits, torch.from_numpy(off).cuda(), W, y=y)
        torch.cuda.synchronize()
        firsts = off[:-1][off[1:] > off[:-1]]
        lasts = off[1:][off[1:] > off[:-1]] - 1
        rows = np.unique(np.concatenate([firsts, lasts, sample_rows(total, 30, sd)]))
        check_grouped_rows(y.cpu().numpy()[rows], q, d, off, wq.reshape(E, n, k),
                           dwq.reshape(E, n, k // 32), rows, k, "random grouped %d" % i, TOL)
    assert "expert-slot" in seen and any(s.startswith("grouped") for s in seen), seen


def test_random_expert_glue(torch):
    """Random token counts, expert counts and widths through the expert
    layer's glue: the expert sort (bit-exact), the gathered grouped product
    (within the fp32 bound), SwiGLU -> rotate -> quantize (bit-exact codes and
    scales) and the weighted combine (bit-exact)."""
    rng = np.random.default_rng(SEED + 2)
    for i in range(16):
        experts = int(rng.integers(1, 513))
        topk = int(rng.integers(1, min(8, experts) + 1))
        tokens = int(rng.integers(1, 400))
        e_of, w_route = synth.draw_routes(rng, tokens, experts, topk)
        print("random glue", i, tokens, topk, experts, flush=True)
        ed = torch.from_numpy(e_of).cuda()
        off, row_token, slot_of = bb.moe_route_sort(ed, tokens, topk, experts)
        torch.cuda.synchronize()
        ref_off, ref_entry, ref_slot = oracle.route_sort(e_of, experts)
        assert np.array_equal(off.cpu().numpy(), ref_off)
        assert np.array_equal(row_token.cpu().numpy(), ref_entry // topk)
        assert np.array_equal(slot_of.cpu().numpy(), ref_slot)

        # the gathered product over these routes (up to 64 experts: small weights)
        if experts <= 64:
            bits = int(rng.choice([4, 8]))
            n = int(rng.choice([64, 96, 128, 256, 384]))
            k = 32 * int(rng.integers(1, 33))
            x, _ = synth.draw_activations(rng, tokens, k, "normal")
            x = synth.bf16_bits(x)
            blocks = synth.draw_q4_0(rng, (experts, n), k, 0.002, 0.02)
            codes, scales = bb.quantize_act_h32(act_to_device(x), bits)
            q, d, _ = oracle.quantize(x, bits)
            W = bb.rotate_pack_weights(blocks, bb.SRC_Q4_0_ROTATED, n, k, experts).to("cuda")
            wq, dwq = oracle.q4_0_decode(blocks.reshape(experts * n, k // 32, 18), k)
            y = bb.w4a4_grouped_gemm_gather(codes, scales, bits, row_token, off, W)
            torch.cuda.synchronize()
            rows = sample_rows(tokens * topk, 24, i)
            rt = row_token.cpu().numpy()
            check_grouped_rows(y.cpu().numpy()[rows], q[rt], d[rt], ref_off,
                               wq.reshape(experts, n, k), dwq.reshape(experts, n, k // 32),
                               rows, k, "random gather %d" % i, TOL)

        # SwiGLU -> quantize on the routed rows' width
        inter = 32 * int(rng.integers(1, 65))
        sbits = int(rng.choice([4, 8]))
        gu = np.concatenate([(rng.standard_normal((tokens * topk, inter)) * 3.0),
                             rng.standard_normal((tokens * topk, inter))],
                            axis=1).astype(np.float32)
        c2, s2 = bb.swiglu_quantize_h32(torch.from_numpy(gu).cuda(), inter, sbits)
        torch.cuda.synchronize()
        q2, d2, _ = oracle.swiglu_quantize(gu, inter, sbits)
        assert np.array_equal(c2.cpu().numpy(), oracle_codes(q2, sbits))
        assert np.array_equal(s2.cpu().numpy().view(np.uint32), d2.view(np.uint32))

        # weighted combine of the sorted rows back to tokens
        hidden = 4 * int(rng.integers(1, 513))
        dn = rng.standard_normal((tokens * topk, hidden)).astype(np.float32)
        yc = bb.moe_combine(torch.from_numpy(dn).cuda(), slot_of,
                            torch.from_numpy(w_route).cuda(), tokens, topk)
        torch.cuda.synchronize()
        ref = oracle.moe_combine(dn, ref_slot, w_route, tokens, topk)
        assert np.array_equal(yc.cpu().numpy().view(np.uint32), ref.view(np.uint32))


def test_random_route_variants(torch):
    """Random shapes through the unrotated route and the longer rotations
    (spans of 64 and 128 values): codes and scales bit-exact, outputs within
    the fp32 bound; and the bf16 output, equal to the fp32 output rounded to
    nearest even."""
    rng = np.random.default_rng(SEED + 3)
    for i in range(24):
        rot = int(rng.choice([0, 64, 128]))
        span = max(rot, 32)
        bits = int(rng.choice([4, 8]))
        m = int(rng.choice([int(rng.integers(1, 33)), int(rng.integers(33, 400))]))
        k = span * int(rng.integers(1, max(2, 2048 // span)))
        n = int(rng.choice([32 * int(rng.integers(1, 33)), 128 * int(rng.integers(1, 9)),
                            160 * int(rng.integers(1, 9))]))
        sd = int(rng.integers(1 << 30))
        r2 = np.random.default_rng(sd)
        x, _ = synth.draw_activations(r2, m, k, "normal", 0.02, 20.0)
        w = synth.draw_weights_f32(r2, n, k, 0.02)
        print("random route", i, rot, bits, (m, k, n), flush=True)
        xd = act_to_device(x)
        if rot == 0:
            codes, scales = bb.quantize_act_unrotated(xd, bits)
            q, d, _ = oracle.quantize(x, bits, rotate=False)
            W = bb.pack_weights_unrotated(w, bb.SRC_F32, n, k).to("cuda")
            y = bb.w4a4_gemm_unrotated(codes, scales, bits, W)
            wq, dw = oracle.q4_0_decode(oracle.quantize_weights_q4_0(w, rotate=False), k)
        else:
            codes, scales = bb.quantize_act_rot(xd, rot, bits)
            q, d, _ = oracle.quantize_rot(x, rot, bits)
            W = bb.rotate_pack_weights_rot(w, bb.SRC_F32, n, k, rot).to("cuda")
            y = bb.w4a4_gemm_rot(codes, scales, bits, rot, W)
            wq, dw = oracle.q4_0_decode(oracle.quantize_weights_q4_0_rot(w, rot), k)
        torch.cuda.synchronize()
        assert np.array_equal(codes.cpu().numpy(), oracle_codes(q, bits))
        assert np.array_equal(scales.cpu().numpy().view(np.uint32), d.view(np.uint32))
        rows = np.arange(m) if m <= 32 else sample_rows(m, 16, sd)
        ref = np.concatenate([oracle.gemm_rect(q, d, wq, dw, r, r + 1, 0, n) for r in rows])
        a = np.concatenate([oracle.gemm_abs_rect(q, d, wq, dw, r, r + 1, 0, n) for r in rows])
        yg = y.cpu().numpy()[rows]
        assert row_rel_err(yg, ref) <= TOL
        assert_within_bound(yg, ref, a, k, "random route %d" % i)
    rng = np.random.default_rng(SEED + 4)
    for i in range(12):
        bits = int(rng.choice([4, 8]))
        m = int(rng.choice([int(rng.integers(1, 33)), int(rng.integers(33, 600))]))
        k = 32 * int(rng.integers(1, 65))
        n = int(rng.choice([32 * int(rng.integers(1, 33)), 128 * int(rng.integers(1, 17)),
                            160 * int(rng.integers(1, 33))]))
        case = synth.small_dense(m, k, n, seed=int(rng.integers(1 << 30)), dtype="bf16")
        print("random bf16 out", i, bits, (m, k, n), flush=True)
        codes, scales = bb.quantize_act_h32(act_to_device(case["x"]), bits)
        W = weights_to_device(case["w"], n, k)
        y32 = bb.w4a4_gemm(codes, scales, bits, W)
        y16 = bb.w4a4_gemm_bf16(codes, scales, bits, W)
        torch.cuda.synchronize()
        assert torch.equal(y16.view(torch.int16), y32.to(torch.bfloat16).view(torch.int16))
