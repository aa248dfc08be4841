"""GPU parity of the expert layer's glue around the grouped product: the expert
sort, the gathered grouped GEMM, the SwiGLU -> rotate -> quantize step and the
weighted combine, each against the oracle on the same inputs, and a whole
expert layer run stage by stage.

Bar: sort indices, codes, scales and the combine (an fp32 fma chain on both
sides) bit-exact; GEMM outputs within 1e-3 row-L2 of the oracle's fp64 output
(and within the fp32 accumulation error).
"""
import numpy as np
import pytest

import oracle
from bit_prefill_gemm_amd import binding as bb
from bit_prefill_gemm_amd import synth

from gpu_util import (act_to_device, assert_within_bound, check_grouped_rows, oracle_codes,
                      row_rel_err, sample_rows, torch_mod)

pytestmark = pytest.mark.gpu

TOL = 1e-3


@pytest.fixture(scope="module")
def torch():
    t = torch_mod()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    return t


def sort_and_check(expert_of, tokens, topk, experts):
    torch = torch_mod()
    e = torch.from_numpy(np.ascontiguousarray(expert_of, dtype=np.int32)).cuda()
    off, row_token, slot_of = bb.moe_route_sort(e, tokens, topk, experts)
    torch.cuda.synchronize()
    ref_off, ref_entry, ref_slot = oracle.route_sort(expert_of, experts)
    assert np.array_equal(off.cpu().numpy(), ref_off)
    assert np.array_equal(row_token.cpu().numpy(), ref_entry // topk)
    assert np.array_equal(slot_of.cpu().numpy(), ref_slot)
    return off, row_token, slot_of


# entries per thread (of 256): 16 with 16-byte loads kept in registers (512 x 8;
# 1000 x 4 with a partial last range), 32 with 16-byte loads read twice
# (1024 x 8), 10 and 1 with 4-byte loads (300 x 8, the small ones); the
# limits: 512 experts, 2^20 entries (4096 per thread)
@pytest.mark.parametrize("tokens,topk,experts", [(512, 8, 128), (1, 1, 1), (3, 2, 5),
                                                 (1000, 4, 64), (300, 8, 512), (1024, 8, 128),
                                                 (131072, 8, 512)])
def test_route_sort(torch, tokens, topk, experts):
    rng = np.random.default_rng(tokens + topk + experts)
    e, _ = synth.draw_routes(rng, tokens, experts, topk)
    print("sort", tokens, topk, experts, flush=True)
    sort_and_check(e, tokens, topk, experts)


def test_route_sort_skewed_and_empty_experts(torch):
    rng = np.random.default_rng(11)
    tokens, topk, experts = 700, 2, 40
    # most entries on three experts, many experts empty
    e = rng.choice([0, 7, 39], size=tokens * topk, p=[0.5, 0.3, 0.2]).astype(np.int32)
    sort_and_check(e, tokens, topk, experts)
    sort_and_check(np.full(tokens * topk, 5, dtype=np.int32), tokens, topk, experts)


def quantized_tokens(x, bits):
    torch = torch_mod()
    codes, scales = bb.quantize_act_h32(act_to_device(x), bits)
    q, d, _ = oracle.quantize(x, bits)
    assert np.array_equal(codes.cpu().numpy(), oracle_codes(q, bits))
    return codes, scales, q, d


def expert_weights(blocks, n, k, E):
    W = bb.rotate_pack_weights(blocks, bb.SRC_Q4_0_ROTATED, n, k, E).to("cuda")
    wq, dwq = oracle.q4_0_decode(blocks.reshape(E * n, k // 32, 18), k)
    return W, wq.reshape(E, n, k), dwq.reshape(E, n, k // 32)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("tokens,topk,experts,n,k", [(512, 8, 128, 1536, 2048),
                                                     (37, 3, 6, 96, 160), (64, 2, 4, 64, 1056)])
def test_gathered_grouped_gemm(torch, tokens, topk, experts, n, k, bits):
    rng = np.random.default_rng(tokens + n + k + bits)
    x, _ = synth.draw_activations(rng, tokens, k, "normal")
    x = synth.bf16_bits(x)
    blocks = synth.draw_q4_0(rng, (experts, n), k, 0.002, 0.02)
    e, _ = synth.draw_routes(rng, tokens, experts, topk)
    off, row_token, slot_of = sort_and_check(e, tokens, topk, experts)
    codes, scales, q, d = quantized_tokens(x, bits)
    W, wq, dwq = expert_weights(blocks, n, k, experts)
    print("gather", tokens, topk, experts, n, k, bits, flush=True)
    y = bb.w4a4_grouped_gemm_gather(codes, scales, bits, row_token, off, W)
    # the same product on explicitly permuted rows is bit-identical
    rt = row_token.long()
    y2 = bb.w4a4_grouped_gemm(codes[rt].contiguous(), scales[rt].contiguous(), bits, off, W)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    rows_total = tokens * topk
    rows = sample_rows(rows_total, 24, seed=k)
    rt_np = row_token.cpu().numpy()
    check_grouped_rows(y.cpu().numpy()[rows], q[rt_np], d[rt_np], off.cpu().numpy(), wq, dwq,
                       rows, k, "gather", TOL)


def swiglu_and_check(gu_np, inter, bits):
    torch = torch_mod()
    gu = torch.from_numpy(gu_np).cuda()
    codes, scales = bb.swiglu_quantize_h32(gu, inter, bits)
    torch.cuda.synchronize()
    q, d, _ = oracle.swiglu_quantize(gu_np, inter, bits)
    got = codes.cpu().numpy()
    bad = np.argwhere(got != oracle_codes(q, bits))
    assert bad.size == 0, "codes differ at %s (of %d)" % (bad[:5].tolist(), len(bad))
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), d.view(np.uint32))
    return codes, scales, q, d


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("rows,inter", [(1, 32), (7, 96), (4096, 768), (33, 2048)])
def test_swiglu_quantize(torch, rows, inter, bits):
    rng = np.random.default_rng(rows + inter + bits)
    g = (rng.standard_normal((rows, inter)) * 3.0).astype(np.float32)
    u = rng.standard_normal((rows, inter)).astype(np.float32)
    gu = np.concatenate([g, u], axis=1)
    print("swiglu", rows, inter, bits, flush=True)
    swiglu_and_check(gu, inter, bits)


def test_swiglu_quantize_edge_values(torch):
    rng = np.random.default_rng(12)
    rows, inter = 6, 64
    g = rng.standard_normal((rows, inter)).astype(np.float32)
    u = rng.standard_normal((rows, inter)).astype(np.float32)
    g[0] = 100.0             # saturated gate: exponent clamped, silu(g) = g
    g[1] = -100.0            # silu ~ -0
    g[2, :32] = 0.0          # silu(0) = 0: an all-zero block
    u[3] = 0.0               # all-zero row
    g[4] = np.linspace(-88, 89, inter, dtype=np.float32)
    u[5] = 1e-30             # tiny values
    swiglu_and_check(np.concatenate([g, u], axis=1), inter, 4)
    # subnormal products: scales that underflow to 0 (codes 0) and that do not
    g2, u2 = g.copy(), u.copy()
    g2[0], u2[0] = 1e-22, 1e-22
    g2[1, :32], u2[1, :32] = 1.0, np.float32(2.0 ** -149)
    for bits in (4, 8):
        swiglu_and_check(np.concatenate([g2, u2], axis=1), inter, bits)
    # a leading dimension past the two projections
    wide = np.full((rows, 2 * inter + 64), 1e30, dtype=np.float32)
    wide[:, :inter], wide[:, inter:2 * inter] = g, u
    swiglu_and_check(wide, inter, 4)


def combine_and_check(dn_np, slot_np, w_np, tokens, topk):
    torch = torch_mod()
    dn = torch.from_numpy(dn_np).cuda()
    slot = torch.from_numpy(slot_np).cuda()
    w = torch.from_numpy(w_np).cuda()
    y = bb.moe_combine(dn, slot, w, tokens, topk)
    torch.cuda.synchronize()
    ref = oracle.moe_combine(dn_np, slot_np, w_np, tokens, topk)
    assert np.array_equal(y.cpu().numpy().view(np.uint32), ref.view(np.uint32))
    return y


@pytest.mark.parametrize("tokens,topk,hidden", [(512, 8, 2048), (1, 1, 4), (13, 3, 36)])
def test_combine(torch, tokens, topk, hidden):
    rng = np.random.default_rng(tokens + topk + hidden)
    n = tokens * topk
    dn = rng.standard_normal((n, hidden)).astype(np.float32)
    slot = rng.permutation(n).astype(np.int32)
    _, w = synth.draw_routes(rng, tokens, max(topk, 1), topk)
    combine_and_check(dn, slot, w, tokens, topk)


def test_expert_layer_stage_by_stage(torch):
    """The moe512 layer: sort -> quantize tokens -> gathered gate/up -> SwiGLU
    quantize -> down -> combine.  Each stage is checked against the oracle on
    the GPU's own input to that stage."""
    t = synth.make("moe512")
    c = t["cfg"]
    T, H, E, K8, I = c["tokens"], c["hidden"], c["experts"], c["topk"], c["inter"]
    rng = np.random.default_rng(21)
    e, w = synth.draw_routes(rng, T, E, K8)
    print("layer: sort", flush=True)
    off, row_token, slot_of = sort_and_check(e, T, K8, E)
    codes, scales, q, d = quantized_tokens(t["x_tokens"], 4)
    Wgu, wq_gu, dw_gu = expert_weights(t["w_gu"], 2 * I, H, E)
    Wdn, wq_dn, dw_dn = expert_weights(t["w_dn"], H, I, E)
    print("layer: gate/up", flush=True)
    gu = bb.w4a4_grouped_gemm_gather(codes, scales, 4, row_token, off, Wgu)
    torch.cuda.synchronize()
    rows = sample_rows(T * K8, 12, seed=3)
    rt = row_token.cpu().numpy()
    off_np = off.cpu().numpy()
    check_grouped_rows(gu.cpu().numpy()[rows], q[rt], d[rt], off_np, wq_gu, dw_gu, rows, H,
                       "layer gate/up", TOL)
    print("layer: swiglu", flush=True)
    hc, hs, hq, hd = swiglu_and_check(gu.cpu().numpy(), I, 4)
    print("layer: down", flush=True)
    dn = bb.w4a4_grouped_gemm(hc, hs, 4, off, Wdn)
    torch.cuda.synchronize()
    check_grouped_rows(dn.cpu().numpy()[rows], hq, hd, off_np, wq_dn, dw_dn, rows, I,
                       "layer down", TOL)
    print("layer: combine", flush=True)
    combine_and_check(dn.cpu().numpy(), slot_of.cpu().numpy(), w, T, K8)
