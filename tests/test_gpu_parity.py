"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle.

Bar: activation codes, scales and int32 block sums bit-exact; fp32 outputs
within 1e-3 of the oracle's fp64 output in row-L2 relative error, and every
element within the fp32 accumulation bound (B + 8) * 2^-24 * sum_b |da dw S|.
The block sums of the kernels the products route to are shown exact through
their outputs in test_gpu_exact.py.
"""
import numpy as np
import pytest

import oracle
from bit_prefill_gemm_amd import binding as bb
from bit_prefill_gemm_amd import synth

from gpu_util import (act_to_device, assert_within_bound, quantize_and_check, rects,
                      row_rel_err, sample_rows, torch_mod, weights_to_device)

pytestmark = pytest.mark.gpu

TOL = 1e-3        # row-L2 relative error, the contract


@pytest.fixture(scope="module")
def torch():
    t = torch_mod()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    return t


# ------------------------------------------------------------------ quantizer

@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("name,key", [("tiny", "x"), ("attn512", "x"), ("long1024", "x"),
                                      ("ffn512", "x1"), ("ffn512", "x2"), ("moe512", "x_gu"),
                                      ("moe512", "x_dn"), ("m16_down", "x")])
def test_quantize_parity_workloads(torch, name, key, bits):
    print("quantize", name, key, bits, flush=True)
    quantize_and_check(synth.make(name)[key], bits)


def test_quantize_edge_cases(torch):
    rng = np.random.default_rng(31)
    x = rng.standard_normal((7, 96)).astype(np.float32)
    x[0] = 0.0                                   # all-zero row
    x[1, :32] = 2.5                              # constant block
    x[2, 32:64] = 1e-30                          # tiny block
    x[3, 64:96] = 1e30                           # huge block
    x[4, 5] = -40.0                              # spike
    x[5, :32] = 0.0
    x[5, 17] = 1e-3                              # one nonzero
    tiny = np.float32(2.0 ** -149)
    x[6, :32] = tiny                             # subnormal, nonzero scale
    x[6, 32:64] = 0.0
    x[6, 40] = -7 * tiny                         # the scale underflows to 0
    x[6, 64:96] *= np.float32(1e-40)             # subnormal inputs
    for bits in (4, 8):
        quantize_and_check(x, bits)
        quantize_and_check(x[:1], bits)          # M = 1
        quantize_and_check(np.ascontiguousarray(x[:, :32]), bits)   # K = 32


def test_quantize_strided_rows(torch):
    """ldx > k: quantize the left half of a wider matrix."""
    rng = np.random.default_rng(32)
    full = synth.bf16_bits(rng.standard_normal((33, 256)).astype(np.float32))
    xd = act_to_device(full)[:, :160]
    assert xd.stride(0) == 256
    codes, scales = bb.quantize_act_h32(xd, 4)
    q, d, _ = oracle.quantize(np.ascontiguousarray(full[:, :160]), 4)
    assert np.array_equal(codes.cpu().numpy(), oracle.pack_int4(q))
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), d.view(np.uint32))


def test_quantize_empty(torch):
    x = torch.empty((0, 64), dtype=torch.float32, device="cuda")
    codes, scales = bb.quantize_act_h32(x, 4)
    assert codes.shape == (0, 32) and scales.shape == (0, 2)


# ------------------------------------------------------------------ block sums

def check_blocksums(codes, scales, bits, W, q, w, rect_list, expert=0):
    torch = torch_mod()
    for (m0, m1, n0, n1) in rect_list:
        print("blocksums", bits, (m0, m1, n0, n1), "expert", expert, flush=True)
        s = bb.w4a4_gemm_blocksums(codes, scales, bits, W, m0, m1, n0, n1, expert=expert)
        torch.cuda.synchronize()
        ref = oracle.block_sums(q, w, m0, m1, n0, n1)
        got = s.cpu().numpy()
        bad = np.argwhere(got != ref)
        assert bad.size == 0, "block sums differ at %s" % bad[:5].tolist()


@pytest.mark.parametrize("bits", [4, 8])
def test_blocksums_tiny_full(torch, bits):
    t = synth.make("tiny")
    codes, scales, q, _ = quantize_and_check(t["x"], bits)
    W = weights_to_device(t["w"], 128, 256)
    w, _ = oracle.q4_0_decode(t["w"], 256)
    check_blocksums(codes, scales, bits, W, q, w, [(0, 16, 0, 128), (3, 11, 17, 90)])


@pytest.mark.parametrize("bits", [4, 8])
def test_blocksums_attn512_sampled(torch, bits):
    t = synth.make("attn512")
    codes, scales, q, _ = quantize_and_check(t["x"], bits)
    W = weights_to_device(t["w"], 5120, 5120)
    w, _ = oracle.q4_0_decode(t["w"], 5120)
    check_blocksums(codes, scales, bits, W, q, w, rects(512, 5120, 64, 3, seed=bits))


def test_blocksums_ffn_down_sampled(torch):
    t = synth.make("ffn512")
    codes, scales, q, _ = quantize_and_check(t["x2"], 4)
    W = weights_to_device(t["w_down"], 5120, 17408)
    w, _ = oracle.q4_0_decode(t["w_down"], 17408)
    check_blocksums(codes, scales, 4, W, q, w, rects(512, 5120, 64, 2, seed=5))


# ------------------------------------------------------------------ dense GEMM

def oracle_rows(q, d, w, dw, rows, n):
    """The oracle's output and magnitude sums on `rows` (None: every row), all columns."""
    if rows is None:
        m = q.shape[0]
        return (oracle.gemm_rect(q, d, w, dw, 0, m, 0, n),
                oracle.gemm_abs_rect(q, d, w, dw, 0, m, 0, n))
    ref = np.concatenate([oracle.gemm_rect(q, d, w, dw, r, r + 1, 0, n) for r in rows])
    a = np.concatenate([oracle.gemm_abs_rect(q, d, w, dw, r, r + 1, 0, n) for r in rows])
    return ref, a


def check_gemm(x, blocks, n, k, bits, rows=None, label=""):
    """The product of the workload through w4a4_gemm, on `rows` (None: all)."""
    torch = torch_mod()
    codes, scales, q, d = quantize_and_check(x, bits)
    W = weights_to_device(blocks, n, k)
    print("gemm", label, x.shape, n, bits, bb.w4a4_gemm_kernel_name(bits, x.shape[0], W),
          flush=True)
    y = bb.w4a4_gemm(codes, scales, bits, W)
    torch.cuda.synchronize()
    w, dw = oracle.q4_0_decode(blocks, k)
    yg = y.cpu().numpy() if rows is None else y.cpu().numpy()[rows]
    ref, a = oracle_rows(q, d, w, dw, rows, n)
    err = row_rel_err(yg, ref)
    assert err <= TOL, err
    assert_within_bound(yg, ref, a, k, label)
    return y, err


@pytest.mark.parametrize("bits", [4, 8])
def test_gemm_tiny_full(torch, bits):
    t = synth.make("tiny")
    check_gemm(t["x"], t["w"], 128, 256, bits, label="tiny")


@pytest.mark.parametrize("m,k,n", [(100, 320, 96), (1, 64, 32), (16, 256, 128), (33, 128, 64),
                                   (64, 32, 160), (130, 96, 224), (257, 1056, 64)])
@pytest.mark.parametrize("bits", [4, 8])
def test_gemm_ragged_shapes(torch, m, k, n, bits):
    case = synth.small_dense(m, k, n, seed=m + k + n)
    check_gemm(case["x"], case["w"], n, k, bits, label="ragged")


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("m,k,n", [(200, 1056, 10240), (77, 544, 20480), (130, 96, 8192),
                                   (256, 2080, 10240), (64, 32, 40960)])
def test_gemm_wide_tiles(torch, m, k, n, bits):
    """Shapes large enough in M x N for the wide tiles (4-bit: the 64 x 160
    direct-load kernel; 8-bit: the tiled kernel's 64 x 160 tiles; both the
    strip kernel where N = 8192 is not a multiple of 160): ragged last row
    tile, K with a partial last group and a partial last stage, fewer groups
    than K waves (K = 96 and 32)."""
    case = synth.small_dense(m, k, n, seed=m + 3 * k + n)
    rows = sample_rows(m, 10, seed=m + k)
    check_gemm(case["x"], case["w"], n, k, bits, rows=rows, label="wide")


@pytest.mark.parametrize("m,k,n", [(1000, 1056, 12288), (1000, 448, 12288), (2048, 160, 6144),
                                   (4096, 96, 17408), (1024, 32, 12288), (33, 32, 128),
                                   (40, 1056, 256), (65, 640, 640), (64, 32800, 256)])
@pytest.mark.parametrize("bits", [4, 8])
def test_gemm_strip_tiles(torch, m, k, n, bits):
    """4-bit shapes with more than 32 rows, N a multiple of 128 and 64 x 160
    tiles not the estimator's choice, which run the strip kernel (one
    32-column tile per wave over all of K): ragged last strip (M = 1000, and
    a last strip of one row: M = 33, 65), K with an odd number of 4-block
    groups and a one-block last stage (1056), an even number with a partial
    last group (448), one stage (160), one partial group (96) and a single
    block (32), and a long K (32800: 1025 blocks); a few workgroups (M = 33,
    N = 128) up to thousands.  8-bit
    codes take stages of four blocks (one group) instead of eight."""
    case = synth.small_dense(m, k, n, seed=m + 5 * k + n)
    rows = sample_rows(m, 24, seed=m + k + 1)
    check_gemm(case["x"], case["w"], n, k, bits, rows=rows, label="strip")


@pytest.mark.parametrize("m", [1, 7, 16, 17, 32])
@pytest.mark.parametrize("k,n", [(32, 32), (1056, 96)])
@pytest.mark.parametrize("bits", [4, 8])
def test_gemm_few_rows(torch, m, k, n, bits):
    """M <= 32 runs the weight-stream kernel: one and two row tiles, K shorter
    than one block per wave and K not a multiple of the blocks in flight."""
    case = synth.small_dense(m, k, n, seed=3 * m + k + n + bits)
    check_gemm(case["x"], case["w"], n, k, bits, label="few rows")


@pytest.mark.parametrize("k", [32768, 32800])
def test_gemm_few_rows_long_k(torch, k):
    """The largest K whose transposed row scales fit the weight-stream kernel's
    LDS (1024 blocks for 16 rows), and one block more (the tiled kernel)."""
    case = synth.small_dense(16, k, 64, seed=k)
    check_gemm(case["x"], case["w"], 64, k, 4, label="few rows long K")


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("m,k,n,kernels", [
    (5, 1 << 22, 32, ("tiled 16x32", "tiled 16x32")),
    (33, 1 << 20, 128, ("strip 32x128", "strip 32x128")),
    (512, 1 << 16, 5120, ("wide 64x160", "tiled 64x160"))])
def test_gemm_max_k(torch, m, k, n, kernels, bits):
    """K at the boundary's limit, 2^22 values (131072 blocks: the largest K whose
    per-workgroup operand offsets stay 32-bit), on the kernel few rows route
    to there; 2^20 on the strip kernel and 2^16 (128 stages of 16 blocks) on
    the 64 x 160 tiles; the oracle on sampled rows."""
    case = synth.small_dense(m, k, n, seed=m + bits)
    W = weights_to_device(case["w"], n, k)
    assert bb.w4a4_gemm_kernel_name(bits, m, W) == kernels[0 if bits == 4 else 1]
    rows = None if m <= 8 else sample_rows(m, 3, seed=m)
    check_gemm(case["x"], case["w"], n, k, bits, rows=rows, label="max K")


@pytest.mark.parametrize("bits,k", [(4, 6528), (4, 6560), (8, 3616), (8, 3648)])
@pytest.mark.parametrize("m", [5, 16])
def test_gemm_few_rows_staged_limit(torch, m, k, bits):
    """The weight-stream kernel stages its activation rows in LDS while they
    and the transposed row scales fit 64 KB: the largest such K for each code
    width, and one block more (rows read from L2 with every group)."""
    case = synth.small_dense(m, k, 64, seed=m + k + bits)
    W = weights_to_device(case["w"], 64, k)
    assert bb.w4a4_gemm_kernel_name(bits, m, W) == "weight-stream"
    check_gemm(case["x"], case["w"], 64, k, bits, label="few rows staged limit")


def test_gemm_few_rows_output_stride(torch):
    case = synth.small_dense(20, 160, 96, seed=5)
    codes, scales, q, d = quantize_and_check(case["x"], 8)
    W = weights_to_device(case["w"], 96, 160)
    ybig = torch.full((20, 132), -1.0, device="cuda")
    y = ybig[:, 8:104]
    bb.w4a4_gemm(codes, scales, 8, W, y=y)
    torch.cuda.synchronize()
    yb = ybig.cpu().numpy()
    assert np.all(yb[:, :8] == -1.0) and np.all(yb[:, 104:] == -1.0)
    w, dw = oracle.q4_0_decode(case["w"], 160)
    ref, a = oracle_rows(q, d, w, dw, None, 96)
    assert_within_bound(yb[:, 8:104], ref, a, 160, "few rows, strided")


def test_gemm_m0_is_noop(torch):
    case = synth.small_dense(4, 64, 32, seed=1)
    W = weights_to_device(case["w"], 32, 64)
    codes = torch.zeros((0, 32), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((0, 2), dtype=torch.float32, device="cuda")
    y = torch.full((0, 32), 7.0, device="cuda")
    bb.w4a4_gemm(codes, scales, 4, W, y=y)
    torch.cuda.synchronize()


def test_gemm_output_stride(torch):
    case = synth.small_dense(40, 128, 64, seed=2)
    codes, scales, q, d = quantize_and_check(case["x"], 4)
    W = weights_to_device(case["w"], 64, 128)
    ybig = torch.full((40, 100), -1.0, device="cuda")
    y = ybig[:, 4:68]
    assert y.stride(0) == 100
    bb.w4a4_gemm(codes, scales, 4, W, y=y)
    torch.cuda.synchronize()
    yb = ybig.cpu().numpy()
    assert np.all(yb[:, :4] == -1.0) and np.all(yb[:, 68:] == -1.0)
    w, dw = oracle.q4_0_decode(case["w"], 128)
    ref, a = oracle_rows(q, d, w, dw, None, 64)
    assert_within_bound(yb[:, 4:68], ref, a, 128, "strided")


@pytest.mark.parametrize("m,k,n,bits", [(200, 1056, 10240, 4),   # wide kernel
                                        (200, 1056, 10240, 8),   # tiled 64 x 160
                                        (96, 256, 640, 4),       # strip kernel
                                        (1000, 160, 12288, 8)])  # strip kernel, 8-bit
def test_gemm_output_stride_wide_shapes(torch, m, k, n, bits):
    """A row stride larger than N (the output a column slice of a wider
    matrix) on the kernels for many rows: columns outside the slice stay
    untouched."""
    case = synth.small_dense(m, k, n, seed=m + k + n + bits)
    codes, scales, q, d = quantize_and_check(case["x"], bits)
    W = weights_to_device(case["w"], n, k)
    ybig = torch.full((m, n + 40), -1.0, device="cuda")
    y = ybig[:, 8:8 + n]
    print("gemm stride", m, k, n, bits, flush=True)
    bb.w4a4_gemm(codes, scales, bits, W, y=y)
    torch.cuda.synchronize()
    yb = ybig.cpu().numpy()
    assert np.all(yb[:, :8] == -1.0) and np.all(yb[:, 8 + n:] == -1.0)
    w, dw = oracle.q4_0_decode(case["w"], k)
    rows = sample_rows(m, 8, seed=m)
    ref, a = oracle_rows(q, d, w, dw, rows, n)
    assert_within_bound(yb[rows, 8:8 + n], ref, a, k, "strided")


@pytest.mark.parametrize("bits", [4, 8])
def test_gemm_attn512_full_size(torch, bits):
    """The benchmarked workload, in the benchmarked launch configuration."""
    t = synth.make("attn512")
    check_gemm(t["x"], t["w"], 5120, 5120, bits, label="attn512")


@pytest.mark.parametrize("bits", [4, 8])
def test_gemm_ffn512_full_size(torch, bits):
    """Every output of the FFN pair (the up projection on sampled rows: it runs
    the gate's kernel on other weights)."""
    t = synth.make("ffn512")
    check_gemm(t["x1"], t["w_gate"], 17408, 5120, bits, label="ffn gate")
    check_gemm(t["x1"], t["w_up"], 17408, 5120, bits, rows=sample_rows(512, 8, seed=3),
               label="ffn up")
    check_gemm(t["x2"], t["w_down"], 5120, 17408, bits, label="ffn down")


@pytest.mark.parametrize("name,bits", [("m16_gate", 4), ("m16_down", 4), ("m16_attn", 4),
                                       ("m16_attn", 8)])
def test_gemm_m16_full_size(torch, name, bits):
    t = synth.make(name)
    c = t["cfg"]
    check_gemm(t["x"], t["w"], c["n"], c["k"], bits, label=name)


def test_long1024_routes_and_error_vs_unquantized(torch):
    """Both routes match the oracle on every output; report their error
    against the fp64 unquantized product (on sampled rows)."""
    t = synth.make("long1024")
    rows = sample_rows(1024, 6, seed=4)
    cols = np.arange(17408)
    w, dw = oracle.q4_0_decode(t["w"], 5120)
    rr, cc = np.meshgrid(rows, cols, indexing="ij")
    ref = oracle.ref_points(t["x"], w, dw, rr.ravel(), cc.ravel()).reshape(len(rows), -1)
    errs = {}
    for bits in (4, 8):
        y, _ = check_gemm(t["x"], t["w"], 17408, 5120, bits, label="long1024")
        errs[bits] = row_rel_err(y.cpu().numpy()[rows], ref)
    print("error vs fp64 unquantized: int4 %.4g, q8 %.4g" % (errs[4], errs[8]))
    assert errs[8] < errs[4] < 0.5


# ------------------------------------------------------------------ grouped GEMM

def check_grouped(x, blocks, offsets, n, k, E, bits, rows=None, label=""):
    torch = torch_mod()
    codes, scales, q, d = quantize_and_check(x, bits)
    W = weights_to_device(blocks, n, k, E)
    off = torch.from_numpy(offsets.astype(np.int32)).cuda()
    total = x.shape[0]
    print("grouped", label, total, n, k, E, bits, flush=True)
    y = torch.full((total, n), float("nan"), device="cuda")
    bb.w4a4_grouped_gemm(codes, scales, bits, off, W, y=y)
    torch.cuda.synchronize()
    wq, dwq = oracle.q4_0_decode(blocks.reshape(E * n, k // 32, 18), k)
    wq = wq.reshape(E, n, k)
    dwq = dwq.reshape(E, n, k // 32)
    rows = np.arange(total) if rows is None else rows
    rr, cc = np.meshgrid(rows, np.arange(n), indexing="ij")
    ref = oracle.grouped_points(q, d, offsets, wq, dwq, rr.ravel(), cc.ravel()).reshape(
        len(rows), n)
    a = oracle.grouped_abs_points(q, d, offsets, wq, dwq, rr.ravel(), cc.ravel()).reshape(
        len(rows), n)
    yg = y.cpu().numpy()[rows]
    err = row_rel_err(yg, ref)
    assert err <= TOL, err
    assert_within_bound(yg, ref, a, k, label)
    return y, codes, scales, q, W, wq


@pytest.mark.parametrize("bits", [4, 8])
def test_grouped_moe512(torch, bits):
    t = synth.make("moe512")
    off = t["offsets"]
    # rows across many experts, including the first and last rows of several
    rows = np.unique(np.concatenate([sample_rows(4096, 40, seed=bits), off[1:-1:9],
                                     off[1:-1:9] - 1]))
    check_grouped(t["x_gu"], t["w_gu"], off, 1536, 2048, 128, bits, rows=rows, label="gate/up")
    check_grouped(t["x_dn"], t["w_dn"], off, 2048, 768, 128, bits, rows=rows, label="down")


def test_grouped_ragged_experts(torch):
    rng = np.random.default_rng(41)
    E, n, k = 6, 64, 128
    counts = np.array([0, 1, 70, 0, 33, 129])            # empty, single, > 64, multi-slot
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    x, _ = synth.draw_activations(rng, int(off[-1]), k, "normal", 0.02, 20.0)
    blocks = synth.draw_q4_0(rng, (E, n), k, 0.005, 0.05)
    y, codes, scales, q, W, wq = check_grouped(x, blocks, off, n, k, E, 4, label="ragged")
    # block sums through an expert's weights match too
    check_blocksums(codes, scales, 4, W, q, wq[4], [(off[4], off[5], 0, 64)], expert=4)


@pytest.mark.parametrize("n,k,bits", [(256, 160, 4), (96, 128, 8), (128, 2080, 8), (64, 96, 4)])
def test_grouped_ragged_shapes(torch, n, k, bits):
    """Every grouped tile width (128, 64, 32 columns), K not a multiple of the
    stage or of four blocks, both activation widths."""
    rng = np.random.default_rng(n + k + bits)
    counts = np.array([5, 0, 40, 17, 32, 64, 1])
    E = counts.size
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    x, _ = synth.draw_activations(rng, int(off[-1]), k, "normal", 0.02, 20.0)
    blocks = synth.draw_q4_0(rng, (E, n), k, 0.005, 0.05)
    check_grouped(x, blocks, off, n, k, E, bits, label="ragged shapes")


def test_grouped_leaves_rows_outside_experts(torch):
    rng = np.random.default_rng(42)
    E, n, k, rows = 2, 32, 64, 10
    off = np.array([0, 3, 7], dtype=np.int32)           # rows 7..9 belong to no expert
    x, _ = synth.draw_activations(rng, rows, k, "normal")
    blocks = synth.draw_q4_0(rng, (E, n), k, 0.005, 0.05)
    y, *_ = check_grouped(x, blocks, off, n, k, E, 4, rows=np.arange(7), label="partial")
    assert np.all(np.isnan(y.cpu().numpy()[7:]))


# ------------------------------------------------------------------ determinism

def test_repeat_runs_are_bit_identical(torch):
    t = synth.make("attn512")
    xd = act_to_device(t["x"])
    W = weights_to_device(t["w"], 5120, 5120)
    outs = []
    for _ in range(2):
        codes, scales = bb.quantize_act_h32(xd, 4)
        outs.append(bb.w4a4_gemm(codes, scales, 4, W).cpu().numpy().view(np.uint32))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        codes, scales = bb.quantize_act_h32(xd, 4, stream=s)
        y = bb.w4a4_gemm(codes, scales, 4, W, stream=s)
    s.synchronize()
    outs.append(y.cpu().numpy().view(np.uint32))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
