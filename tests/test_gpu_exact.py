"""Exact int32 block sums on every kernel the products route to, shown through
the products themselves ("509 tokens a second of prompt: the Hadamard route
ships", section "Why prompts are a matrix-unit problem": the product is
integer matrix work over Q4_0 codes; the route must give the same block sums
as the plain definition).

The wide, strip, weight-stream, tiled and expert-slot kernels never write
their block sums S; they apply the scales in an fp32 epilogue.  Two choices
of scales make that epilogue exact, so the output pins S:

  1. every weight scale 2^e (e in [-9, -6], as fp16) and every activation
     scale 2^e (e in [-3, 0]): every term da*dw*S is an integer multiple of
     2^-12, so while sum_b |da*dw*S| < 2^24 * 2^-12 (checked with the oracle)
     every partial sum in any order is exact in fp32, and the whole output
     must equal the oracle's fp64 output bit for bit.  One wrong S anywhere
     changes an output by at least 2^-12;
  2. activation scale 1 on one block b and 0 on every other: the output is
     dw[n][b] * S[m][n][b] exactly, so S of that block is read back for every
     (m, n) and compared with the oracle's block sums.  Blocks are chosen in
     the first, a middle and the last stage, in each K wave of the wide
     kernel and in the last (partial) group.

Each case runs at its workload's full size, in the configuration the
benchmark times, and first asserts which kernel the routing picks.
"""
import zlib

import numpy as np
import pytest

import oracle
from bit_prefill_gemm_amd import binding as bb
from bit_prefill_gemm_amd import synth

from gpu_util import pow2_blocks, pow2_scales, quantize_and_check, torch_mod

pytestmark = pytest.mark.gpu

W_EXP = (-9, -6)   # weight scales 2^-9 .. 2^-6 (the workloads' 0.002 .. 0.02)
A_EXP = (-3, 0)    # activation scales 2^-3 .. 1
UNIT = 2.0 ** (W_EXP[0] + A_EXP[0])


@pytest.fixture(scope="module")
def torch():
    t = torch_mod()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    return t


def masked_blocks(nblk):
    """Blocks to read back one at a time: K waves 0..3 of the wide kernel's
    first stage (groups 0..3), the first block of the second stage, a middle
    block and the last group (the last one partial when B % 4 != 0)."""
    cand = [0, 3, 4, 9, 14, 15, 16, nblk // 2 + 1, nblk - 4, nblk - 2, nblk - 1]
    return sorted({b for b in cand if 0 <= b < nblk})


def seed_of(label):
    return zlib.crc32(label.encode())


def exact_output(y, ref, a, what):
    assert a.max() < 2.0 ** 24 * UNIT, "%s: exactness precondition fails (%g)" % (what, a.max())
    got = y.astype(np.float64)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, "%s: %d outputs differ, first %s: %r vs %r (step %g)" % (
        what, len(bad), bad[0].tolist(), got[tuple(bad[0])], ref[tuple(bad[0])], UNIT)


def exact_block(y, S, dwb, what, b):
    """y[m][n] must be dw[n][b] * S[m][n] exactly; reports S mismatches."""
    got = y.astype(np.float64) / dwb[None, :]
    bad = np.argwhere(got != S)
    assert bad.size == 0, "%s: block %d: %d block sums differ, first %s: %r vs %d" % (
        what, b, len(bad), bad[0].tolist(), got[tuple(bad[0])], S[tuple(bad[0])])


DENSE = [
    # workload, activation key, weight key, bits, kernel
    ("attn512", "x", "w", 4, "wide 64x160"),
    ("attn512", "x", "w", 8, "tiled 64x160"),
    ("ffn512", "x1", "w_gate", 4, "strip 32x128"),
    ("ffn512", "x1", "w_gate", 8, "strip 32x128"),
    ("ffn512", "x2", "w_down", 4, "wide 64x160"),
    ("ffn512", "x2", "w_down", 8, "tiled 64x160"),
    ("long1024", "x", "w", 4, "strip 32x128"),
    ("long1024", "x", "w", 8, "strip 32x128"),
    ("m16_gate", "x", "w", 4, "weight-stream"),
    ("m16_gate", "x", "w", 8, "weight-stream"),
    ("m16_down", "x", "w", 4, "weight-stream"),
    ("m16_down", "x", "w", 8, "weight-stream"),
    ("m16_attn", "x", "w", 4, "weight-stream"),
    ("m16_attn", "x", "w", 8, "weight-stream"),
    ("tiny", "x", "w", 4, "weight-stream"),
    ("tiny", "x", "w", 8, "weight-stream"),
]


@pytest.mark.parametrize("name,xkey,wkey,bits,kernel", DENSE,
                         ids=["%s-%s-%d" % (c[0], c[2], c[3]) for c in DENSE])
def test_dense_block_sums_exact(torch, name, xkey, wkey, bits, kernel):
    t = synth.make(name)
    x, blocks = t[xkey], t[wkey]
    m, k = x.shape
    n = blocks.shape[0]
    nblk = k // 32
    label = "%s %s %d-bit" % (name, wkey, bits)
    rng = np.random.default_rng(seed_of(label))
    codes, _, q, _ = quantize_and_check(x, bits)
    pblocks = pow2_blocks(blocks, rng, *W_EXP)
    W = bb.rotate_pack_weights(pblocks, bb.SRC_Q4_0_ROTATED, n, k).to("cuda")
    assert bb.w4a4_gemm_kernel_name(bits, m, W) == kernel
    w, dw = oracle.q4_0_decode(pblocks, k)

    # 1. power-of-two scales: the whole output exact
    da = pow2_scales(m, nblk, rng, *A_EXP)
    print("exact", label, kernel, flush=True)
    y = bb.w4a4_gemm(codes, torch.from_numpy(da).cuda(), bits, W)
    torch.cuda.synchronize()
    ref = oracle.gemm_rect(q, da, w, dw, 0, m, 0, n)
    a = oracle.gemm_abs_rect(q, da, w, dw, 0, m, 0, n)
    exact_output(y.cpu().numpy(), ref, a, label)

    # 2. one block at a time: S read back for every (m, n)
    for b in masked_blocks(nblk):
        dm = np.zeros((m, nblk), dtype=np.float32)
        dm[:, b] = 1.0
        print("masked", label, "block", b, flush=True)
        y = bb.w4a4_gemm(codes, torch.from_numpy(dm).cuda(), bits, W)
        torch.cuda.synchronize()
        qb = np.ascontiguousarray(q[:, 32 * b:32 * b + 32])
        wb = np.ascontiguousarray(w[:, 32 * b:32 * b + 32])
        S = oracle.block_sums(qb, wb, 0, m, 0, n)[:, :, 0]
        exact_block(y.cpu().numpy(), S, dw[:, b], label, b)


def expert_decode(pblocks, n, k, E):
    w, dw = oracle.q4_0_decode(pblocks.reshape(E * n, k // 32, 18), k)
    return w.reshape(E, n, k), dw.reshape(E, n, k // 32)


def grouped_rect(fn, q, d, off, wq, dwq):
    """fn (oracle.gemm_rect or gemm_abs_rect) over each expert's rows, all columns."""
    E, n, _ = wq.shape
    out = np.full((q.shape[0], n), np.nan)
    for e in range(E):
        if off[e + 1] > off[e]:
            out[off[e]:off[e + 1]] = fn(q, d, wq[e], dwq[e], off[e], off[e + 1], 0, n)
    return out


GROUPED = [
    # which projection, bits, gathered rows, kernel
    ("gu", 4, False, "expert-slot"),
    ("gu", 4, True, "expert-slot"),
    ("dn", 4, False, "expert-slot"),
    ("gu", 8, False, "grouped 32x128"),
    ("dn", 8, False, "grouped 32x128"),
]


@pytest.mark.parametrize("which,bits,gather,kernel", GROUPED,
                         ids=["%s-%d%s" % (c[0], c[1], "-gather" if c[2] else "")
                              for c in GROUPED])
def test_grouped_block_sums_exact(torch, which, bits, gather, kernel):
    t = synth.make("moe512")
    cfg = t["cfg"]
    E, H, I = cfg["experts"], cfg["hidden"], cfg["inter"]
    n, k = (2 * I, H) if which == "gu" else (H, I)
    off = t["offsets"].astype(np.int32)
    total = int(off[-1])
    nblk = k // 32
    label = "moe512 %s %d-bit%s" % (which, bits, " gathered" if gather else "")
    rng = np.random.default_rng(seed_of(label))
    if gather:
        # the tokens are quantized once; sorted row r reads token row_token[r]
        codes, _, q_tok, _ = quantize_and_check(t["x_tokens"], bits)
        ids = t["token_of_row"].astype(np.int32)
        q = q_tok[ids]
        src = q_tok.shape[0]
    else:
        x = t["x_gu"] if which == "gu" else t["x_dn"]
        codes, _, q, _ = quantize_and_check(x, bits)
        src = total
    pblocks = pow2_blocks(t["w_gu"] if which == "gu" else t["w_dn"], rng, *W_EXP)
    W = bb.rotate_pack_weights(pblocks, bb.SRC_Q4_0_ROTATED, n, k, E).to("cuda")
    assert bb.w4a4_grouped_gemm_kernel_name(bits, total, W, src_rows=src if gather else 0) == kernel
    wq, dwq = expert_decode(pblocks, n, k, E)
    offd = torch.from_numpy(off).cuda()
    idd = torch.from_numpy(ids).cuda() if gather else None

    def run(da_src):
        dd = torch.from_numpy(da_src).cuda()
        if gather:
            y = bb.w4a4_grouped_gemm_gather(codes, dd, bits, idd, offd, W)
        else:
            y = bb.w4a4_grouped_gemm(codes, dd, bits, offd, W)
        torch.cuda.synchronize()
        return y.cpu().numpy()

    # 1. power-of-two scales: every output exact
    da_src = pow2_scales(src, nblk, rng, *A_EXP)
    da = da_src[ids] if gather else da_src
    print("exact", label, kernel, flush=True)
    y = run(da_src)
    ref = grouped_rect(oracle.gemm_rect, q, da, off, wq, dwq)
    a = grouped_rect(oracle.gemm_abs_rect, q, da, off, wq, dwq)
    exact_output(y, ref, a, label)

    # 2. one block at a time, each row against its expert's weights
    for b in masked_blocks(nblk):
        dm = np.zeros((src, nblk), dtype=np.float32)
        dm[:, b] = 1.0
        print("masked", label, "block", b, flush=True)
        y = run(dm)
        qb = np.ascontiguousarray(q[:, 32 * b:32 * b + 32])
        for e in range(E):
            r0, r1 = int(off[e]), int(off[e + 1])
            if r1 == r0:
                continue
            wb = np.ascontiguousarray(wq[e][:, 32 * b:32 * b + 32])
            S = oracle.block_sums(qb, wb, r0, r1, 0, n)[:, :, 0]
            exact_block(y[r0:r1], S, dwq[e][:, b], "%s expert %d" % (label, e), b)
