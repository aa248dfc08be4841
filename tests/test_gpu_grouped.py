"""GPU parity of the grouped product on 64-row expert slots (the kernel that
runs 4-bit grouped products with N a multiple of 128 and at most 1024
experts): slot shapes (empty experts, one row, 32, 33, 64, 65 and several
slots per expert), K with a partial last stage, with a single stage and long
(2^18), many
experts (the slot lookup over several chunks of the table), fewer work items
than compute units, gathered rows with repeats, repeat runs, and offsets that
break the ordering rule (accesses stay in bounds; rows that exactly one
expert owns are still right).

Bar: within 1e-3 row-L2 of the oracle's fp64 output on the same codes, and
every compared element within the fp32 accumulation bound; gathered rows
bit-identical to the same product on explicitly permuted rows.
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


def offsets_of(counts):
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)


def quantized(x):
    torch = torch_mod()
    codes, scales = bb.quantize_act_h32(act_to_device(x), 4)
    q, d, _ = oracle.quantize(x, 4)
    torch.cuda.synchronize()
    assert np.array_equal(codes.cpu().numpy(), oracle_codes(q, 4))
    return codes, scales, q, d


def expert_weights(blocks, n, k, E):
    W = bb.rotate_pack_weights(blocks, bb.SRC_Q4_0_ROTATED, n, k, E).to("cuda")
    wq, dwq = oracle.q4_0_decode(blocks.reshape(E * n, k // 32, 18), k)
    return W, wq.reshape(E, n, k), dwq.reshape(E, n, k // 32)


def edge_rows(off, extra, seed):
    """First and last row of every expert plus a random sample."""
    total = int(off[-1])
    firsts = off[:-1][off[1:] > off[:-1]]
    lasts = off[1:][off[1:] > off[:-1]] - 1
    return np.unique(np.concatenate([firsts, lasts, sample_rows(total, extra, seed)]))


def run_grouped(counts, n, k, seed, rows_extra=40):
    torch = torch_mod()
    rng = np.random.default_rng(seed)
    E = len(counts)
    off = offsets_of(counts)
    total = int(off[-1])
    x, _ = synth.draw_activations(rng, total, k, "normal", 0.02, 20.0)
    blocks = synth.draw_q4_0(rng, (E, n), k, 0.005, 0.05)
    codes, scales, q, d = quantized(x)
    W, wq, dwq = expert_weights(blocks, n, k, E)
    offd = torch.from_numpy(off).cuda()
    print("grouped slots", E, total, n, k, flush=True)
    y = torch.full((total, n), float("nan"), device="cuda")
    bb.w4a4_grouped_gemm(codes, scales, 4, offd, W, y=y)
    torch.cuda.synchronize()
    rows = edge_rows(off, rows_extra, seed)
    yg = y.cpu().numpy()
    check_grouped_rows(yg[rows], q, d, off, wq, dwq, rows, k, "slots", TOL)
    return yg, codes, scales, offd, W


def test_slot_shapes_and_partial_last_stage(torch):
    # empty, one row, 32, 33, 64, 65 (64 + 1), 97 (64 + 33), 128, 200 (3 x 64 + 8);
    # K = 1056: 33 blocks, the third stage holds one block
    run_grouped([0, 1, 32, 33, 64, 65, 97, 128, 200], 384, 1056, seed=51)


def test_single_stage_k(torch):
    # K = 160: five blocks, one stage with two groups (the second partial)
    run_grouped([3, 70, 0, 31, 64], 256, 160, seed=52)


def test_many_experts_lookup(torch):
    # 1000 experts with 0..3 rows: the slot lookup reads four chunks of the table
    rng = np.random.default_rng(53)
    counts = rng.integers(0, 4, size=1000)
    run_grouped(counts, 128, 64, seed=53, rows_extra=80)


@pytest.mark.parametrize("E,kernel", [(1024, "expert-slot"), (1025, "grouped 32x128")])
def test_expert_count_limit(torch, E, kernel):
    """The slot table holds 1024 experts (four full chunks of the lookup); one
    expert more routes to the tiled grouped kernel."""
    rng = np.random.default_rng(E)
    counts = rng.integers(0, 3, size=E)
    blocks = synth.draw_q4_0(rng, (E, 128), 64, 0.005, 0.05)
    W = bb.rotate_pack_weights(blocks, bb.SRC_Q4_0_ROTATED, 128, 64, E)
    assert bb.w4a4_grouped_gemm_kernel_name(4, int(counts.sum()), W) == kernel
    run_grouped(counts, 128, 64, seed=E, rows_extra=60)


def test_long_k(torch):
    # K = 2^18 (8192 blocks, 1024 stages of two groups per item): the weight
    # image offsets of an expert and the rows' code offsets far from zero
    run_grouped([33, 0, 70], 128, 1 << 18, seed=56, rows_extra=8)


def test_fewer_items_than_compute_units(torch):
    run_grouped([5, 40], 128, 512, seed=54)


def test_repeat_runs_bit_identical(torch):
    y, codes, scales, offd, W = run_grouped([20, 47, 64, 1, 90], 512, 2048, seed=55)
    y2 = bb.w4a4_grouped_gemm(codes, scales, 4, offd, W)
    torch.cuda.synchronize()
    assert np.array_equal(y.view(np.uint32), y2.cpu().numpy().view(np.uint32))


def test_gathered_rows_with_repeats(torch):
    rng = np.random.default_rng(56)
    counts = np.array([0, 1, 32, 33, 64, 65, 97, 0, 130])
    E, n, k, src = counts.size, 256, 1056, 150
    off = offsets_of(counts)
    total = int(off[-1])
    x, _ = synth.draw_activations(rng, src, k, "normal", 0.02, 20.0)
    blocks = synth.draw_q4_0(rng, (E, n), k, 0.005, 0.05)
    codes, scales, q, d = quantized(x)
    W, wq, dwq = expert_weights(blocks, n, k, E)
    ids = rng.integers(0, src, size=total).astype(np.int32)   # repeats, any order
    offd = torch.from_numpy(off).cuda()
    idd = torch.from_numpy(ids).cuda()
    print("gathered slots", total, src, flush=True)
    y = bb.w4a4_grouped_gemm_gather(codes, scales, 4, idd, offd, W)
    il = idd.long()
    y2 = bb.w4a4_grouped_gemm(codes[il].contiguous(), scales[il].contiguous(), 4, offd, W)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    rows = edge_rows(off, 40, 56)
    check_grouped_rows(y.cpu().numpy()[rows], q[ids], d[ids], off, wq, dwq, rows, k, "gathered",
                       TOL)


def test_offsets_that_break_the_rule_stay_in_bounds(torch):
    """Offsets clamped to [0, rows]; an expert whose end is before its start
    owns no rows.  Rows that exactly one expert's clamped range holds are
    that expert's product; y has no row past total_rows to overwrite (the
    output is allocated with exactly total_rows rows)."""
    rng = np.random.default_rng(57)
    E, n, k, total = 6, 128, 256, 60
    off = np.array([-7, 10, 5, 40, 40, 1000, 55], dtype=np.int32)
    x, _ = synth.draw_activations(rng, total, k, "normal")
    blocks = synth.draw_q4_0(rng, (E, n), k, 0.005, 0.05)
    codes, scales, q, d = quantized(x)
    W, wq, dwq = expert_weights(blocks, n, k, E)
    offd = torch.from_numpy(off).cuda()
    y = torch.full((total, n), float("nan"), device="cuda")
    print("broken offsets", flush=True)
    bb.w4a4_grouped_gemm(codes, scales, 4, offd, W, y=y)
    torch.cuda.synchronize()
    yg = y.cpu().numpy()
    lo = np.clip(off[:-1], 0, total)
    hi = np.clip(off[1:], 0, total)
    owners = [[e for e in range(E) if lo[e] <= r < hi[e]] for r in range(total)]
    cols = np.arange(n)
    for e in range(E):
        rows = np.array([r for r in range(total) if owners[r] == [e]], dtype=np.int64)
        if rows.size == 0:
            continue
        rr, cc = np.meshgrid(rows, cols, indexing="ij")
        ref = oracle.gemm_points(q, d, wq[e], dwq[e], rr.ravel(), cc.ravel()).reshape(
            rows.size, n)
        a = np.concatenate([oracle.gemm_abs_rect(q, d, wq[e], dwq[e], r, r + 1, 0, n)
                            for r in rows])
        err = row_rel_err(yg[rows], ref)
        assert err <= TOL, (e, err)
        assert_within_bound(yg[rows], ref, a, k, "expert %d" % e)
    # rows no expert owns stay untouched
    free = [r for r in range(total) if not owners[r]]
    assert np.all(np.isnan(yg[free]))
