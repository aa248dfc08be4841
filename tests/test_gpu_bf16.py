"""GPU parity of the bf16-output variants: every element equals the fp32
variant's result rounded to bf16 (round to nearest even), bit for bit, on each
kernel family (wide 4-bit tiles, the strip kernel, tiled 8-bit, the weight-stream kernel for a
few rows, the expert-slot kernel, the tiled grouped kernel); the bf16 result
is also within bf16 rounding of the oracle; grouped rows outside every
expert's range stay untouched.
"""
import numpy as np
import pytest

import oracle
from bit_prefill_gemm_amd import binding as bb
from bit_prefill_gemm_amd import synth

from gpu_util import act_to_device, row_rel_err, sample_rows, torch_mod, weights_to_device

pytestmark = pytest.mark.gpu

# bf16 keeps 8 significant bits: rounding to nearest moves an element by at
# most half a unit in its last place, 2^-8 of it relative; the fp32 result is
# itself within 2e-5 row-L2 of the oracle
BF16_TOL = 2.0 ** -8 + 2e-5


@pytest.fixture(scope="module")
def torch():
    t = torch_mod()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    return t


def quantized(x, bits):
    codes, scales = bb.quantize_act_h32(act_to_device(x), bits)
    q, d, _ = oracle.quantize(x, bits)
    return codes, scales, q, d


@pytest.mark.parametrize("m,k,n,bits", [
    (200, 1056, 10240, 4),   # wide kernel, 64x160 tiles, ragged rows
    (130, 512, 1024, 4),     # strip kernel
    (1000, 448, 12288, 4),   # strip kernel, ragged last strip
    (130, 1056, 1024, 8),    # strip kernel, 8-bit
    (77, 320, 96, 8),        # tiled kernel, 8-bit
    (16, 2048, 512, 4),      # weight-stream kernel
    (5, 96, 64, 8),          # weight-stream kernel, 8-bit, tiny
])
def test_dense_bf16_is_rounded_fp32(torch, m, k, n, bits):
    rng = np.random.default_rng(m + k + n + bits)
    x, _ = synth.draw_activations(rng, m, k, "normal", 0.02, 20.0)
    blocks = synth.draw_q4_0(rng, (n,), k, 0.005, 0.05)
    codes, scales, q, d = quantized(x, bits)
    W = weights_to_device(blocks, n, k)
    print("bf16 dense", m, k, n, bits, flush=True)
    y32 = bb.w4a4_gemm(codes, scales, bits, W)
    y16 = bb.w4a4_gemm_bf16(codes, scales, bits, W)
    torch.cuda.synchronize()
    assert y16.dtype == torch.bfloat16
    assert torch.equal(y16.view(torch.int16), y32.to(torch.bfloat16).view(torch.int16))
    wq, dwq = oracle.q4_0_decode(blocks, k)
    rows = sample_rows(m, 8, seed=m)
    rr, cc = np.meshgrid(rows, np.arange(n), indexing="ij")
    ref = oracle.gemm_points(q, d, wq, dwq, rr.ravel(), cc.ravel()).reshape(len(rows), n)
    assert row_rel_err(y16.float().cpu().numpy()[rows], ref) <= BF16_TOL


def test_dense_bf16_output_stride(torch):
    rng = np.random.default_rng(61)
    m, k, n = 96, 256, 640
    x, _ = synth.draw_activations(rng, m, k, "normal")
    blocks = synth.draw_q4_0(rng, (n,), k, 0.005, 0.05)
    codes, scales, _, _ = quantized(x, 4)
    W = weights_to_device(blocks, n, k)
    big = torch.full((m, n + 24), 7.0, dtype=torch.bfloat16, device="cuda")
    y16 = bb.w4a4_gemm_bf16(codes, scales, 4, W, y=big[:, :n])
    y32 = bb.w4a4_gemm(codes, scales, 4, W)
    torch.cuda.synchronize()
    assert torch.equal(big[:, :n].view(torch.int16), y32.to(torch.bfloat16).view(torch.int16))
    assert torch.all(big[:, n:] == 7.0)


@pytest.mark.parametrize("n,k,bits", [(384, 1056, 4), (96, 160, 8)])
def test_grouped_bf16_is_rounded_fp32(torch, n, k, bits):
    """The expert-slot kernel (4-bit, N % 128 == 0) and the tiled grouped kernel
    (8-bit); rows 0..2 belong to no expert and stay untouched."""
    rng = np.random.default_rng(n + k + bits)
    counts = np.array([0, 1, 32, 33, 70, 5, 130])
    off = np.concatenate([[3], 3 + np.cumsum(counts)]).astype(np.int32)
    total = int(off[-1]) + 4
    E = counts.size
    x, _ = synth.draw_activations(rng, total, k, "normal", 0.02, 20.0)
    blocks = synth.draw_q4_0(rng, (E, n), k, 0.005, 0.05)
    codes, scales, q, d = quantized(x, bits)
    W = bb.rotate_pack_weights(blocks, bb.SRC_Q4_0_ROTATED, n, k, E).to("cuda")
    offd = torch.from_numpy(off).cuda()
    print("bf16 grouped", n, k, bits, flush=True)
    y16 = torch.full((total, n), float("nan"), dtype=torch.bfloat16, device="cuda")
    bb.w4a4_grouped_gemm_bf16(codes, scales, bits, offd, W, y=y16)
    y32 = bb.w4a4_grouped_gemm(codes, scales, bits, offd, W)
    torch.cuda.synchronize()
    inside = slice(int(off[0]), int(off[-1]))
    assert torch.equal(y16[inside].view(torch.int16),
                       y32[inside].to(torch.bfloat16).view(torch.int16))
    assert torch.all(torch.isnan(y16[:int(off[0])])) and torch.all(torch.isnan(y16[int(off[-1]):]))
    wq, dwq = oracle.q4_0_decode(blocks.reshape(E * n, k // 32, 18), k)
    rows = np.arange(int(off[0]), int(off[-1]), 7)
    rr, cc = np.meshgrid(rows, np.arange(n), indexing="ij")
    ref = oracle.grouped_points(q, d, off, wq.reshape(E, n, k), dwq.reshape(E, n, k // 32),
                                rr.ravel(), cc.ravel()).reshape(len(rows), n)
    assert row_rel_err(y16.float().cpu().numpy()[rows], ref) <= BF16_TOL
