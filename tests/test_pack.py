"""rotate_pack_weights (host code of the library) against the documented image
layout and, for float sources, bit-exact against the oracle's offline path."""
import numpy as np
import pytest

import oracle
from bit_prefill_gemm_amd import binding as bb
from bit_prefill_gemm_amd import synth


def image_regions(img: np.ndarray, n: int, k: int, e: int):
    """The documented layout: one 2304-byte block per (expert, tile, group of four
    blocks): codes uint32 [4 slots][32 cols][4 blocks], then scales fp16 bits
    [16][2][4 blocks] (column 16h + c16 at [c16][h]).  Returns codes
    [e][n/32][G][4][32][4] and scales [e][n/32][G][32 cols][4 blocks]."""
    B = k // 32
    G, T = (B + 3) // 4, n // 32
    assert img.size == e * T * G * 2304
    blk = img.reshape(e, T, G, 2304)
    codes = np.ascontiguousarray(blk[..., :2048]).view("<u4").reshape(e, T, G, 4, 32, 4)
    sc = np.ascontiguousarray(blk[..., 2048:]).view("<u2").reshape(e, T, G, 16, 2, 4)
    scales = sc.transpose(0, 1, 2, 4, 3, 5).reshape(e, T, G, 32, 4)   # [h][c16] -> column
    return codes, scales


def unpack_image(img: np.ndarray, n: int, k: int, e: int) -> np.ndarray:
    """Read the image back per its documented layout into canonical blocks [e, n, k/32, 18]."""
    B = k // 32
    codes, scales = image_regions(img, n, k, e)
    out = np.empty((e, n, B, 18), dtype=np.uint8)
    for b in range(B):
        gi, q = divmod(b, 4)
        d = np.ascontiguousarray(codes[:, :, gi, :, :, q].transpose(0, 1, 3, 2))  # [e][t][c][slot]
        out[:, :, b, 2:] = d.view(np.uint8).reshape(e, n, 16)
        sc = np.ascontiguousarray(scales[:, :, gi, :, q]).reshape(e, n)
        out[:, :, b, 0:2] = sc.view(np.uint8).reshape(e, n, 2)
    return out


def test_blocks_past_k_are_zero_valued():
    """K = 160 (5 blocks): the second group's last three blocks are padding,
    codes 0x88 (u = 8, value 0) and scale 0."""
    n, k = 64, 160
    blocks = synth.draw_q4_0(np.random.default_rng(7), (n,), k, 0.002, 0.02)
    W = bb.rotate_pack_weights(blocks, bb.SRC_Q4_0_ROTATED, n, k, 1)
    codes, scales = image_regions(W.image, n, k, 1)
    pad_codes = codes[:, :, 1, :, :, 1:]
    assert np.all(pad_codes == 0x88888888)
    assert np.all(scales[:, :, 1, :, 1:] == 0)


@pytest.mark.parametrize("n,k,e", [(32, 32, 1), (96, 160, 1), (64, 256, 3), (32, 416, 2)])
def test_q4_0_source_is_relaid_out_verbatim(n, k, e):
    blocks = synth.draw_q4_0(np.random.default_rng(n + k + e), (e, n), k, 0.002, 0.02)
    W = bb.rotate_pack_weights(blocks, bb.SRC_Q4_0_ROTATED, n, k, e)
    assert W.desc.rotation == 32 and W.desc.num_experts == e
    assert np.array_equal(unpack_image(W.image, n, k, e), blocks)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_float_source_matches_oracle_bit_exact(dtype):
    rng = np.random.default_rng(21)
    n, k, e = 64, 320, 2
    w = rng.standard_normal((e * n, k)).astype(np.float32) * 0.03
    w[:, rng.choice(k, 6, replace=False)] *= 12.0          # outlier input channels
    w[3, 32:64] = 0.0                                       # an all-zero block
    w[5, 64:96] = 1e-6                                      # a tiny constant block
    w[6, 96:128] = 1e-9                                     # fp16(amax/7) underflows: codes 8
    w[7, :32] = 1e-40                                       # fp32 subnormal weights
    w[8, 32:64] = 0.0
    w[8, 40] = -2e-5                                        # fp16-subnormal scale
    src = w if dtype == "f32" else synth.bf16_bits(w)
    kind = bb.SRC_F32 if dtype == "f32" else bb.SRC_BF16
    W = bb.rotate_pack_weights(src, kind, n, k, e)
    got = unpack_image(W.image, n, k, e).reshape(e * n, k // 32, 18)
    ref = oracle.quantize_weights_q4_0(src, rotate=True)
    assert np.array_equal(got, ref)


def test_float_source_reproduces_unrotated_product():
    """Packed float weights stand for H w / sqrt(32): the route's product is x . w."""
    rng = np.random.default_rng(22)
    n, k = 32, 128
    w = rng.standard_normal((n, k)).astype(np.float32) * 0.05
    W = bb.rotate_pack_weights(w, bb.SRC_F32, n, k, 1)
    blocks = unpack_image(W.image, n, k, 1)[0]
    wq, dw = oracle.q4_0_decode(blocks, k)
    x = rng.standard_normal((4, k)).astype(np.float32)
    rows, cols = np.meshgrid(np.arange(4), np.arange(n), indexing="ij")
    y = oracle.ref_points(x, wq, dw, rows.ravel(), cols.ravel()).reshape(4, n)
    exact = x.astype(np.float64) @ w.astype(np.float64).T
    assert np.linalg.norm(y - exact) / np.linalg.norm(exact) < 0.1


# ------------------------------------------------------------ unrotated route

@pytest.mark.parametrize("n,k,e", [(32, 32, 1), (96, 160, 1), (64, 256, 2)])
def test_unrotated_q4_0_source_is_relaid_out_verbatim(n, k, e):
    blocks = synth.draw_q4_0(np.random.default_rng(5 * n + k + e), (e, n), k, 0.002, 0.02)
    W = bb.pack_weights_unrotated(blocks, bb.SRC_Q4_0, n, k, e)
    assert W.desc.rotation == 0 and W.desc.num_experts == e
    assert np.array_equal(unpack_image(W.image, n, k, e), blocks)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_unrotated_float_source_matches_oracle_bit_exact(dtype):
    rng = np.random.default_rng(23)
    n, k, e = 64, 288, 2
    w = synth.draw_weights_f32(rng, e * n, k, 0.03)
    w[:, rng.choice(k, 5, replace=False)] *= 10.0
    w[7, 96:128] = 0.0
    src = w if dtype == "f32" else synth.bf16_bits(w)
    kind = bb.SRC_F32 if dtype == "f32" else bb.SRC_BF16
    W = bb.pack_weights_unrotated(src, kind, n, k, e)
    got = unpack_image(W.image, n, k, e).reshape(e * n, k // 32, 18)
    ref = oracle.quantize_weights_q4_0(src, rotate=False)
    assert np.array_equal(got, ref)
    # and the two routes differ: the rotated image holds other blocks
    R = bb.rotate_pack_weights(src, kind, n, k, e)
    assert not np.array_equal(unpack_image(R.image, n, k, e).reshape(e * n, k // 32, 18), got)


# ------------------------------------------------------------ longer rotations

@pytest.mark.parametrize("rot", [32, 64, 128])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_rot_float_source_matches_oracle_bit_exact(rot, dtype):
    rng = np.random.default_rng(rot + len(dtype))
    n, k, e = 64, 384, 2
    w = synth.draw_weights_f32(rng, e * n, k, 0.03)
    w[:, rng.choice(k, 4, replace=False)] *= 15.0
    src = w if dtype == "f32" else synth.bf16_bits(w)
    kind = bb.SRC_F32 if dtype == "f32" else bb.SRC_BF16
    W = bb.rotate_pack_weights_rot(src, kind, n, k, rot, e)
    assert W.desc.rotation == rot
    got = unpack_image(W.image, n, k, e).reshape(e * n, k // 32, 18)
    assert np.array_equal(got, oracle.quantize_weights_q4_0_rot(src, rot))
    if rot == 32:
        R = bb.rotate_pack_weights(src, kind, n, k, e)
        assert np.array_equal(R.image, W.image)
