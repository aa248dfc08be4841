"""The Python binding checks every tensor before it calls the C ABI (which sees
only pointers and sizes): shapes, dtypes and layouts first, devices last, so
each error below is raised as ValueError on a host without a GPU and before
any library call.  Also the host-only routing query.
"""
import ctypes

import numpy as np
import pytest
import torch

from bit_prefill_gemm_amd import binding as bb


def desc(n=64, k=128, e=1, rotation=32):
    d = bb.WeightsDesc()
    d.magic, d.version, d.rotation, d.layout = 0x57475042, 1, rotation, 3
    d.n, d.k, d.num_experts = n, k, e
    d.bytes = e * (n // 32) * ((k // 32 + 3) // 4) * 2304
    d.scales_offset = 2048
    return d


def weights(n=64, k=128, e=1, image_bytes=None):
    d = desc(n, k, e)
    nbytes = d.bytes if image_bytes is None else image_bytes
    return bb.Weights(d, torch.zeros(nbytes, dtype=torch.uint8))


def acts(m=4, k=128, bits=4):
    codes = torch.zeros((m, k // 2 if bits == 4 else k), dtype=torch.uint8)
    scales = torch.zeros((m, k // 32), dtype=torch.float32)
    return codes, scales


def raises(fn, *args, match, **kwargs):
    with pytest.raises(ValueError, match=match):
        fn(*args, **kwargs)


# ------------------------------------------------------------------ dense product

@pytest.mark.parametrize("fn", [bb.w4a4_gemm, bb.w4a4_gemm_unrotated, bb.w4a4_gemm_bf16])
def test_gemm_checks(fn):
    W = weights()
    codes, scales = acts()
    raises(fn, codes, scales, 3, W, match="act_bits")
    # 4-bit codes passed as 8-bit: each row would be read twice as long
    raises(fn, codes, scales, 8, W, match="codes has shape")
    raises(fn, codes[:, :-1], scales, 4, W, match="codes has shape")
    raises(fn, codes.to(torch.int32), scales, 4, W, match="codes has dtype")
    raises(fn, codes, scales[:3], 4, W, match="scales has shape")
    raises(fn, codes, scales.double(), 4, W, match="scales has dtype")
    raises(fn, codes, scales.t().contiguous().t(), 4, W, match="scales must be contiguous")
    wide = torch.zeros((4, 128), dtype=torch.uint8)
    raises(fn, wide[:, ::2], scales, 4, W, match="codes must be contiguous")
    raises(fn, codes, scales, 4, weights(image_bytes=100), match="weight image has 100 bytes")
    Wh = bb.Weights(desc(), np.zeros(desc().bytes, dtype=np.uint8))
    raises(fn, codes, scales, 4, Wh, match="on the host")
    ydt = torch.bfloat16 if fn is bb.w4a4_gemm_bf16 else torch.float32
    raises(fn, codes, scales, 4, W, y=torch.zeros((3, 64), dtype=ydt), match="y has shape")
    raises(fn, codes, scales, 4, W, y=torch.zeros((4, 64), dtype=torch.float16),
           match="y has dtype")
    raises(fn, codes, scales, 4, W, y=torch.zeros((64, 4), dtype=ydt).t(),
           match="unit column stride")
    # every shape right: stops at the device check (CPU tensors)
    raises(fn, codes, scales, 4, W, match="cuda device")
    raises(fn, codes, scales, 4, W, y=torch.zeros((4, 80), dtype=ydt)[:, 8:72],
           match="cuda device")


def test_gemm_8bit_shapes_pass_to_device_check():
    W = weights()
    codes, scales = acts(bits=8)
    raises(bb.w4a4_gemm, codes, scales, 8, W, match="cuda device")
    raises(bb.w4a4_gemm, codes.view(torch.int8), scales, 8, W, match="cuda device")
    raises(bb.w4a4_gemm, codes, scales, 4, W, match="codes has shape")


def test_gemm_rot_checks():
    W = weights()
    codes, scales = acts()
    raises(bb.w4a4_gemm_rot, codes[:, :32], scales, 4, 64, W, match="codes has shape")
    raises(bb.w4a4_gemm_rot, codes, scales, 4, 64, W, match="cuda device")


# ------------------------------------------------------------------ grouped product

@pytest.mark.parametrize("fn", [bb.w4a4_grouped_gemm, bb.w4a4_grouped_gemm_bf16])
def test_grouped_checks(fn):
    W = weights(e=3)
    codes, scales = acts(m=10)
    off = torch.tensor([0, 3, 7, 10], dtype=torch.int32)
    raises(fn, codes, scales, 4, off[:3], W, match="expert_offsets has shape")
    raises(fn, codes, scales, 4, off.long(), W, match="expert_offsets has dtype")
    raises(fn, codes, scales[:9], 4, off, W, match="scales has shape")
    raises(fn, codes, scales, 8, off, W, match="codes has shape")
    ydt = torch.bfloat16 if fn is bb.w4a4_grouped_gemm_bf16 else torch.float32
    raises(fn, codes, scales, 4, off, W, y=torch.zeros((9, 64), dtype=ydt), match="y has shape")
    raises(fn, codes, scales, 4, off, W, match="cuda device")


def test_gather_checks():
    W = weights(e=3)
    codes, scales = acts(m=6)
    ids = torch.zeros(10, dtype=torch.int32)
    off = torch.tensor([0, 3, 7, 10], dtype=torch.int32)
    fn = bb.w4a4_grouped_gemm_gather
    raises(fn, codes, scales, 4, ids.long(), off, W, match="row_ids has dtype")
    raises(fn, codes, scales, 4, ids.view(2, 5), off, W, match="row_ids must be a 1-D")
    raises(fn, codes, scales, 4, ids, off[1:], W, match="expert_offsets has shape")
    raises(fn, codes, scales[:5], 4, ids, off, W, match="scales has shape")
    raises(fn, codes, scales, 4, ids, off, W, y=torch.zeros((6, 64)), match="y has shape")
    raises(fn, codes, scales, 4, ids, off, W, match="cuda device")


def test_blocksums_checks():
    W = weights()
    codes, scales = acts(m=8)
    fn = bb.w4a4_gemm_blocksums
    raises(fn, codes, scales, 4, W, 0, 9, 0, 64, match="outside")
    raises(fn, codes, scales, 4, W, 0, 8, 0, 96, match="outside")
    raises(fn, codes, scales, 4, W, 5, 4, 0, 64, match="outside")
    raises(fn, codes, scales, 4, W, 0, 8, 0, 64, expert=1, match="outside")
    raises(fn, codes, scales, 4, W, 0, 8, 0, 64,
           sums=torch.zeros((8, 64, 3), dtype=torch.int32), match="sums has shape")
    raises(fn, codes, scales, 4, W, 0, 8, 0, 64,
           sums=torch.zeros((8, 64, 4), dtype=torch.int64), match="sums has dtype")
    raises(fn, codes, None, 4, W, 0, 8, 0, 64, match="cuda device")


# ------------------------------------------------------------------ quantizers and glue

@pytest.mark.parametrize("fn", [bb.quantize_act_h32, bb.quantize_act_unrotated])
def test_quantize_checks(fn):
    x = torch.zeros((4, 128), dtype=torch.float32)
    codes, scales = acts()
    raises(fn, x, 4, codes=codes[:3], match="codes has shape")
    raises(fn, x, 8, codes=codes, match="codes has shape")
    raises(fn, x, 4, codes=codes, scales=scales[:, :3], match="scales has shape")
    raises(fn, x, 5, match="act_bits")
    raises(fn, torch.zeros((4, 100)), 4, match="not a multiple of 32")
    raises(fn, torch.zeros((8, 128))[:, ::2], 4, match="unit stride")
    with pytest.raises(TypeError):
        fn(x.double(), 4)
    raises(fn, x, 4, match="cuda device")


def test_quantize_rot_checks():
    raises(bb.quantize_act_rot, torch.zeros((4, 96)), 64, 4, match="multiple of 64")
    raises(bb.quantize_act_rot, torch.zeros((4, 128)), 48, 4, match="rotation")
    raises(bb.quantize_act_rot, torch.zeros((4, 128)), 128, 4, match="cuda device")


def test_route_sort_checks():
    e = torch.zeros(12, dtype=torch.int32)
    raises(bb.moe_route_sort, e, 4, 2, 8, match="expert_of has shape")
    raises(bb.moe_route_sort, e.long(), 4, 3, 8, match="expert_of has dtype")
    raises(bb.moe_route_sort, e, 4, 3, 8, match="cuda device")


def test_swiglu_checks():
    gu = torch.zeros((5, 128), dtype=torch.float32)
    fn = bb.swiglu_quantize_h32
    raises(fn, gu, 96, match="inter")
    raises(fn, gu, 48, match="inter")
    raises(fn, gu.double(), 64, match="float32")
    raises(fn, gu, 64, codes=torch.zeros((5, 64), dtype=torch.uint8), match="codes has shape")
    raises(fn, gu, 64, 8, codes=torch.zeros((5, 64), dtype=torch.uint8),
           scales=torch.zeros((5, 3)), match="scales has shape")
    raises(fn, gu, 64, match="cuda device")


def test_combine_checks():
    dn = torch.zeros((12, 64), dtype=torch.float32)
    slot = torch.zeros(8, dtype=torch.int32)
    wts = torch.zeros(8, dtype=torch.float32)
    fn = bb.moe_combine
    raises(fn, dn, slot[:7], wts, 4, 2, match="slot_of has shape")
    raises(fn, dn, slot, wts.double(), 4, 2, match="weights has dtype")
    raises(fn, dn, slot, wts, 4, 2, y=torch.zeros((4, 32)), match="y has shape")
    raises(fn, dn.t(), slot, wts, 4, 2, match="unit stride")
    raises(fn, dn, slot, wts, 4, 2, match="cuda device")


# ------------------------------------------------------------------ routing query

@pytest.mark.parametrize("bits,m,k,n,kernel", [
    (4, 512, 5120, 5120, "wide 64x160"), (8, 512, 5120, 5120, "tiled 64x160"),
    (4, 512, 5120, 17408, "strip 32x128"), (8, 512, 5120, 17408, "strip 32x128"),
    (4, 512, 17408, 5120, "wide 64x160"), (8, 512, 17408, 5120, "tiled 64x160"),
    (4, 1024, 5120, 17408, "strip 32x128"), (8, 1024, 5120, 17408, "strip 32x128"),
    (4, 16, 5120, 17408, "weight-stream"), (8, 16, 17408, 5120, "weight-stream"),
    (4, 32, 256, 128, "weight-stream"), (4, 16, 32800, 64, "tiled 16x32"),
    (4, 0, 256, 128, "none")])
def test_gemm_kernel_name(bits, m, k, n, kernel):
    W = bb.Weights(desc(n, k), None)
    assert bb.w4a4_gemm_kernel_name(bits, m, W) == kernel


def test_grouped_kernel_name():
    W = bb.Weights(desc(1536, 2048, 128), None)
    assert bb.w4a4_grouped_gemm_kernel_name(4, 4096, W) == "expert-slot"
    assert bb.w4a4_grouped_gemm_kernel_name(4, 4096, W, src_rows=512) == "expert-slot"
    assert bb.w4a4_grouped_gemm_kernel_name(8, 4096, W) == "grouped 32x128"
    assert bb.w4a4_grouped_gemm_kernel_name(4, 100, bb.Weights(desc(96, 256, 4), None)) == \
        "grouped 32x32"
    assert bb.w4a4_grouped_gemm_kernel_name(4, 0, W) == "none"


def test_kernel_name_refuses_bad_arguments():
    lib = bb.lib()
    d = desc()
    assert lib.w4a4_gemm_kernel_name(3, 4, ctypes.byref(d)) is None
    assert lib.w4a4_gemm_kernel_name(4, -1, ctypes.byref(d)) is None
    assert lib.w4a4_gemm_kernel_name(4, 4, None) is None
    bad = desc()
    bad.magic = 0
    assert lib.w4a4_gemm_kernel_name(4, 4, ctypes.byref(bad)) is None
    assert lib.w4a4_gemm_kernel_name(4, 4, ctypes.byref(desc(e=2))) is None
    assert lib.w4a4_grouped_gemm_kernel_name(4, 4, 0, ctypes.byref(desc(rotation=0))) is None
    assert lib.w4a4_grouped_gemm_kernel_name(4, 4, -1, ctypes.byref(d)) is None
    with pytest.raises(ValueError):
        bb.w4a4_gemm_kernel_name(5, 4, bb.Weights(d, None))
