"""The C ABI: the library loads without a GPU, exports every declared entry
point, and reports every argument and stamp error from the host, before any
HIP call.  Pointers used here are never dereferenced: each call fails its
checks first (or, for the last test, at the device check on a GPU-less host).
"""
import ctypes
import os
import re

import numpy as np
import pytest

from bit_prefill_gemm_amd import binding as bb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bpg.h")

OK, NULL, SHAPE, ALIGN, DTYPE, STAMP, BUFFER, DEVICE = 0, 1, 2, 3, 4, 5, 6, 7

P = ctypes.c_void_p(0x100000)        # aligned, never dereferenced
P2 = ctypes.c_void_p(0x200000)
MIS = ctypes.c_void_p(0x100004)      # 4-byte aligned only
NUL = ctypes.c_void_p(0)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w \*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_function():
    lib = bb.lib()
    names = declared_functions()
    assert set(names) == set(bb.ENTRY_POINTS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    lib = bb.lib()
    for s in range(9):
        assert lib.bpg_status_str(s)
    assert b"unknown" in lib.bpg_status_str(99)


def good_desc(n=64, k=128, e=1):
    d = bb.WeightsDesc()
    d.magic, d.version, d.rotation, d.layout = 0x57475042, 1, 32, 3
    d.n, d.k, d.num_experts = n, k, e
    groups = (k // 32 + 3) // 4
    d.bytes = e * (n // 32) * groups * 2304
    d.scales_offset = 2048
    return d


def q(x=P, dt=0, m=4, k=128, ldx=128, bits=4, codes=P2, scales=P, stream=NUL):
    return bb.lib().quantize_act_h32(x, dt, m, k, ldx, bits, codes, scales, stream)


def gemm(codes=P, scales=P2, bits=4, m=4, desc=None, wdev=P, y=P2, ldy=64, stream=NUL):
    d = desc if desc is not None else good_desc()
    return bb.lib().w4a4_gemm(codes, scales, bits, m, ctypes.byref(d), wdev, y, ldy, stream)


def grouped(codes=P, scales=P2, bits=4, rows=4, off=P, desc=None, wdev=P, y=P2, ldy=64,
            stream=NUL):
    d = desc if desc is not None else good_desc(e=3)
    return bb.lib().w4a4_grouped_gemm(codes, scales, bits, rows, off, ctypes.byref(d), wdev, y,
                                      ldy, stream)


def sums(codes=P, scales=P2, bits=4, m=4, desc=None, wdev=P, expert=0, m0=0, m1=4, n0=0,
         n1=64, out=P2, stream=NUL):
    d = desc if desc is not None else good_desc()
    return bb.lib().w4a4_gemm_blocksums(codes, scales, bits, m, ctypes.byref(d), wdev, expert,
                                        m0, m1, n0, n1, out, stream)


@pytest.mark.parametrize("kwargs,status", [
    (dict(dt=2), DTYPE), (dict(bits=3), DTYPE), (dict(bits=16), DTYPE),
    (dict(k=100, ldx=100), SHAPE), (dict(k=0, ldx=0), SHAPE), (dict(m=-1), SHAPE),
    (dict(ldx=96), SHAPE),
    (dict(x=NUL), NULL), (dict(codes=NUL), NULL), (dict(scales=NUL), NULL),
    (dict(x=MIS), ALIGN), (dict(codes=MIS), ALIGN), (dict(ldx=130), ALIGN),
])
def test_quantize_errors(kwargs, status):
    assert q(**kwargs) == status


def _desc_with(**kw):
    d = good_desc()
    for a, v in kw.items():
        setattr(d, a, v)
    return d


@pytest.mark.parametrize("kwargs,status", [
    (dict(desc=_desc_with(magic=0)), STAMP),
    (dict(desc=_desc_with(version=2)), STAMP),
    (dict(desc=_desc_with(rotation=0)), STAMP),      # an unrotated image is refused
    (dict(desc=_desc_with(rotation=64)), STAMP),
    (dict(desc=_desc_with(layout=0)), STAMP),
    (dict(desc=_desc_with(layout=1)), STAMP),        # earlier layouts
    (dict(desc=_desc_with(layout=2)), STAMP),
    (dict(desc=_desc_with(bytes=1)), STAMP),
    (dict(desc=_desc_with(scales_offset=8)), STAMP),
    (dict(desc=_desc_with(n=48)), STAMP),
    (dict(desc=good_desc(e=2)), STAMP),              # dense call on an expert image
    (dict(bits=2), DTYPE), (dict(m=-3), SHAPE), (dict(ldy=32), SHAPE),
    (dict(codes=NUL), NULL), (dict(scales=NUL), NULL), (dict(wdev=NUL), NULL),
    (dict(y=NUL), NULL), (dict(y=MIS), ALIGN), (dict(codes=MIS), ALIGN), (dict(ldy=66), ALIGN),
])
def test_gemm_errors(kwargs, status):
    assert gemm(**kwargs) == status


def test_zero_rows_accept_null_buffers():
    """Empty tensors may carry NULL pointers; with no rows nothing is touched."""
    if os.path.exists("/dev/kfd"):
        pytest.skip("host has a GPU driver")
    assert q(x=NUL, codes=NUL, scales=NUL, m=0) == DEVICE
    assert gemm(codes=NUL, scales=NUL, y=NUL, m=0) == DEVICE
    assert gemm(codes=NUL, m=1) == NULL


def test_gemm_k_limit():
    """K up to 2^22 passes every host check (then the device check, without a
    GPU); one block more is refused before any HIP call."""
    if os.path.exists("/dev/kfd"):
        pytest.skip("host has a GPU driver")
    assert gemm(desc=good_desc(k=1 << 22)) == DEVICE
    assert gemm(desc=good_desc(k=(1 << 22) + 32)) == SHAPE
    assert sums(desc=good_desc(k=(1 << 22) + 32)) == SHAPE


def test_gemm_null_desc():
    lib = bb.lib()
    assert lib.w4a4_gemm(P, P2, 4, 4, None, P, P2, 64, NUL) == NULL


@pytest.mark.parametrize("kwargs,status", [
    (dict(off=NUL), NULL), (dict(off=ctypes.c_void_p(0x100002)), ALIGN),
    (dict(bits=7), DTYPE), (dict(rows=-1), SHAPE),
    (dict(desc=_desc_with(magic=1)), STAMP),
])
def test_grouped_errors(kwargs, status):
    assert grouped(**kwargs) == status


@pytest.mark.parametrize("kwargs,status", [
    (dict(m0=3, m1=2), SHAPE), (dict(m1=5), SHAPE), (dict(n1=65), SHAPE), (dict(n0=-1), SHAPE),
    (dict(expert=1), SHAPE), (dict(expert=-1), SHAPE), (dict(out=NUL), NULL),
    (dict(bits=1), DTYPE), (dict(out=MIS), ALIGN), (dict(desc=_desc_with(rotation=16)), STAMP),
])
def test_blocksum_errors(kwargs, status):
    assert sums(**kwargs) == status


def test_pack_errors():
    lib = bb.lib()
    d = bb.WeightsDesc()
    src = np.zeros(64 * 4 * 18, dtype=np.uint8)
    dst = np.zeros(64 * 4 * 18, dtype=np.uint8)
    sp, dp = src.ctypes.data_as(ctypes.c_void_p), dst.ctypes.data_as(ctypes.c_void_p)
    assert lib.rotate_pack_weights(sp, 9, 64, 128, 1, dp, dst.nbytes, ctypes.byref(d)) == DTYPE
    assert lib.rotate_pack_weights(sp, 2, 48, 128, 1, dp, dst.nbytes, ctypes.byref(d)) == SHAPE
    assert lib.rotate_pack_weights(sp, 2, 64, 100, 1, dp, dst.nbytes, ctypes.byref(d)) == SHAPE
    assert lib.rotate_pack_weights(sp, 2, 64, 128, 0, dp, dst.nbytes, ctypes.byref(d)) == SHAPE
    assert lib.rotate_pack_weights(NUL, 2, 64, 128, 1, dp, dst.nbytes, ctypes.byref(d)) == NULL
    assert lib.rotate_pack_weights(sp, 2, 64, 128, 1, dp, dst.nbytes - 1, ctypes.byref(d)) == BUFFER
    assert lib.rotate_pack_weights(sp, 2, 64, 128, 1, dp, dst.nbytes, ctypes.byref(d)) == OK
    assert lib.rotate_pack_weights_bytes(64, 128, 1) == 64 * 4 * 18
    assert lib.rotate_pack_weights_bytes(64, 160, 1) == 2 * 2 * 2304   # two groups, three pad blocks
    assert lib.rotate_pack_weights_bytes(63, 128, 1) == 0
    assert lib.rotate_pack_weights_bytes(64, 128, -1) == 0


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="host has a GPU driver")
def test_valid_calls_stop_at_device_check_without_gpu():
    assert q() == DEVICE
    assert gemm() == DEVICE
    assert grouped() == DEVICE
    assert sums() == DEVICE


def test_binding_raises_typed_error():
    with pytest.raises(bb.BpgError) as ei:
        bb.rotate_pack_weights(np.zeros(10, dtype=np.uint8), 7, 64, 128)
    assert ei.value.status == DTYPE


# ------------------------------------------------------------ unrotated route

def gemm_u(desc=None, **kw):
    d = desc if desc is not None else _desc_with(rotation=0)
    a = dict(codes=P, scales=P2, bits=4, m=4, wdev=P, y=P2, ldy=64, stream=NUL)
    a.update(kw)
    return bb.lib().w4a4_gemm_unrotated(a["codes"], a["scales"], a["bits"], a["m"],
                                        ctypes.byref(d), a["wdev"], a["y"], a["ldy"], a["stream"])


def q_u(**kw):
    a = dict(x=P, dt=0, m=4, k=128, ldx=128, bits=4, codes=P2, scales=P, stream=NUL)
    a.update(kw)
    return bb.lib().quantize_act_unrotated(a["x"], a["dt"], a["m"], a["k"], a["ldx"], a["bits"],
                                           a["codes"], a["scales"], a["stream"])


@pytest.mark.parametrize("kwargs,status", [
    (dict(desc=good_desc()), STAMP),                 # a rotated image is refused
    (dict(desc=_desc_with(rotation=0, magic=3)), STAMP),
    (dict(desc=_desc_with(rotation=0, bytes=5)), STAMP),
    (dict(bits=5), DTYPE), (dict(ldy=32), SHAPE), (dict(y=NUL), NULL), (dict(y=MIS), ALIGN),
])
def test_unrotated_gemm_errors(kwargs, status):
    assert gemm_u(**kwargs) == status


@pytest.mark.parametrize("kwargs,status", [
    (dict(dt=5), DTYPE), (dict(bits=2), DTYPE), (dict(k=48, ldx=48), SHAPE),
    (dict(x=NUL), NULL), (dict(codes=MIS), ALIGN),
])
def test_unrotated_quantize_errors(kwargs, status):
    assert q_u(**kwargs) == status


def test_unrotated_pack_errors_and_stamp():
    lib = bb.lib()
    d = bb.WeightsDesc()
    src = np.zeros(64 * 4 * 18, dtype=np.uint8)
    dst = np.zeros(64 * 4 * 18, dtype=np.uint8)
    sp, dp = src.ctypes.data_as(ctypes.c_void_p), dst.ctypes.data_as(ctypes.c_void_p)
    # each packer takes only its own route's Q4_0 tensors
    assert lib.pack_weights_unrotated(sp, 2, 64, 128, 1, dp, dst.nbytes, ctypes.byref(d)) == DTYPE
    assert lib.rotate_pack_weights(sp, 3, 64, 128, 1, dp, dst.nbytes, ctypes.byref(d)) == DTYPE
    assert lib.pack_weights_unrotated(sp, 3, 64, 100, 1, dp, dst.nbytes, ctypes.byref(d)) == SHAPE
    assert lib.pack_weights_unrotated(sp, 3, 64, 128, 1, NUL, dst.nbytes, ctypes.byref(d)) == NULL
    assert lib.pack_weights_unrotated(sp, 3, 64, 128, 1, dp, 100, ctypes.byref(d)) == BUFFER
    assert lib.pack_weights_unrotated(sp, 3, 64, 128, 1, dp, dst.nbytes, ctypes.byref(d)) == OK
    assert d.rotation == 0 and d.layout == 3 and d.bytes == dst.nbytes
    # the rotated route refuses the unrotated image, and blocksums / grouped do too
    assert gemm(desc=d) == STAMP
    assert sums(desc=d) == STAMP


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="host has a GPU driver")
def test_unrotated_valid_calls_stop_at_device_check_without_gpu():
    assert q_u() == DEVICE
    assert gemm_u() == DEVICE


# ------------------------------------------------------------ expert layer glue

def test_route_sort_errors():
    lib = bb.lib()
    f = lambda **kw: lib.moe_route_sort(kw.get("e", P), kw.get("t", 4), kw.get("k", 2),
                                        kw.get("E", 8), kw.get("off", P2), kw.get("rt", P),
                                        kw.get("so", P2), NUL)
    assert f(E=0) == SHAPE and f(E=513) == SHAPE and f(k=0) == SHAPE and f(t=-1) == SHAPE
    assert f(t=1 << 20, k=2) == SHAPE
    assert f(off=NUL) == NULL and f(e=NUL) == NULL and f(rt=NUL) == NULL
    assert f(so=ctypes.c_void_p(0x200002)) == ALIGN
    if not os.path.exists("/dev/kfd"):
        assert f() == DEVICE
        assert f(t=0, e=NUL, rt=NUL, so=NUL) == DEVICE


def test_gather_errors():
    lib = bb.lib()
    d = good_desc(e=3)
    f = lambda **kw: lib.w4a4_grouped_gemm_gather(
        kw.get("codes", P), kw.get("scales", P2), kw.get("bits", 4), kw.get("src", 10),
        kw.get("ids", P), kw.get("rows", 4), kw.get("off", P), ctypes.byref(kw.get("desc", d)),
        kw.get("wdev", P), kw.get("y", P2), kw.get("ldy", 64), NUL)
    assert f(ids=NUL) == NULL
    assert f(src=0) == SHAPE and f(src=-1) == SHAPE and f(rows=-2) == SHAPE
    assert f(src=1 << 30) == SHAPE           # gathered rows need 32-bit offsets
    assert f(ids=ctypes.c_void_p(0x100002)) == ALIGN
    assert f(bits=5) == DTYPE and f(desc=_desc_with(magic=2)) == STAMP
    if not os.path.exists("/dev/kfd"):
        assert f() == DEVICE


def test_swiglu_quantize_errors():
    lib = bb.lib()
    f = lambda **kw: lib.swiglu_quantize_h32(kw.get("gu", P), kw.get("rows", 4),
                                             kw.get("inter", 64), kw.get("ld", 128),
                                             kw.get("bits", 4), kw.get("codes", P2),
                                             kw.get("scales", P), NUL)
    assert f(bits=3) == DTYPE
    assert f(inter=48) == SHAPE and f(ld=127) == SHAPE and f(rows=-1) == SHAPE
    assert f(gu=NUL) == NULL and f(codes=NUL) == NULL
    assert f(gu=MIS) == ALIGN and f(ld=130) == ALIGN
    if not os.path.exists("/dev/kfd"):
        assert f() == DEVICE
        assert f(rows=0, gu=NUL, codes=NUL, scales=NUL) == DEVICE


def test_combine_errors():
    lib = bb.lib()
    f = lambda **kw: lib.moe_combine(kw.get("dn", P), kw.get("lddn", 64), kw.get("rows", 8),
                                     kw.get("slot", P2), kw.get("w", P), kw.get("t", 4),
                                     kw.get("k", 2), kw.get("h", 64), kw.get("y", P2),
                                     kw.get("ldy", 64), NUL)
    assert f(h=62) == SHAPE and f(lddn=32) == SHAPE and f(ldy=32) == SHAPE and f(k=0) == SHAPE
    assert f(rows=0) == SHAPE
    assert f(dn=NUL) == NULL and f(slot=NUL) == NULL and f(w=NUL) == NULL and f(y=NUL) == NULL
    assert f(dn=MIS) == ALIGN and f(lddn=66) == ALIGN and f(w=ctypes.c_void_p(0x100002)) == ALIGN
    if not os.path.exists("/dev/kfd"):
        assert f() == DEVICE


# ------------------------------------------------------------ longer rotations

def test_rotation_length_errors():
    lib = bb.lib()
    d = bb.WeightsDesc()
    src = np.zeros(64 * 8 * 18, dtype=np.uint8)
    dst = np.zeros(64 * 8 * 18, dtype=np.uint8)
    sp, dp = src.ctypes.data_as(ctypes.c_void_p), dst.ctypes.data_as(ctypes.c_void_p)
    for r in (0, 16, 96, 256):
        assert lib.rotate_pack_weights_rot(sp, 2, 64, 256, 1, r, dp, dst.nbytes, ctypes.byref(d)) == SHAPE
        assert lib.quantize_act_rot(P, 0, 4, 256, 256, 4, r, P2, P, NUL) == SHAPE
    # K must be a multiple of the span
    assert lib.rotate_pack_weights_rot(sp, 0, 64, 160, 1, 64, dp, dst.nbytes, ctypes.byref(d)) == SHAPE
    assert lib.quantize_act_rot(P, 0, 4, 192, 192, 4, 128, P2, P, NUL) == SHAPE
    assert lib.rotate_pack_weights_rot(sp, 3, 64, 256, 1, 64, dp, dst.nbytes, ctypes.byref(d)) == DTYPE
    assert lib.rotate_pack_weights_rot(sp, 2, 64, 256, 1, 128, dp, dst.nbytes, ctypes.byref(d)) == OK
    assert d.rotation == 128
    # the product checks the span against the stamp
    dd = _desc_with(rotation=128)
    g = lambda r, desc: lib.w4a4_gemm_rot(P, P2, 4, r, 4, ctypes.byref(desc), P, P2, 64, NUL)
    assert g(64, dd) == STAMP and g(96, dd) == SHAPE
    assert gemm(desc=dd) == STAMP
    if not os.path.exists("/dev/kfd"):
        assert g(128, dd) == DEVICE
        assert g(32, good_desc()) == DEVICE
        assert lib.quantize_act_rot(P, 0, 4, 256, 256, 4, 64, P2, P, NUL) == DEVICE


def gemm_b(desc=None, **kw):
    d = desc if desc is not None else good_desc()
    a = dict(codes=P, scales=P2, bits=4, m=4, wdev=P, y=P2, ldy=64, stream=NUL)
    a.update(kw)
    return bb.lib().w4a4_gemm_bf16(a["codes"], a["scales"], a["bits"], a["m"], ctypes.byref(d),
                                   a["wdev"], a["y"], a["ldy"], a["stream"])


def grouped_b(desc=None, **kw):
    d = desc if desc is not None else good_desc(e=3)
    a = dict(codes=P, scales=P2, bits=4, rows=4, off=P, wdev=P, y=P2, ldy=64, stream=NUL)
    a.update(kw)
    return bb.lib().w4a4_grouped_gemm_bf16(a["codes"], a["scales"], a["bits"], a["rows"],
                                           a["off"], ctypes.byref(d), a["wdev"], a["y"],
                                           a["ldy"], a["stream"])


@pytest.mark.parametrize("kwargs,status", [
    (dict(desc=_desc_with(magic=0)), STAMP), (dict(desc=good_desc(e=2)), STAMP),
    (dict(bits=2), DTYPE), (dict(m=-3), SHAPE), (dict(ldy=32), SHAPE),
    (dict(codes=NUL), NULL), (dict(y=NUL), NULL), (dict(y=MIS), ALIGN),
    (dict(ldy=68), ALIGN),                           # bf16 rows: ldy % 8 (16-byte rows)
])
def test_gemm_bf16_errors(kwargs, status):
    assert gemm_b(**kwargs) == status


@pytest.mark.parametrize("kwargs,status", [
    (dict(off=NUL), NULL), (dict(y=MIS), ALIGN), (dict(ldy=68), ALIGN), (dict(bits=7), DTYPE),
    (dict(rows=-1), SHAPE), (dict(ldy=16), SHAPE), (dict(desc=_desc_with(magic=1)), STAMP),
])
def test_grouped_bf16_errors(kwargs, status):
    assert grouped_b(**kwargs) == status


def test_bf16_ldy_multiple_of_8_passes_checks():
    """A bf16 output with ldy a multiple of 8 (not of 16) passes every argument check; on a
    host without a GPU the call then stops at the device check."""
    if os.path.exists("/dev/kfd"):
        pytest.skip("host has a GPU driver")
    assert gemm_b(ldy=72) == DEVICE
    assert grouped_b(ldy=72) == DEVICE
