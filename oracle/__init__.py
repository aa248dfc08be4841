"""CPU oracle for the Hadamard-rotated W4A4 prompt GEMM (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package; the product path
(``bit_prefill_gemm_amd``) never does.  The arithmetic lives in ``oracle.c``,
plain C loops written from the pages' description of the method (see the
header of that file for the passages and the readings taken).  This module
only marshals numpy arrays.

Parity status per function (what pins it is in ``tests/test_oracle_pins.py``):
every function here is pinned by at least one closed form, invariant,
library reduction or brute-force check; no function is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
          "-std=c11", "-Wall", "-Wextra"]


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc into liboracle.so (in place)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None

_i64 = ctypes.c_int64
_p = ctypes.c_void_p


def _load():
    global _lib
    if _lib is not None:
        return _lib
    lib = ctypes.CDLL(build())
    sig = {
        "orc_f16_to_f64": (ctypes.c_double, [ctypes.c_uint16]),
        "orc_f64_to_f16": (ctypes.c_uint16, [ctypes.c_double]),
        "orc_inv_sqrt32_f32": (ctypes.c_float, []),
        "orc_rotate_f32": (None, [_p, _p, _i64]),
        "orc_rotate_f64": (None, [_p, _p, _i64]),
        "orc_quantize": (_i64, [_p, ctypes.c_int, _i64, _i64, _i64, ctypes.c_int, ctypes.c_int,
                                _p, _p]),
        "orc_pack_int4": (None, [_p, _i64, _i64, _p]),
        "orc_q4_0_decode": (None, [_p, _i64, _i64, _p, _p]),
        "orc_quantize_weights_q4_0": (None, [_p, ctypes.c_int, _i64, _i64, ctypes.c_int, _p]),
        "orc_block_sums": (None, [_p, _p, _i64, _i64, _i64, _i64, _i64, _p]),
        "orc_gemm_rect": (None, [_p, _p, _p, _p, _i64, _i64, _i64, _i64, _i64, _p]),
        "orc_gemm_points": (None, [_p, _p, _p, _p, _i64, _p, _p, _i64, _p]),
        "orc_gemm_abs_rect": (None, [_p, _p, _p, _p, _i64, _i64, _i64, _i64, _i64, _p]),
        "orc_grouped_abs_points": (None, [_p, _p, _p, _i64, _p, _p, _i64, _i64, _p, _p, _i64,
                                          _p]),
        "orc_grouped_points": (None, [_p, _p, _p, _i64, _p, _p, _i64, _i64, _p, _p, _i64, _p]),
        "orc_ref_points": (None, [_p, ctypes.c_int, _i64, _p, _p, _i64, _p, _p, _i64, _p]),
        "orc_num_threads": (ctypes.c_int, []),
        "orc_exp_f32": (ctypes.c_float, [ctypes.c_float]),
        "orc_rotate_n_f32": (None, [_p, _p, _i64, ctypes.c_int]),
        "orc_rotate_n_f64": (None, [_p, _p, _i64, ctypes.c_int]),
        "orc_quantize_rot": (_i64, [_p, ctypes.c_int, _i64, _i64, _i64, ctypes.c_int, ctypes.c_int,
                                    _p, _p]),
        "orc_quantize_weights_q4_0_rot": (None, [_p, ctypes.c_int, _i64, _i64, ctypes.c_int, _p]),
        "orc_silu_f32": (ctypes.c_float, [ctypes.c_float]),
        "orc_swiglu_quantize": (_i64, [_p, _i64, _i64, _i64, ctypes.c_int, _p, _p]),
        "orc_moe_combine": (None, [_p, _i64, _p, _p, _i64, _i64, _i64, _p, _i64]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _act(x: np.ndarray):
    """Accept fp32 activations, or bf16 activations given as raw uint16 bits."""
    if x.dtype == np.float32:
        return np.ascontiguousarray(x), 0
    if x.dtype == np.uint16:
        return np.ascontiguousarray(x), 1
    raise TypeError("activations must be float32 or bf16 bits (uint16), got %s" % x.dtype)


# ---------------------------------------------------------------- scalars

def f16_to_f64(h: int) -> float:
    return _load().orc_f16_to_f64(int(h))


def f64_to_f16(x: float) -> int:
    return int(_load().orc_f64_to_f16(float(x)))


def inv_sqrt32_f32() -> np.float32:
    return np.float32(_load().orc_inv_sqrt32_f32())


# ---------------------------------------------------------------- rotation

def rotate_f32(x: np.ndarray) -> np.ndarray:
    """FWHT-32 per trailing block of 32 in fp32, then x fp32(1/sqrt 32)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    assert x.shape[-1] % 32 == 0
    v = np.empty_like(x)
    _load().orc_rotate_f32(_ptr(x), _ptr(v), x.size // 32)
    return v


def rotate_f64(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    assert x.shape[-1] % 32 == 0
    v = np.empty_like(x)
    _load().orc_rotate_f64(_ptr(x), _ptr(v), x.size // 32)
    return v


# ---------------------------------------------------------------- activations

def quantize(x: np.ndarray, bits: int = 4, rotate: bool = True):
    """Rotate (optionally) and quantize activations.

    Returns (q, d, ties): q int8 [m, k] code values in natural element order,
    d float32 [m, k/32] block scales, ties = number of exact .5 quotients.
    """
    assert bits in (4, 8)
    x, dt = _act(x)
    m, k = x.shape
    assert k % 32 == 0
    q = np.empty((m, k), dtype=np.int8)
    d = np.empty((m, k // 32), dtype=np.float32)
    ties = _load().orc_quantize(_ptr(x), dt, m, k, k, bits, 1 if rotate else 0, _ptr(q), _ptr(d))
    return q, d, int(ties)


def pack_int4(q: np.ndarray) -> np.ndarray:
    """Byte layout of 4-bit codes: [m, k/2], byte j of a block = q[j] | q[j+16] << 4."""
    q = np.ascontiguousarray(q, dtype=np.int8)
    m, k = q.shape
    out = np.empty((m, k // 2), dtype=np.uint8)
    _load().orc_pack_int4(_ptr(q), m, k, _ptr(out))
    return out


# ---------------------------------------------------------------- weights

def q4_0_decode(blocks: np.ndarray, k: int):
    """Canonical Q4_0 blocks (uint8 [..., k/32, 18]) -> (w int8 [rows, k], dw f64 [rows, k/32])."""
    blocks = np.ascontiguousarray(blocks, dtype=np.uint8)
    rows = blocks.size // (18 * (k // 32))
    w = np.empty((rows, k), dtype=np.int8)
    dw = np.empty((rows, k // 32), dtype=np.float64)
    _load().orc_q4_0_decode(_ptr(blocks), rows, k, _ptr(w), _ptr(dw))
    return w, dw


def quantize_weights_q4_0(w: np.ndarray, rotate: bool = True) -> np.ndarray:
    """Float weights [n, k] (fp32 or bf16 bits) -> canonical Q4_0 blocks [n, k/32, 18]."""
    w, dt = _act(w)
    n, k = w.shape
    out = np.empty((n, k // 32, 18), dtype=np.uint8)
    _load().orc_quantize_weights_q4_0(_ptr(w), dt, n, k, 1 if rotate else 0, _ptr(out))
    return out


# ---------------------------------------------------------------- products

def block_sums(q, w, m0, m1, n0, n1) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.int8)
    w = np.ascontiguousarray(w, dtype=np.int8)
    k = q.shape[1]
    assert w.shape[1] == k and 0 <= m0 <= m1 <= q.shape[0] and 0 <= n0 <= n1 <= w.shape[0]
    S = np.empty((m1 - m0, n1 - n0, k // 32), dtype=np.int32)
    _load().orc_block_sums(_ptr(q), _ptr(w), k, m0, m1, n0, n1, _ptr(S))
    return S


def gemm_rect(q, da, w, dw, m0, m1, n0, n1) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.int8)
    da = np.ascontiguousarray(da, dtype=np.float32)
    w = np.ascontiguousarray(w, dtype=np.int8)
    dw = np.ascontiguousarray(dw, dtype=np.float64)
    k = q.shape[1]
    assert w.shape[1] == k and 0 <= m0 <= m1 <= q.shape[0] and 0 <= n0 <= n1 <= w.shape[0]
    y = np.empty((m1 - m0, n1 - n0), dtype=np.float64)
    _load().orc_gemm_rect(_ptr(q), _ptr(da), _ptr(w), _ptr(dw), k, m0, m1, n0, n1, _ptr(y))
    return y


def gemm_abs_rect(q, da, w, dw, m0, m1, n0, n1) -> np.ndarray:
    """sum_b |da dw S| per output of the rectangle (the scale of the fp32 error bound)."""
    q = np.ascontiguousarray(q, dtype=np.int8)
    da = np.ascontiguousarray(da, dtype=np.float32)
    w = np.ascontiguousarray(w, dtype=np.int8)
    dw = np.ascontiguousarray(dw, dtype=np.float64)
    k = q.shape[1]
    assert w.shape[1] == k and 0 <= m0 <= m1 <= q.shape[0] and 0 <= n0 <= n1 <= w.shape[0]
    a = np.empty((m1 - m0, n1 - n0), dtype=np.float64)
    _load().orc_gemm_abs_rect(_ptr(q), _ptr(da), _ptr(w), _ptr(dw), k, m0, m1, n0, n1, _ptr(a))
    return a


def gemm_points(q, da, w, dw, rows, cols) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.int8)
    da = np.ascontiguousarray(da, dtype=np.float32)
    w = np.ascontiguousarray(w, dtype=np.int8)
    dw = np.ascontiguousarray(dw, dtype=np.float64)
    ri = np.ascontiguousarray(rows, dtype=np.int64)
    ci = np.ascontiguousarray(cols, dtype=np.int64)
    assert ri.shape == ci.shape
    assert ri.size == 0 or (ri.min() >= 0 and ri.max() < q.shape[0])
    assert ci.size == 0 or (ci.min() >= 0 and ci.max() < w.shape[0])
    y = np.empty(ri.shape, dtype=np.float64)
    _load().orc_gemm_points(_ptr(q), _ptr(da), _ptr(w), _ptr(dw), q.shape[1], _ptr(ri), _ptr(ci),
                            ri.size, _ptr(y))
    return y


def grouped_points(q, da, offsets, w, dw, rows, cols) -> np.ndarray:
    """w: int8 [E, n, k]; dw: f64 [E, n, k/32]; offsets int32 [E+1]."""
    q = np.ascontiguousarray(q, dtype=np.int8)
    da = np.ascontiguousarray(da, dtype=np.float32)
    off = np.ascontiguousarray(offsets, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.int8)
    dw = np.ascontiguousarray(dw, dtype=np.float64)
    E, n, k = w.shape
    assert off.shape == (E + 1,)
    ri = np.ascontiguousarray(rows, dtype=np.int64)
    ci = np.ascontiguousarray(cols, dtype=np.int64)
    y = np.empty(ri.shape, dtype=np.float64)
    _load().orc_grouped_points(_ptr(q), _ptr(da), _ptr(off), E, _ptr(w), _ptr(dw), n, k,
                               _ptr(ri), _ptr(ci), ri.size, _ptr(y))
    return y


def grouped_abs_points(q, da, offsets, w, dw, rows, cols) -> np.ndarray:
    """As grouped_points, with sum_b |da dw S| in place of the output."""
    q = np.ascontiguousarray(q, dtype=np.int8)
    da = np.ascontiguousarray(da, dtype=np.float32)
    off = np.ascontiguousarray(offsets, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.int8)
    dw = np.ascontiguousarray(dw, dtype=np.float64)
    E, n, k = w.shape
    assert off.shape == (E + 1,)
    ri = np.ascontiguousarray(rows, dtype=np.int64)
    ci = np.ascontiguousarray(cols, dtype=np.int64)
    a = np.empty(ri.shape, dtype=np.float64)
    _load().orc_grouped_abs_points(_ptr(q), _ptr(da), _ptr(off), E, _ptr(w), _ptr(dw), n, k,
                                   _ptr(ri), _ptr(ci), ri.size, _ptr(a))
    return a


def ref_points(x, w, dw, rows, cols) -> np.ndarray:
    """Unquantized fp64 reference (rotation in fp64 on both sides)."""
    x, dt = _act(x)
    w = np.ascontiguousarray(w, dtype=np.int8)
    dw = np.ascontiguousarray(dw, dtype=np.float64)
    ri = np.ascontiguousarray(rows, dtype=np.int64)
    ci = np.ascontiguousarray(cols, dtype=np.int64)
    y = np.empty(ri.shape, dtype=np.float64)
    _load().orc_ref_points(_ptr(x), dt, x.shape[1], _ptr(w), _ptr(dw), x.shape[1], _ptr(ri),
                           _ptr(ci), ri.size, _ptr(y))
    return y


def num_threads() -> int:
    return int(_load().orc_num_threads())


# ---------------------------------------------------------------- MoE glue

def exp_f32(x: np.ndarray) -> np.ndarray:
    """The fp32 exponential of the SwiGLU reading (elementwise)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    f = _load().orc_exp_f32
    return np.array([f(float(v)) for v in x.ravel()], dtype=np.float32).reshape(x.shape)


def silu_f32(g: np.ndarray) -> np.ndarray:
    g = np.ascontiguousarray(g, dtype=np.float32)
    f = _load().orc_silu_f32
    return np.array([f(float(v)) for v in g.ravel()], dtype=np.float32).reshape(g.shape)


def swiglu_quantize(gu: np.ndarray, inter: int, bits: int = 4):
    """gu: fp32 [rows, >= 2 inter] (gate then up).  Returns (q, d, ties) as quantize()."""
    gu = np.ascontiguousarray(gu, dtype=np.float32)
    rows, ld = gu.shape
    assert inter % 32 == 0 and ld >= 2 * inter and bits in (4, 8)
    q = np.empty((rows, inter), dtype=np.int8)
    d = np.empty((rows, inter // 32), dtype=np.float32)
    ties = _load().orc_swiglu_quantize(_ptr(gu), rows, inter, ld, bits, _ptr(q), _ptr(d))
    return q, d, int(ties)


def route_sort(expert_of: np.ndarray, experts: int):
    """Expert-sorted order of routed rows (token t, choice j) -> entry t*k + j.

    Stable by (expert, entry).  Returns (offsets int32 [E+1], row_entry int32
    [N]: the entry at each sorted position, slot_of int32 [N]: the sorted
    position of each entry)."""
    e = np.ascontiguousarray(expert_of, dtype=np.int64).ravel()
    assert e.size == 0 or (e.min() >= 0 and e.max() < experts)
    order = np.argsort(e, kind="stable")
    counts = np.bincount(e, minlength=experts)
    offsets = np.zeros(experts + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    slot_of = np.empty(e.size, dtype=np.int32)
    slot_of[order] = np.arange(e.size, dtype=np.int32)
    return offsets, order.astype(np.int32), slot_of


def moe_combine(dn: np.ndarray, slot_of: np.ndarray, weights: np.ndarray, tokens: int,
                topk: int) -> np.ndarray:
    dn = np.ascontiguousarray(dn, dtype=np.float32)
    slot = np.ascontiguousarray(slot_of, dtype=np.int32)
    w = np.ascontiguousarray(weights, dtype=np.float32)
    assert slot.size == tokens * topk and w.size == tokens * topk
    assert slot.size == 0 or (slot.min() >= 0 and slot.max() < dn.shape[0])
    hidden = dn.shape[1]
    out = np.empty((tokens, hidden), dtype=np.float32)
    _load().orc_moe_combine(_ptr(dn), dn.shape[1], _ptr(slot), _ptr(w), tokens, topk, hidden,
                            _ptr(out), hidden)
    return out


# ---------------------------------------------------------------- longer rotations

def rotate_n_f32(x: np.ndarray, n: int) -> np.ndarray:
    """H_n (Sylvester order) over each trailing span of n values, fp32, times fp32(1/sqrt n)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    assert n in (32, 64, 128) and x.shape[-1] % n == 0
    v = np.empty_like(x)
    _load().orc_rotate_n_f32(_ptr(x), _ptr(v), x.size // n, n)
    return v


def rotate_n_f64(x: np.ndarray, n: int) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    assert n in (32, 64, 128) and x.shape[-1] % n == 0
    v = np.empty_like(x)
    _load().orc_rotate_n_f64(_ptr(x), _ptr(v), x.size // n, n)
    return v


def quantize_rot(x: np.ndarray, rot: int, bits: int = 4):
    """Activation codes with rotation rot (0 = none, 32, 64, 128); as quantize()."""
    assert bits in (4, 8) and rot in (0, 32, 64, 128)
    x, dt = _act(x)
    m, k = x.shape
    assert k % max(rot, 32) == 0
    q = np.empty((m, k), dtype=np.int8)
    d = np.empty((m, k // 32), dtype=np.float32)
    ties = _load().orc_quantize_rot(_ptr(x), dt, m, k, k, bits, rot, _ptr(q), _ptr(d))
    return q, d, int(ties)


def quantize_weights_q4_0_rot(w: np.ndarray, rot: int) -> np.ndarray:
    """Float weights [n, k] -> canonical Q4_0 blocks [n, k/32, 18] with rotation rot."""
    assert rot in (0, 32, 64, 128)
    w, dt = _act(w)
    n, k = w.shape
    assert k % max(rot, 32) == 0
    out = np.empty((n, k // 32, 18), dtype=np.uint8)
    _load().orc_quantize_weights_q4_0_rot(_ptr(w), dt, n, k, rot, _ptr(out))
    return out
