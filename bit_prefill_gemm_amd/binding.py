"""Thin Python binding over libbpg.so (the C ABI in include/bpg.h).

Argument marshalling only: every step of the route runs in the library's HIP
kernels (or, for rotate_pack_weights, in its host code).  PyTorch provides
device memory and streams.  If the library has not been built, the first call
raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbpg.so")

BPG_OK = 0
STATUS_NAMES = {0: "BPG_OK", 1: "BPG_ERR_NULL", 2: "BPG_ERR_SHAPE", 3: "BPG_ERR_ALIGN",
                4: "BPG_ERR_DTYPE", 5: "BPG_ERR_STAMP", 6: "BPG_ERR_BUFFER",
                7: "BPG_ERR_DEVICE", 8: "BPG_ERR_LAUNCH"}

SRC_F32, SRC_BF16, SRC_Q4_0_ROTATED, SRC_Q4_0 = 0, 1, 2, 3
X_F32, X_BF16 = 0, 1

ENTRY_POINTS = ("bpg_status_str", "rotate_pack_weights_bytes", "rotate_pack_weights",
                "quantize_act_h32", "w4a4_gemm", "w4a4_grouped_gemm", "w4a4_gemm_blocksums",
                "pack_weights_unrotated", "quantize_act_unrotated", "w4a4_gemm_unrotated",
                "moe_route_sort", "w4a4_grouped_gemm_gather", "swiglu_quantize_h32", "moe_combine",
                "rotate_pack_weights_rot", "quantize_act_rot", "w4a4_gemm_rot",
                "w4a4_gemm_bf16", "w4a4_grouped_gemm_bf16", "w4a4_gemm_kernel_name",
                "w4a4_grouped_gemm_kernel_name")


class WeightsDesc(ctypes.Structure):
    _fields_ = [("magic", ctypes.c_uint32), ("version", ctypes.c_uint32),
                ("rotation", ctypes.c_uint32), ("layout", ctypes.c_uint32),
                ("n", ctypes.c_int64), ("k", ctypes.c_int64), ("num_experts", ctypes.c_int64),
                ("bytes", ctypes.c_uint64), ("scales_offset", ctypes.c_uint64)]


class BpgError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s (%s)" % (where, STATUS_NAMES.get(status, str(status)),
                                          _lib_handle().bpg_status_str(status).decode()))


_lib = None
_i64 = ctypes.c_int64
_vp = ctypes.c_void_p


def _lib_handle():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libbpg.so is not built (run __graft_entry__.build() or "
                           "python bit_prefill_gemm_amd/build.py); there is no fallback path")
    lib = ctypes.CDLL(LIB_PATH)
    lib.bpg_status_str.restype = ctypes.c_char_p
    lib.bpg_status_str.argtypes = [ctypes.c_int]
    lib.rotate_pack_weights_bytes.restype = ctypes.c_size_t
    lib.rotate_pack_weights_bytes.argtypes = [_i64, _i64, _i64]
    for name in ("rotate_pack_weights", "pack_weights_unrotated"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [_vp, ctypes.c_int, _i64, _i64, _i64, _vp, ctypes.c_size_t,
                       ctypes.POINTER(WeightsDesc)]
    for name in ("quantize_act_h32", "quantize_act_unrotated"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [_vp, ctypes.c_int, _i64, _i64, _i64, ctypes.c_int, _vp, _vp, _vp]
    for name in ("w4a4_gemm", "w4a4_gemm_unrotated", "w4a4_gemm_bf16"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [_vp, _vp, ctypes.c_int, _i64, ctypes.POINTER(WeightsDesc), _vp, _vp,
                       _i64, _vp]
    for name in ("w4a4_grouped_gemm", "w4a4_grouped_gemm_bf16"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [_vp, _vp, ctypes.c_int, _i64, _vp, ctypes.POINTER(WeightsDesc), _vp, _vp,
                       _i64, _vp]
    lib.rotate_pack_weights_rot.restype = ctypes.c_int
    lib.rotate_pack_weights_rot.argtypes = [_vp, ctypes.c_int, _i64, _i64, _i64, ctypes.c_int, _vp,
                                            ctypes.c_size_t, ctypes.POINTER(WeightsDesc)]
    lib.quantize_act_rot.restype = ctypes.c_int
    lib.quantize_act_rot.argtypes = [_vp, ctypes.c_int, _i64, _i64, _i64, ctypes.c_int, ctypes.c_int,
                                     _vp, _vp, _vp]
    lib.w4a4_gemm_rot.restype = ctypes.c_int
    lib.w4a4_gemm_rot.argtypes = [_vp, _vp, ctypes.c_int, ctypes.c_int, _i64,
                                  ctypes.POINTER(WeightsDesc), _vp, _vp, _i64, _vp]
    lib.moe_route_sort.restype = ctypes.c_int
    lib.moe_route_sort.argtypes = [_vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp]
    lib.w4a4_grouped_gemm_gather.restype = ctypes.c_int
    lib.w4a4_grouped_gemm_gather.argtypes = [_vp, _vp, ctypes.c_int, _i64, _vp, _i64, _vp,
                                             ctypes.POINTER(WeightsDesc), _vp, _vp, _i64, _vp]
    lib.swiglu_quantize_h32.restype = ctypes.c_int
    lib.swiglu_quantize_h32.argtypes = [_vp, _i64, _i64, _i64, ctypes.c_int, _vp, _vp, _vp]
    lib.moe_combine.restype = ctypes.c_int
    lib.moe_combine.argtypes = [_vp, _i64, _i64, _vp, _vp, _i64, _i64, _i64, _vp, _i64, _vp]
    lib.w4a4_gemm_blocksums.restype = ctypes.c_int
    lib.w4a4_gemm_blocksums.argtypes = [_vp, _vp, ctypes.c_int, _i64,
                                        ctypes.POINTER(WeightsDesc), _vp, _i64, _i64, _i64, _i64,
                                        _i64, _vp, _vp]
    lib.w4a4_gemm_kernel_name.restype = ctypes.c_char_p
    lib.w4a4_gemm_kernel_name.argtypes = [ctypes.c_int, _i64, ctypes.POINTER(WeightsDesc)]
    lib.w4a4_grouped_gemm_kernel_name.restype = ctypes.c_char_p
    lib.w4a4_grouped_gemm_kernel_name.argtypes = [ctypes.c_int, _i64, _i64,
                                                  ctypes.POINTER(WeightsDesc)]
    _lib = lib
    return lib


def lib():
    """The loaded ctypes library (raises if it is not built)."""
    return _lib_handle()


def _check(status: int, where: str):
    if status != BPG_OK:
        raise BpgError(status, where)


# ------------------------------------------------------------------ helpers

def _torch():
    import torch
    return torch


def _stream_handle(stream, device=None):
    """The hipStream_t of `stream`, or of the current stream of `device` (an
    int, e.g. a tensor's get_device(); the current device if None) as an int.
    The raw query of torch's current stream costs a tenth of building the
    stream object; torch builds without it fall back to that."""
    if stream is not None:
        return stream.cuda_stream
    torch = _torch()
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:
        return raw(device if device is not None and device >= 0 else torch.cuda.current_device())
    return torch.cuda.current_stream().cuda_stream


def _dptr(t):
    """A tensor's device address as an int (ctypes passes it as void *), 0 for None."""
    return t.data_ptr() if t is not None else 0


# Argument checks.  The C ABI sees only pointers and sizes, so a tensor of the
# wrong shape would become an out-of-bounds device access; every entry point
# below checks its tensors here first.  Shapes, dtypes and layouts are checked
# before devices, so that every shape error is reported the same way with or
# without a GPU.

def _fail(where, msg):
    raise ValueError("%s: %s" % (where, msg))


def _tensor(where, name, t, dtypes, shape, contiguous=True):
    """t must have one of `dtypes`, exactly `shape` and (if asked) be contiguous."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        _fail(where, "%s must be a torch tensor" % name)
    if t.dtype not in dtypes:
        _fail(where, "%s has dtype %s, expected %s" % (name, t.dtype,
                                                       " or ".join(str(d) for d in dtypes)))
    if t.shape != tuple(shape):
        _fail(where, "%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if contiguous and not t.is_contiguous():
        _fail(where, "%s must be contiguous" % name)


def _rows_out(where, name, t, dtype, rows, cols):
    """An output matrix [rows][cols] with unit column stride and any row stride >= cols."""
    _tensor(where, name, t, (dtype,), (rows, cols), contiguous=False)
    if cols > 0 and rows > 0 and (t.stride(1) != 1 or t.stride(0) < cols):
        _fail(where, "%s must have unit column stride and row stride >= %d" % (name, cols))


def _same_device(where, *tensors):
    """Every tensor on one cuda device (checked last: see above); returns its
    index.  get_device() is -1 for a host tensor."""
    idx = {t.get_device() for t in tensors if t is not None}
    if -1 in idx or len(idx) > 1:
        devs = {t.device for t in tensors if t is not None}
        if any(d.type != "cuda" for d in devs):
            _fail(where, "every tensor must be on a cuda device (got %s)"
                  % ", ".join(sorted(str(d) for d in devs)))
        _fail(where, "tensors are on different devices: %s"
              % ", ".join(sorted(str(d) for d in devs)))
    return idx.pop() if idx else None


def _check_bits(where, act_bits):
    if act_bits not in (4, 8):
        _fail(where, "act_bits must be 4 or 8, got %r" % (act_bits,))


def _code_cols(k, act_bits):
    return k // 2 if act_bits == 4 else k


def _check_codes(where, codes, scales, act_bits, rows, k):
    """Codes [rows][k/2] (4-bit) or [rows][k] (8-bit) bytes, scales [rows][k/32] fp32."""
    torch = _torch()
    _check_bits(where, act_bits)
    _tensor(where, "codes", codes, (torch.uint8, torch.int8), (rows, _code_cols(k, act_bits)))
    _tensor(where, "scales", scales, (torch.float32,), (rows, k // 32))


def _check_image(where, w):
    """The device image holds at least the bytes its stamp names."""
    torch = _torch()
    img = w.image
    if not isinstance(img, torch.Tensor):
        _fail(where, "the weight image is on the host: call .to(device) first")
    if img.dtype != torch.uint8 or img.dim() != 1 or not img.is_contiguous():
        _fail(where, "the weight image must be a contiguous 1-D uint8 tensor")
    if img.numel() < w.desc.bytes:
        _fail(where, "the weight image has %d bytes, its stamp names %d"
              % (img.numel(), w.desc.bytes))


class Weights:
    """A packed weight image on the device plus its stamp."""

    def __init__(self, desc: WeightsDesc, image):
        self.desc = desc
        self.image = image  # torch uint8 tensor on the device (or numpy on the host)

    @property
    def n(self):
        return self.desc.n

    @property
    def k(self):
        return self.desc.k

    @property
    def num_experts(self):
        return self.desc.num_experts

    def to(self, device):
        torch = _torch()
        img = self.image
        if isinstance(img, np.ndarray):
            img = torch.from_numpy(img)
        return Weights(self.desc, img.to(device))


# ------------------------------------------------------------------ entry points

def rotate_pack_weights_bytes(n: int, k: int, num_experts: int = 1) -> int:
    return int(_lib_handle().rotate_pack_weights_bytes(n, k, num_experts))


def _pack(name: str, src: np.ndarray, kind: int, n: int, k: int, num_experts: int) -> Weights:
    src = np.ascontiguousarray(src)
    nbytes = rotate_pack_weights_bytes(n, k, num_experts)
    if nbytes == 0:
        raise BpgError(2, name)
    img = np.empty(nbytes, dtype=np.uint8)
    desc = WeightsDesc()
    st = getattr(_lib_handle(), name)(src.ctypes.data_as(_vp), kind, n, k, num_experts,
                                      img.ctypes.data_as(_vp), img.nbytes, ctypes.byref(desc))
    _check(st, name)
    return Weights(desc, img)


def rotate_pack_weights(src: np.ndarray, kind: int, n: int, k: int,
                        num_experts: int = 1) -> Weights:
    """Host-side packing; returns Weights with a numpy image (call .to(device))."""
    return _pack("rotate_pack_weights", src, kind, n, k, num_experts)


def pack_weights_unrotated(src: np.ndarray, kind: int, n: int, k: int,
                           num_experts: int = 1) -> Weights:
    """Host-side packing of the unrotated route (stamp rotation 0)."""
    return _pack("pack_weights_unrotated", src, kind, n, k, num_experts)


def _quantize_args(name, x, act_bits, codes, scales, span=32):
    """Checks of the activation-quantize entry points; returns (dtype code, m, k, codes, scales)."""
    torch = _torch()
    if not isinstance(x, torch.Tensor) or x.dim() != 2 or (x.numel() > 0 and x.stride(1) != 1):
        _fail(name, "x must be a 2-D tensor with unit stride along K")
    dt = {torch.float32: X_F32, torch.bfloat16: X_BF16}.get(x.dtype)
    if dt is None:
        raise TypeError("%s: x must be float32 or bfloat16" % name)
    _check_bits(name, act_bits)
    m, k = x.shape
    if k % span != 0:
        _fail(name, "K = %d is not a multiple of %d" % (k, span))
    if codes is None:
        codes = torch.empty((m, _code_cols(k, act_bits)), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((m, k // 32), dtype=torch.float32, device=x.device)
    _check_codes(name, codes, scales, act_bits, m, k)
    _same_device(name, x, codes, scales)
    return dt, m, k, codes, scales


def _quantize(name: str, x, act_bits, codes, scales, stream):
    dt, m, k, codes, scales = _quantize_args(name, x, act_bits, codes, scales)
    st = getattr(_lib_handle(), name)(_dptr(x), dt, m, k, x.stride(0), act_bits, _dptr(codes),
                                      _dptr(scales), _stream_handle(stream, x.get_device()))
    _check(st, name)
    return codes, scales


def quantize_act_h32(x, act_bits: int = 4, codes=None, scales=None, stream=None):
    """x: 2-D cuda tensor (float32 or bfloat16, unit stride along K).  Returns (codes, scales)."""
    return _quantize("quantize_act_h32", x, act_bits, codes, scales, stream)


def quantize_act_unrotated(x, act_bits: int = 4, codes=None, scales=None, stream=None):
    """As quantize_act_h32 without the rotation."""
    return _quantize("quantize_act_unrotated", x, act_bits, codes, scales, stream)


def _gemm_args(name, codes, scales, act_bits, w, y, dtype):
    """Checks of the dense product entry points; returns (m, y)."""
    torch = _torch()
    if not isinstance(codes, torch.Tensor) or codes.dim() != 2:
        _fail(name, "codes must be a 2-D tensor")
    m = codes.shape[0]
    _check_codes(name, codes, scales, act_bits, m, w.k)
    _check_image(name, w)
    if y is None:
        y = torch.empty((m, w.n), dtype=dtype, device=codes.device)
    _rows_out(name, "y", y, dtype, m, w.n)
    _same_device(name, codes, scales, w.image, y)
    return m, y


def _gemm(name: str, codes, scales, act_bits, w, y, stream, dtype=None):
    m, y = _gemm_args(name, codes, scales, act_bits, w, y, dtype or _torch().float32)
    st = getattr(_lib_handle(), name)(_dptr(codes), _dptr(scales), act_bits, m,
                                      ctypes.byref(w.desc), _dptr(w.image), _dptr(y),
                                      y.stride(0), _stream_handle(stream, codes.get_device()))
    _check(st, name)
    return y


def w4a4_gemm(codes, scales, act_bits: int, w: Weights, y=None, stream=None):
    return _gemm("w4a4_gemm", codes, scales, act_bits, w, y, stream)


def w4a4_gemm_bf16(codes, scales, act_bits: int, w: Weights, y=None, stream=None):
    """As w4a4_gemm with the result rounded to bf16 at the store (y: torch.bfloat16)."""
    return _gemm("w4a4_gemm_bf16", codes, scales, act_bits, w, y, stream, _torch().bfloat16)


def w4a4_gemm_unrotated(codes, scales, act_bits: int, w: Weights, y=None, stream=None):
    """The product of the unrotated route (image from pack_weights_unrotated)."""
    return _gemm("w4a4_gemm_unrotated", codes, scales, act_bits, w, y, stream)


def _check_offsets(name, expert_offsets, w):
    torch = _torch()
    _tensor(name, "expert_offsets", expert_offsets, (torch.int32,), (w.num_experts + 1,))


def _grouped(name, codes, scales, act_bits, expert_offsets, w, y, stream, dtype):
    torch = _torch()
    if not isinstance(codes, torch.Tensor) or codes.dim() != 2:
        _fail(name, "codes must be a 2-D tensor")
    rows = codes.shape[0]
    _check_codes(name, codes, scales, act_bits, rows, w.k)
    _check_offsets(name, expert_offsets, w)
    _check_image(name, w)
    if y is None:
        y = torch.empty((rows, w.n), dtype=dtype, device=codes.device)
    _rows_out(name, "y", y, dtype, rows, w.n)
    _same_device(name, codes, scales, expert_offsets, w.image, y)
    st = getattr(_lib_handle(), name)(_dptr(codes), _dptr(scales), act_bits, rows,
                                      _dptr(expert_offsets), ctypes.byref(w.desc),
                                      _dptr(w.image), _dptr(y), y.stride(0),
                                      _stream_handle(stream, codes.get_device()))
    _check(st, name)
    return y


def w4a4_grouped_gemm(codes, scales, act_bits: int, expert_offsets, w: Weights, y=None,
                      stream=None):
    return _grouped("w4a4_grouped_gemm", codes, scales, act_bits, expert_offsets, w, y, stream,
                    _torch().float32)


def w4a4_grouped_gemm_bf16(codes, scales, act_bits: int, expert_offsets, w: Weights, y=None,
                           stream=None):
    """As w4a4_grouped_gemm with the result rounded to bf16 at the store."""
    return _grouped("w4a4_grouped_gemm_bf16", codes, scales, act_bits, expert_offsets, w, y,
                    stream, _torch().bfloat16)


def w4a4_gemm_blocksums(codes, scales, act_bits: int, w: Weights, m0: int, m1: int, n0: int,
                        n1: int, expert: int = 0, sums=None, stream=None):
    """Exact int32 block sums of rows [m0, m1) x columns [n0, n1) of expert `expert`
    (always the tiled kernel's 32 x 32 main loop; see include/bpg.h)."""
    torch = _torch()
    where = "w4a4_gemm_blocksums"
    if not isinstance(codes, torch.Tensor) or codes.dim() != 2:
        _fail(where, "codes must be a 2-D tensor")
    m = codes.shape[0]
    _check_bits(where, act_bits)
    _tensor(where, "codes", codes, (torch.uint8, torch.int8), (m, _code_cols(w.k, act_bits)))
    if not (0 <= m0 <= m1 <= m and 0 <= n0 <= n1 <= w.n and 0 <= expert < w.num_experts):
        _fail(where, "rectangle [%d,%d) x [%d,%d) of expert %d is outside %d rows, %d columns, "
              "%d experts" % (m0, m1, n0, n1, expert, m, w.n, w.num_experts))
    _check_image(where, w)
    if sums is None:
        sums = torch.empty((m1 - m0, n1 - n0, w.k // 32), dtype=torch.int32, device=codes.device)
    _tensor(where, "sums", sums, (torch.int32,), (m1 - m0, n1 - n0, w.k // 32))
    _same_device(where, codes, w.image, sums, scales if isinstance(scales, torch.Tensor) else None)
    st = _lib_handle().w4a4_gemm_blocksums(_dptr(codes), _dptr(scales), act_bits, m,
                                           ctypes.byref(w.desc), _dptr(w.image), expert, m0, m1,
                                           n0, n1, _dptr(sums),
                                                         _stream_handle(stream, codes.get_device()))
    _check(st, "w4a4_gemm_blocksums")
    return sums


def w4a4_gemm_kernel_name(act_bits: int, m: int, w: Weights) -> str:
    """The kernel w4a4_gemm runs for m rows of act_bits codes against w (host only)."""
    r = _lib_handle().w4a4_gemm_kernel_name(act_bits, m, ctypes.byref(w.desc))
    if r is None:
        raise ValueError("w4a4_gemm_kernel_name: invalid act_bits, m or stamp")
    return r.decode()


def w4a4_grouped_gemm_kernel_name(act_bits: int, total_rows: int, w: Weights,
                                  src_rows: int = 0) -> str:
    """The kernel w4a4_grouped_gemm (src_rows = 0) or w4a4_grouped_gemm_gather runs."""
    r = _lib_handle().w4a4_grouped_gemm_kernel_name(act_bits, total_rows, src_rows,
                                                    ctypes.byref(w.desc))
    if r is None:
        raise ValueError("w4a4_grouped_gemm_kernel_name: invalid arguments or stamp")
    return r.decode()


# ------------------------------------------------------------------ expert layer glue

def moe_route_sort(expert_of, tokens: int, topk: int, experts: int, stream=None):
    """expert_of: cuda int32 [tokens*topk].  Returns (offsets [E+1], row_token, slot_of)."""
    torch = _torch()
    n = tokens * topk
    _tensor("moe_route_sort", "expert_of", expert_of, (torch.int32,), (n,))
    _same_device("moe_route_sort", expert_of)
    dev = expert_of.device
    offsets = torch.empty(experts + 1, dtype=torch.int32, device=dev)
    row_token = torch.empty(n, dtype=torch.int32, device=dev)
    slot_of = torch.empty(n, dtype=torch.int32, device=dev)
    st = _lib_handle().moe_route_sort(_dptr(expert_of), tokens, topk, experts, _dptr(offsets),
                                      _dptr(row_token), _dptr(slot_of),
                                      _stream_handle(stream, expert_of.get_device()))
    _check(st, "moe_route_sort")
    return offsets, row_token, slot_of


def w4a4_grouped_gemm_gather(codes, scales, act_bits: int, row_ids, expert_offsets, w: Weights,
                             y=None, stream=None):
    torch = _torch()
    where = "w4a4_grouped_gemm_gather"
    if not isinstance(codes, torch.Tensor) or codes.dim() != 2:
        _fail(where, "codes must be a 2-D tensor")
    if not isinstance(row_ids, torch.Tensor) or row_ids.dim() != 1:
        _fail(where, "row_ids must be a 1-D tensor")
    src_rows = codes.shape[0]
    rows = row_ids.shape[0]
    _check_codes(where, codes, scales, act_bits, src_rows, w.k)
    _tensor(where, "row_ids", row_ids, (torch.int32,), (rows,))
    _check_offsets(where, expert_offsets, w)
    _check_image(where, w)
    if y is None:
        y = torch.empty((rows, w.n), dtype=torch.float32, device=codes.device)
    _rows_out(where, "y", y, torch.float32, rows, w.n)
    _same_device(where, codes, scales, row_ids, expert_offsets, w.image, y)
    st = _lib_handle().w4a4_grouped_gemm_gather(_dptr(codes), _dptr(scales), act_bits, src_rows,
                                                _dptr(row_ids), rows, _dptr(expert_offsets),
                                                ctypes.byref(w.desc), _dptr(w.image), _dptr(y),
                                                y.stride(0),
                                                         _stream_handle(stream, codes.get_device()))
    _check(st, "w4a4_grouped_gemm_gather")
    return y


def swiglu_quantize_h32(gu, inter: int, act_bits: int = 4, codes=None, scales=None, stream=None):
    """gu: cuda fp32 [rows, >= 2*inter] (gate then up).  Returns (codes, scales)."""
    torch = _torch()
    where = "swiglu_quantize_h32"
    if (not isinstance(gu, torch.Tensor) or gu.dim() != 2 or gu.dtype != torch.float32 or
            (gu.numel() > 0 and gu.stride(1) != 1)):
        _fail(where, "gu must be a 2-D float32 tensor with unit stride along columns")
    _check_bits(where, act_bits)
    rows = gu.shape[0]
    if inter <= 0 or inter % 32 != 0 or gu.shape[1] < 2 * inter:
        _fail(where, "inter = %d must be a positive multiple of 32 with 2*inter <= %d columns"
              % (inter, gu.shape[1]))
    if codes is None:
        codes = torch.empty((rows, _code_cols(inter, act_bits)), dtype=torch.uint8,
                            device=gu.device)
    if scales is None:
        scales = torch.empty((rows, inter // 32), dtype=torch.float32, device=gu.device)
    _check_codes(where, codes, scales, act_bits, rows, inter)
    _same_device(where, gu, codes, scales)
    st = _lib_handle().swiglu_quantize_h32(_dptr(gu), rows, inter, gu.stride(0), act_bits,
                                           _dptr(codes), _dptr(scales),
                                           _stream_handle(stream, gu.get_device()))
    _check(st, "swiglu_quantize_h32")
    return codes, scales


def moe_combine(dn, slot_of, weights, tokens: int, topk: int, y=None, stream=None):
    """dn: cuda fp32 [rows, hidden] (sorted rows).  Returns y [tokens, hidden]."""
    torch = _torch()
    where = "moe_combine"
    if (not isinstance(dn, torch.Tensor) or dn.dim() != 2 or dn.dtype != torch.float32 or
            (dn.numel() > 0 and dn.stride(1) != 1)):
        _fail(where, "dn must be a 2-D float32 tensor with unit stride along columns")
    rows, hidden = dn.shape
    _tensor(where, "slot_of", slot_of, (torch.int32,), (tokens * topk,))
    _tensor(where, "weights", weights, (torch.float32,), (tokens * topk,))
    if y is None:
        y = torch.empty((tokens, hidden), dtype=torch.float32, device=dn.device)
    _rows_out(where, "y", y, torch.float32, tokens, hidden)
    _same_device(where, dn, slot_of, weights, y)
    st = _lib_handle().moe_combine(_dptr(dn), dn.stride(0), rows, _dptr(slot_of), _dptr(weights),
                                   tokens, topk, hidden, _dptr(y), y.stride(0),
                                   _stream_handle(stream, dn.get_device()))
    _check(st, "moe_combine")
    return y


# ------------------------------------------------------------------ longer rotations

def rotate_pack_weights_rot(src: np.ndarray, kind: int, n: int, k: int, rotation: int,
                            num_experts: int = 1) -> Weights:
    src = np.ascontiguousarray(src)
    nbytes = rotate_pack_weights_bytes(n, k, num_experts)
    if nbytes == 0:
        raise BpgError(2, "rotate_pack_weights_rot")
    img = np.empty(nbytes, dtype=np.uint8)
    desc = WeightsDesc()
    st = _lib_handle().rotate_pack_weights_rot(src.ctypes.data_as(_vp), kind, n, k, num_experts,
                                               rotation, img.ctypes.data_as(_vp), img.nbytes,
                                               ctypes.byref(desc))
    _check(st, "rotate_pack_weights_rot")
    return Weights(desc, img)


def quantize_act_rot(x, rotation: int, act_bits: int = 4, codes=None, scales=None, stream=None):
    if rotation not in (32, 64, 128):
        _fail("quantize_act_rot", "rotation must be 32, 64 or 128, got %r" % (rotation,))
    dt, m, k, codes, scales = _quantize_args("quantize_act_rot", x, act_bits, codes, scales,
                                             span=rotation)
    st = _lib_handle().quantize_act_rot(_dptr(x), dt, m, k, x.stride(0), act_bits, rotation,
                                        _dptr(codes), _dptr(scales),
                                                            _stream_handle(stream, x.get_device()))
    _check(st, "quantize_act_rot")
    return codes, scales


def w4a4_gemm_rot(codes, scales, act_bits: int, rotation: int, w: Weights, y=None, stream=None):
    m, y = _gemm_args("w4a4_gemm_rot", codes, scales, act_bits, w, y, _torch().float32)
    st = _lib_handle().w4a4_gemm_rot(_dptr(codes), _dptr(scales), act_bits, rotation, m,
                                     ctypes.byref(w.desc), _dptr(w.image), _dptr(y), y.stride(0),
                                     _stream_handle(stream, codes.get_device()))
    _check(st, "w4a4_gemm_rot")
    return y
