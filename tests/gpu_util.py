"""Helpers shared by the GPU tests: device inputs, oracle references, error metric."""
import numpy as np

import oracle
from bit_prefill_gemm_amd import binding as bb


def torch_mod():
    import torch
    return torch


def act_to_device(x: np.ndarray):
    """fp32 array or bf16 bit array (uint16) -> cuda tensor of float32 / bfloat16."""
    torch = torch_mod()
    if x.dtype == np.float32:
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()
    assert x.dtype == np.uint16
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)


def weights_to_device(blocks: np.ndarray, n: int, k: int, e: int = 1):
    W = bb.rotate_pack_weights(blocks, bb.SRC_Q4_0_ROTATED, n, k, e)
    return W.to("cuda")


def oracle_codes(q: np.ndarray, bits: int) -> np.ndarray:
    """The byte layout the GPU writes, from the oracle's code values."""
    return oracle.pack_int4(q) if bits == 4 else q.view(np.uint8)


def row_rel_err(y: np.ndarray, ref: np.ndarray) -> float:
    """max over rows of ||y - ref||_2 / ||ref||_2."""
    y = y.astype(np.float64)
    num = np.linalg.norm(y - ref, axis=1)
    den = np.linalg.norm(ref, axis=1)
    den = np.where(den == 0, 1.0, den)
    return float((num / den).max())


def sample_rows(m: int, count: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    if m <= count:
        return np.arange(m)
    rows = rng.choice(m, count - 2, replace=False)
    return np.unique(np.concatenate([rows, [0, m - 1]]))


def rects(m: int, n: int, size: int, count: int, seed: int):
    """Seeded row/column rectangles of at most size x size (always includes the last tile)."""
    rng = np.random.default_rng(seed)
    out = [(max(0, m - size), m, max(0, n - size), n)]
    for _ in range(count - 1):
        m0 = int(rng.integers(0, max(1, m - size + 1)))
        n0 = int(rng.integers(0, max(1, n - size + 1)))
        out.append((m0, min(m, m0 + size), n0, min(n, n0 + size)))
    return out


def quantize_and_check(x, bits):
    """Quantize on the GPU, compare codes and scales bit-exactly with the
    oracle; return (device codes, device scales, oracle codes, oracle scales)."""
    torch = torch_mod()
    xd = act_to_device(x)
    codes, scales = bb.quantize_act_h32(xd, bits)
    torch.cuda.synchronize()
    q, d, _ = oracle.quantize(x, bits)
    got_codes = codes.cpu().numpy()
    got_scales = scales.cpu().numpy()
    exp_codes = oracle_codes(q, bits)
    bad = np.argwhere(got_codes != exp_codes)
    assert bad.size == 0, "codes differ at %s (of %d)" % (bad[:5].tolist(), len(bad))
    assert np.array_equal(got_scales.view(np.uint32), d.view(np.uint32)), "scales differ"
    return codes, scales, q, d


# fp32 error bound of a product: every output is a sum of B terms
# da*dw*S (exact block sums, exact products for 4-bit codes and one rounding
# of S*dw for 8-bit ones) added in some order with one rounding per addition,
# so |y - exact| <= (B + 8) * 2^-24 * sum_b |da*dw*S| for any order the
# kernels use (per-wave chains, then the wave partials).

def fp32_bound(a: np.ndarray, k: int) -> np.ndarray:
    return (k // 32 + 8) * 2.0 ** -24 * a


def assert_within_bound(y: np.ndarray, ref: np.ndarray, a: np.ndarray, k: int, what=""):
    """Element-wise |y - ref| <= fp32_bound(a) (the oracle's own fp64 error is
    below 2^-40 of that)."""
    err = np.abs(y.astype(np.float64) - ref)
    lim = fp32_bound(a, k) * (1 + 2.0 ** -20)
    bad = np.argwhere(err > lim)
    assert bad.size == 0, "%s: %d elements outside the fp32 bound, first %s: |d| %g > %g" % (
        what, len(bad), bad[0].tolist(), err[tuple(bad[0])], lim[tuple(bad[0])])


def pow2_blocks(blocks: np.ndarray, rng, lo: int, hi: int) -> np.ndarray:
    """A copy of canonical Q4_0 blocks [..., 18] whose fp16 scales are replaced
    by powers of two 2^e, e uniform in [lo, hi] (codes unchanged)."""
    out = np.array(blocks, dtype=np.uint8, copy=True)
    e = rng.integers(lo, hi + 1, size=out.shape[:-1])
    h = np.ldexp(np.ones(e.shape), e).astype(np.float16)
    out[..., 0:2] = h.view(np.uint8).reshape(*e.shape, 2)
    return out


def pow2_scales(rows: int, nblk: int, rng, lo: int, hi: int) -> np.ndarray:
    """Activation scales [rows][nblk] fp32, powers of two 2^e, e uniform in [lo, hi]."""
    e = rng.integers(lo, hi + 1, size=(rows, nblk))
    return np.ldexp(np.ones((rows, nblk)), e).astype(np.float32)


def check_grouped_rows(y_rows, q, d, off, wq, dwq, rows, k, what="", tol=1e-3):
    """Rows `rows` of a grouped product against the oracle: row-L2 error within
    tol and every element within the fp32 bound."""
    n = wq.shape[1]
    rr, cc = np.meshgrid(rows, np.arange(n), indexing="ij")
    ref = oracle.grouped_points(q, d, off, wq, dwq, rr.ravel(), cc.ravel()).reshape(len(rows), n)
    a = oracle.grouped_abs_points(q, d, off, wq, dwq, rr.ravel(), cc.ravel()).reshape(
        len(rows), n)
    err = row_rel_err(y_rows, ref)
    assert err <= tol, (what, err)
    assert_within_bound(y_rows, ref, a, k, what)
    return err
