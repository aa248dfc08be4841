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
