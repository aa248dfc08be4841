"""Seeded synthetic inputs for the Hadamard-rotated W4A4 prompt GEMM.

This module draws inputs only: random activations, random Q4_0 weight files
and random MoE routings.  It holds none of the method's arithmetic (no
rotation, no quantizer, no product), so that the CPU oracle and the HIP path
can both be fed from it without sharing code.

Workloads (shapes follow the pages' own measurements: prompt processing of a
dense 27B model at 512 tokens, "509 tokens a second of prompt: the Hadamard
route ships", section "The numbers"; the MoE experts of a 30B-A3B model,
"Where the engine is going: HRX and the NPU", section "4-bit activations reach
the MoE experts"; 1,024-token micro-batches, same section).  The pages measure
on a model and wikitext-2, which are not available here: these seeded
synthetic tensors of the same shapes stand in for them.

Recipe (one ``numpy.random.default_rng(0)`` per workload, draws in this order:
activations, outlier channels, then for each weight tensor its nibble bytes
and its fp16 scales, then the routing):

* activations: fp32 N(0, 1) (or Student-t with 3 degrees of freedom); a set of
  ``round(p * K)`` distinct outlier channels drawn without replacement is
  multiplied by a fixed factor in every row; bf16 inputs are the fp32 values
  rounded to nearest-even after the outlier scaling;
* weights: canonical Q4_0 blocks (fp16 scale little-endian, then 16 bytes of
  nibbles); the 16 bytes are uniform over 0..255, so every 4-bit code is
  uniform over 0..15; scales are uniform in a range, rounded to fp16.  The
  drawn codes are taken to be already rotated weights;
* MoE routing: each token picks 8 distinct experts uniformly; the (token,
  expert) rows are sorted stably by expert, then token.
"""
from __future__ import annotations

import numpy as np

QK = 32


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even (finite inputs)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def draw_activations(rng, m, k, dist="normal", outlier_frac=0.0, outlier_mult=1.0):
    """Return (x fp32 [m, k], outlier channel indices)."""
    if dist == "normal":
        x = rng.standard_normal((m, k), dtype=np.float32)
    elif dist == "t3":
        x = rng.standard_t(3, size=(m, k)).astype(np.float32)
    else:
        raise ValueError(dist)
    nch = int(round(outlier_frac * k))
    ch = np.sort(rng.choice(k, nch, replace=False)) if nch else np.zeros(0, dtype=np.int64)
    if nch:
        x[:, ch] *= np.float32(outlier_mult)
    return x, ch


def draw_q4_0(rng, rows_shape, k, d_lo, d_hi) -> np.ndarray:
    """Canonical Q4_0 blocks uint8 [*rows_shape, k/32, 18]."""
    shape = tuple(rows_shape) + (k // QK,)
    qs = rng.integers(0, 256, size=shape + (16,), dtype=np.uint8)
    d = rng.uniform(d_lo, d_hi, size=shape).astype("<f2")
    blocks = np.empty(shape + (18,), dtype=np.uint8)
    blocks[..., 0:2] = d.view(np.uint8).reshape(shape + (2,))
    blocks[..., 2:18] = qs
    return blocks


def draw_weights_f32(rng, rows, k, std) -> np.ndarray:
    """Unquantized float weights [rows, k], normal with the given std (the
    source of both offline packers in the route comparison)."""
    return (rng.standard_normal((rows, k)) * std).astype(np.float32)


def draw_routing(rng, tokens, experts, topk):
    """Return (token_of_row [tokens*topk], expert_of_row, offsets [experts+1] int32)."""
    choice = np.argsort(rng.random((tokens, experts)), axis=1)[:, :topk]
    tok = np.repeat(np.arange(tokens), topk)
    exp = choice.reshape(-1)
    order = np.lexsort((tok, exp))  # primary key expert, then token
    tok, exp = tok[order], exp[order]
    counts = np.bincount(exp, minlength=experts)
    offsets = np.zeros(experts + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    return tok.astype(np.int64), exp.astype(np.int64), offsets


def draw_routes(rng, tokens, experts, topk):
    """Routed choices in entry order (entry t*topk + j): expert ids int32
    [tokens*topk], topk distinct experts per token, and routing weights fp32
    (a softmax over topk standard-normal logits per token)."""
    choice = np.argsort(rng.random((tokens, experts)), axis=1)[:, :topk]
    logits = rng.standard_normal((tokens, topk))
    w = np.exp(logits - logits.max(axis=1, keepdims=True))
    w /= w.sum(axis=1, keepdims=True)
    return choice.reshape(-1).astype(np.int32), w.reshape(-1).astype(np.float32)


# name -> recipe.  'gemms' lists (input name, weight name) pairs in step order.
CONFIGS = {
    "tiny": dict(desc="Tiny W4A4: M=16, K=256, N=128, fp32 activations",
                 m=16, k=256, n=128, dtype="f32", dist="normal", outlier_frac=0.02,
                 outlier_mult=20.0, d_range=(0.005, 0.05)),
    "attn512": dict(desc="Dense attention projection pp512: M=512, K=5120, N=5120",
                    m=512, k=5120, n=5120, dtype="bf16", dist="normal", outlier_frac=0.005,
                    outlier_mult=30.0, d_range=(0.002, 0.02)),
    "ffn512": dict(desc="Dense FFN pair pp512: gate/up 512x5120x17408, down 512x17408x5120",
                   m=512, k=5120, n=17408, dtype="bf16", dist="t3", d_range=(0.002, 0.02)),
    "moe512": dict(desc="MoE grouped GEMM: 512 tokens, hidden 2048, 128 experts, top-8, "
                        "expert intermediate 768",
                   tokens=512, hidden=2048, experts=128, topk=8, inter=768, dtype="bf16",
                   d_range=(0.002, 0.02)),
    "long1024": dict(desc="Long-prompt micro-batch: M=1024, K=5120, N=17408",
                     m=1024, k=5120, n=17408, dtype="bf16", dist="normal", outlier_frac=0.01,
                     outlier_mult=50.0, d_range=(0.002, 0.02)),
    # weight-streaming cases: 16 tokens against the large projections
    "m16_gate": dict(desc="Weight streaming: M=16, K=5120, N=17408", m=16, k=5120, n=17408,
                     dtype="bf16", dist="normal", outlier_frac=0.02, outlier_mult=20.0,
                     d_range=(0.002, 0.02)),
    "m16_down": dict(desc="Weight streaming: M=16, K=17408, N=5120", m=16, k=17408, n=5120,
                     dtype="bf16", dist="normal", outlier_frac=0.02, outlier_mult=20.0,
                     d_range=(0.002, 0.02)),
    "m16_attn": dict(desc="Weight streaming: M=16, K=5120, N=5120", m=16, k=5120, n=5120,
                     dtype="bf16", dist="normal", outlier_frac=0.02, outlier_mult=20.0,
                     d_range=(0.002, 0.02)),
}


def _act_out(x, dtype):
    return x if dtype == "f32" else bf16_bits(x)


def make(name: str, seed: int = 0) -> dict:
    """Draw one workload.  Activations are fp32 arrays or bf16 bit arrays (uint16)."""
    cfg = CONFIGS[name]
    rng = np.random.default_rng(seed)
    out = dict(name=name, cfg=cfg)
    lo, hi = cfg["d_range"]
    if name == "ffn512":
        m, k, n = cfg["m"], cfg["k"], cfg["n"]
        x1, _ = draw_activations(rng, m, k, "t3")
        x2, _ = draw_activations(rng, m, n, "t3")
        out["x1"] = _act_out(x1, cfg["dtype"])
        out["x2"] = _act_out(x2, cfg["dtype"])
        out["w_gate"] = draw_q4_0(rng, (n,), k, lo, hi)
        out["w_up"] = draw_q4_0(rng, (n,), k, lo, hi)
        out["w_down"] = draw_q4_0(rng, (k,), n, lo, hi)
        return out
    if name == "moe512":
        T, H, E, K8, I = cfg["tokens"], cfg["hidden"], cfg["experts"], cfg["topk"], cfg["inter"]
        x, _ = draw_activations(rng, T, H, "normal")
        xd, _ = draw_activations(rng, T * K8, I, "normal")
        out["w_gu"] = draw_q4_0(rng, (E, 2 * I), H, lo, hi)
        out["w_dn"] = draw_q4_0(rng, (E, H), I, lo, hi)
        tok, exp, off = draw_routing(rng, T, E, K8)
        out["x_tokens"] = _act_out(x, cfg["dtype"])
        out["x_gu"] = out["x_tokens"][tok]  # expert-sorted rows
        out["x_dn"] = _act_out(xd, cfg["dtype"])
        out["token_of_row"], out["expert_of_row"], out["offsets"] = tok, exp, off
        return out
    m, k, n = cfg["m"], cfg["k"], cfg["n"]
    x, ch = draw_activations(rng, m, k, cfg["dist"], cfg.get("outlier_frac", 0.0),
                             cfg.get("outlier_mult", 1.0))
    out["x"] = _act_out(x, cfg["dtype"])
    out["outlier_channels"] = ch
    out["w"] = draw_q4_0(rng, (n,), k, lo, hi)
    return out


def small_dense(m, k, n, seed=0, dtype="f32", outlier_frac=0.02, outlier_mult=20.0,
                d_range=(0.005, 0.05), dist="normal"):
    """A small dense case with the tiny recipe at arbitrary sizes (tests)."""
    rng = np.random.default_rng(seed)
    x, ch = draw_activations(rng, m, k, dist, outlier_frac, outlier_mult)
    w = draw_q4_0(rng, (n,), k, *d_range)
    return dict(x=_act_out(x, dtype), w=w, outlier_channels=ch)
