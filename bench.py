#!/usr/bin/env python3
"""Benchmark of the Hadamard-rotated W4A4 prompt GEMM on one MI355X.

A step is one pass of the route over one batch: quantize_act_h32 (FWHT-32 +
4-bit quantization of the activations) then w4a4_gemm, by default on the
dense attention projection at 512 prompt tokens (M=512, K=5120, N=5120, bf16
activations, rotated Q4_0 weights).  The weight image is packed once, outside
the timed region (it is the offline step).  Inputs are resident in HBM before
the timed region; each step uses a different copy of the weights and
activations, cycling through enough copies (>= 512 MB) that the 256 MB
last-level cache cannot hold them.

Other workloads (--workload): the long-prompt and FFN-sized GEMM, three
weight-streaming cases with 16 tokens, and the two grouped expert GEMMs of the
MoE workload (512 tokens routed top-8 over 128 experts; `value` counts the 512
tokens), and the whole expert layer (moe512_layer: expert sort, token
quantization, gathered gate/up GEMM, SwiGLU-rotate-quantize, down GEMM,
weighted combine; `kernel_us` gives each kernel's own duration).

Prints ONE JSON line.  `value` is prompt tokens per second of the step: the
K timed steps are one captured graph, uploaded to the device beforehand and
replayed between two synchronisations right after an untimed replay of the W
warm-up steps (an idle GPU's clock needs tens of milliseconds of load to come
up; the default W covers that), and `eager_step_us` gives the same steps
issued one binding call at a time.  The
`roofline` object covers the GEMM kernel (the dominant kernel).  Its average
duration is measured with HIP events recorded on the launch stream around a
graph replay of 40 back-to-back GEMM launches over the same cold copies,
right after the timed steps (an event pair around each single launch would
add its two queue packets to every launch).  `gemm_in_step_us` is the same
kernel inside whole steps: a graph replay of quantize + GEMM steps less the
quantizer's own replay (the product right after the quantizer that wrote its
codes runs a few percent longer than back to back).  The bound is whichever algorithmic floor
of the contraction is larger: its 2*M*N*K integer ops at the dense int8
matrix peak ("mfma"), or its HBM bytes at the HBM peak ("hbm": a few rows, and
the grouped expert GEMMs, whose weight stream is larger).  `epilogue_valu`
gives the same launch against the other floor this method has on gfx950: the
fp32 epilogue (two FMAs per output element and 32-block) at the fp32 vector
peak.
`traffic` comes from the committed rocprofv3 counter summary for this kernel
and workload, and is null if that kernel's sources (its own file and the
shared routing and operand code) or the compile flags changed since it was
taken.
`configs` (default workload only) measures every other workload in the same
run, with fewer steps and no CPU baseline: GEMM time, kernel, roofline
fraction and tokens/s of each.
`cpu_baseline` times the CPU oracle on the same workload (test
infrastructure, not the product path).

`--copy-calibration BYTES` instead runs a plain device copy of that size
(for scaling the FETCH_SIZE / WRITE_SIZE counters) and prints nothing else.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X published peaks
PEAK_INT8_OPS = 5.0e15                    # dense int8 matrix ops/s
PEAK_HBM = 8.0e12                         # bytes/s
# fp32 vector peak: 256 CUs x 4 SIMDs x 32 lanes x 2 flops (one FMA) x 2.4 GHz.
# gfx950 issues a non-packed wave64 FMA in two cycles, so this peak applies to
# the plain fp32 FMAs of the epilogue (a pure FMA loop measures ~125 TFLOP/s).
PEAK_FP32_FLOPS = 157.3e12

WORKLOADS = {
    "attn512": dict(m=512, k=5120, n=5120),
    "long1024": dict(m=1024, k=5120, n=17408),
    # the dense FFN pair (Student-t activations): gate (up is the same shape)
    # and down projections
    "ffn512_gate": dict(m=512, k=5120, n=17408, src="ffn512", x="x1", w="w_gate"),
    "ffn512_down": dict(m=512, k=17408, n=5120, src="ffn512", x="x2", w="w_down"),
    "m16_gate": dict(m=16, k=5120, n=17408),
    "m16_down": dict(m=16, k=17408, n=5120),
    "m16_attn": dict(m=16, k=5120, n=5120),
    # grouped expert GEMMs of the MoE workload (512 tokens, top-8 of 128
    # experts: 4096 expert-sorted rows)
    "moe512_gu": dict(m=4096, k=2048, n=1536, experts=128, tokens=512, src="moe512", x="x_gu",
                      w="w_gu"),
    "moe512_dn": dict(m=4096, k=768, n=2048, experts=128, tokens=512, src="moe512", x="x_dn",
                      w="w_dn"),
    # the whole expert layer: expert sort, token quantization, gathered gate/up
    # GEMM, SwiGLU-rotate-quantize, down GEMM, weighted combine
    "moe512_layer": dict(m=512, k=2048, n=2048, experts=128, tokens=512, layer=True),
}
# kernel sources of the GEMM paths (the tiled, wide, strip and grouped kernels,
# the weight-stream kernel used for a few rows, and the headers they share)
_CSRC = os.path.join(ROOT, "bit_prefill_gemm_amd", "csrc")
GEMM_SRCS = [os.path.join(_CSRC, f)
             for f in ("gemm.hip", "skinny.hip", "wide.hip", "strip.hip", "grouped.hip",
                       "operands.h", "internal.h")]
# what every GEMM launch depends on (routing, the tiled kernel, shared operand
# code) and, by the kernel name the routing query returns, its own source
SHARED_SRCS = [os.path.join(_CSRC, f) for f in ("gemm.hip", "operands.h", "internal.h")]
KERNEL_SRC = {"weight-stream": "skinny.hip", "wide": "wide.hip", "strip": "strip.hip",
              "expert-slot": "grouped.hip", "grouped": "grouped.hip", "tiled": "gemm.hip"}
# the workloads measured beside the default one (name, activation bits)
CONFIG_RUNS = [("attn512", 8), ("ffn512_gate", 4), ("ffn512_down", 4), ("ffn512_gate", 8),
               ("ffn512_down", 8), ("long1024", 4), ("long1024", 8), ("moe512_gu", 4),
               ("moe512_dn", 4), ("moe512_layer", 4), ("m16_gate", 4), ("m16_down", 4),
               ("m16_attn", 4)]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_traffic.json")
GRAPH_LAUNCHES = 40   # launches per captured graph when a kernel is timed alone
GRAPH_REPLAYS = 5


def upload_graph(torch, graph, stream):
    """Upload a captured graph's executable to the device before it first
    runs (hipGraphUpload), so that its first replay does not pay for it.
    Skipped where the runtime or this PyTorch does not offer it."""
    exec_handle = getattr(graph, "raw_cuda_graph_exec", None)
    if exec_handle is None:
        return
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        fn = hip.hipGraphUpload
    except (OSError, AttributeError):
        return
    fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    fn.restype = ctypes.c_int
    rc = fn(ctypes.c_void_p(exec_handle()), ctypes.c_void_p(stream.cuda_stream))
    if rc != 0:
        raise RuntimeError("hipGraphUpload failed (%d)" % rc)


def timed_steps(torch, stream, step, steps, warmup, copies):
    """(ms per step, ms per eager step).  The warm-up steps and the timed
    steps are captured as two graphs (step j = j % copies, the timed ones
    following the warm-up ones) and uploaded to the device; the warm-up graph
    is replayed untimed, then the timed region replays the `steps` steps
    between two synchronisations of the device.  Replaying a captured sequence
    is how a fixed prompt pipeline runs on the device (no host work between
    the kernels).  The clock of an idle GPU takes tens of milliseconds of
    load to come up, which is what the warm-up steps are for.  The same steps
    issued one binding call at a time are timed afterwards, for comparison
    (larger shapes lose a few percent that way, the 16-row ones are bound by
    the binding's host time)."""
    graphs = []
    for n, first in ((warmup, 0), (steps, warmup)):
        g = None
        if n > 0:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for i in range(n):
                    step((first + i) % copies)
        graphs.append(g)
    torch.cuda.synchronize()
    for g in graphs:
        if g is not None:
            upload_graph(torch, g, stream)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        if graphs[0] is not None:
            graphs[0].replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        graphs[1].replay()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    del graphs
    graph_ms = (t1 - t0) * 1e3 / steps
    with torch.cuda.stream(stream):
        for i in range(warmup):
            step(i % copies)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            step((warmup + i) % copies)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    return graph_ms, (t1 - t0) * 1e3 / steps


def graph_time_us(torch, stream, launch, n=GRAPH_LAUNCHES, replays=GRAPH_REPLAYS):
    """The median of graph_time_spread_us."""
    return graph_time_spread_us(torch, stream, launch, n, replays)[0]


def graph_time_spread_us(torch, stream, launch, n=GRAPH_LAUNCHES, replays=GRAPH_REPLAYS):
    """Per-launch duration of launch(0), ..., launch(n-1) on `stream`, replayed
    from one captured graph: the kernels run back to back with no host work and
    no event packets between them, so the time between the two events around a
    replay, divided by n, is one kernel's duration plus one dispatch gap.  (An
    event pair around each launch instead adds the cost of its two packets to
    every launch, several microseconds, which dominates a short kernel.)  The
    median over `replays` replays after one untimed replay, with the fastest and
    the slowest of them: (median, min, max)."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(n):
            launch(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ts = []
    with torch.cuda.stream(stream):
        g.replay()
        for _ in range(replays):
            e0.record(stream)
            g.replay()
            e1.record(stream)
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3 / n)
    torch.cuda.synchronize()
    del g
    return float(np.median(ts)), float(min(ts)), float(max(ts))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=400)
    ap.add_argument("--workload", default="attn512", choices=sorted(WORKLOADS))
    ap.add_argument("--bits", type=int, default=4, choices=(4, 8))
    ap.add_argument("--out", default="f32", choices=("f32", "bf16"),
                    help="output type of the GEMM (bf16: the rounded-output entry points)")
    ap.add_argument("--cold-bytes", type=float, default=512e6,
                    help="total bytes of distinct input copies cycled through")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workloads (measured only with the default one)")
    ap.add_argument("--config-steps", type=int, default=40)
    ap.add_argument("--config-warmup", type=int, default=200)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-calibration", type=float, default=0.0)
    return ap.parse_args()


def gemm_bytes(m, k, n, bits, experts=1, out_bytes=4):
    """Algorithmic HBM bytes of one GEMM: weight image, codes, scales, output (fp32: 4 bytes
    an element, bf16: 2)."""
    return experts * n * k * 18 // 32 + m * k * bits // 8 + m * (k // 32) * 4 + m * n * out_bytes


def strip_comments(text):
    """C++ source without its comments (string and character literals kept)
    and with every run of whitespace made one space, so that an edit of
    comments alone does not change the hash below."""
    out, i, n = [], 0, len(text)
    while i < n:
        ch = text[i]
        if ch in "\"'":
            j = i + 1
            while j < n and text[j] != ch:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(ch)
            i += 1
    return " ".join("".join(out).split())


def kernel_srcs(kname=None):
    """The sources one routed kernel depends on (kname as the routing query
    names it, e.g. "wide 64x160"), or every GEMM source (kname None)."""
    if kname is None:
        return GEMM_SRCS
    own = KERNEL_SRC.get(kname.split()[0])
    if own is None:
        raise ValueError("no source known for kernel %r" % kname)
    return SHARED_SRCS + [os.path.join(_CSRC, own)]


def source_hash(kname=None):
    """First 16 hex digits of sha256 over the kernel sources (comments
    removed; those of one routed kernel, or of all) and the flags they are
    compiled with."""
    from bit_prefill_gemm_amd.build import KERNEL_FLAGS
    h = hashlib.sha256()
    for f in sorted(set(kernel_srcs(kname))):
        h.update(strip_comments(open(f, encoding="utf-8").read()).encode("utf-8"))
    h.update(" ".join(KERNEL_FLAGS).encode("utf-8"))
    return h.hexdigest()[:16]


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def measured_traffic(workload, bits, kname, out="f32"):
    """HBM bytes per GEMM launch from the committed counter summary, if taken
    on the same kernel (its name and the hash of its sources are unchanged)."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    e = rec.get("workloads", {}).get("%s/%d%s" % (workload, bits, "" if out == "f32" else "/" + out))
    if not e or e.get("kernel") != kname or e.get("source_sha256_16") != source_hash(kname):
        return None
    return e["fetch_bytes"] + e["write_bytes"]


def cpu_baseline(data, wl, name, bits, seconds):
    import oracle
    x = data[wl.get("x", "x")]
    m, k, n = wl["m"], wl["k"], wl["n"]
    blocks = data[wl.get("w", "w")]
    if "experts" in wl:
        dec = [oracle.q4_0_decode(blocks[e], k) for e in range(wl["experts"])]
        off = data["offsets"]
    else:
        dec = [oracle.q4_0_decode(blocks, k)]
        off = np.array([0, m])
    reps, t0 = 0, time.perf_counter()
    while True:
        q, d, _ = oracle.quantize(x, bits)
        for e, (w, dw) in enumerate(dec):
            if off[e + 1] > off[e]:
                oracle.gemm_rect(q[off[e]:off[e + 1]], d[off[e]:off[e + 1]], w, dw,
                                 0, off[e + 1] - off[e], 0, n)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 50:
            break
    return {"value": reps * m / el, "unit": "tokens/s", "cores": oracle.num_threads(),
            "cpu": cpu_model(), "kind": "oracle",
            "sample": "whole %s workload (quantize %dx%d, then %dx%dx%d GEMM with fp64 "
                      "output), %d repetition(s) in %.1f s" % (name, m, k, m, k, n, reps, el)}


def roofline_of(kernel, m, k, n, bits, experts, seconds, traffic, out_bytes=4):
    """The binding roofline of one GEMM launch: whichever algorithmic floor of
    the contraction is larger, its 2*M*N*K int8 matrix ops at the dense int8
    peak or its HBM bytes at 8 TB/s."""
    gbytes = gemm_bytes(m, k, n, bits, experts, out_bytes)
    ops = 2.0 * m * n * k
    if gbytes / PEAK_HBM >= ops / PEAK_INT8_OPS:
        return {"bound": "hbm", "achieved": gbytes / seconds / 1e9, "peak": PEAK_HBM / 1e9,
                "unit": "GB/s", "frac": gbytes / seconds / PEAK_HBM, "traffic": traffic,
                "kernel": kernel}
    return {"bound": "mfma", "achieved": ops / seconds / 1e12, "peak": PEAK_INT8_OPS / 1e12,
            "unit": "TOP/s", "frac": ops / seconds / PEAK_INT8_OPS, "traffic": traffic,
            "kernel": kernel}


def epilogue_of(m, k, n, seconds):
    """The same launch against the fp32 epilogue floor: two FMAs (4 flops) per
    output element and 32-block at the fp32 vector peak."""
    flops = 4.0 * m * n * (k // 32)
    return {"achieved": flops / seconds / 1e12, "peak": PEAK_FP32_FLOPS / 1e12,
            "unit": "TFLOP/s", "frac": flops / seconds / PEAK_FP32_FLOPS}


def copy_calibration(nbytes):
    import torch
    n = int(nbytes) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()


def load_data(name, cache):
    from bit_prefill_gemm_amd import synth
    if name not in cache:
        cache[name] = synth.make(name)
    return cache[name]


def run_gemm(workload, bits, out_kind, steps, warmup, cold_bytes, cache):
    """quantize_act_h32 + w4a4_gemm (or the grouped product) on one workload:
    `steps` timed steps after `warmup`, cycling cold copies of the inputs."""
    import torch

    from bit_prefill_gemm_amd import binding as bb

    wl = WORKLOADS[workload]
    m, k, n = wl["m"], wl["k"], wl["n"]
    experts = wl.get("experts", 1)
    data = load_data(wl.get("src", workload), cache)
    W0 = bb.rotate_pack_weights(data[wl.get("w", "w")], bb.SRC_Q4_0_ROTATED, n, k, experts)

    dev = torch.device("cuda:0")
    x0 = torch.from_numpy(data[wl.get("x", "x")].view(np.int16)).to(dev).view(torch.bfloat16)
    offsets = (torch.from_numpy(data["offsets"].astype(np.int32)).to(dev)
               if experts > 1 else None)
    img0 = torch.from_numpy(W0.image).to(dev)
    per_copy = img0.numel() + x0.numel() * 2
    copies = max(1, int(math.ceil(cold_bytes / per_copy)))
    imgs = [img0] + [img0.clone() for _ in range(copies - 1)]
    xs = [x0] + [x0.clone() for _ in range(copies - 1)]
    Ws = [bb.Weights(W0.desc, im) for im in imgs]
    codes = torch.empty((m, k // 2 if bits == 4 else k), dtype=torch.uint8, device=dev)
    scales = torch.empty((m, k // 32), dtype=torch.float32, device=dev)
    bf16_out = out_kind == "bf16"
    out_bytes = 2 if bf16_out else 4
    y = torch.empty((m, n), dtype=torch.bfloat16 if bf16_out else torch.float32, device=dev)
    stream = torch.cuda.Stream(device=dev)
    if offsets is None:
        kname = bb.w4a4_gemm_kernel_name(bits, m, W0)
    else:
        kname = bb.w4a4_grouped_gemm_kernel_name(bits, m, W0)

    def quantize(j):
        bb.quantize_act_h32(xs[j], bits, codes=codes, scales=scales, stream=stream)

    def gemm(j):
        if offsets is None:
            f = bb.w4a4_gemm_bf16 if bf16_out else bb.w4a4_gemm
            f(codes, scales, bits, Ws[j], y=y, stream=stream)
        else:
            f = bb.w4a4_grouped_gemm_bf16 if bf16_out else bb.w4a4_grouped_gemm
            f(codes, scales, bits, offsets, Ws[j], y=y, stream=stream)

    def step(j):
        quantize(j)
        gemm(j)

    # The timed steps (one quantize and one product each) replay one captured
    # graph; the same steps issued eagerly are timed too (eager_step_us).
    # Each kernel's own duration is taken afterwards from a graph replay of
    # back-to-back launches over the same cold copies (graph_time_us).
    ms_per_step, eager_ms = timed_steps(torch, stream, step, steps, warmup, copies)
    gemm_spread = graph_time_spread_us(torch, stream, lambda i: gemm(i % copies))
    gemm_ms = gemm_spread[0] * 1e-3
    quant_ms = graph_time_us(torch, stream, lambda i: quantize(i % copies)) * 1e-3
    # whole steps replayed the same way: the product right after the quantizer
    # that wrote its codes runs a few percent longer than back to back
    step_graph_ms = graph_time_us(torch, stream,
                                  lambda i: (quantize(i % copies), gemm(i % copies))) * 1e-3

    gemm_s = gemm_ms * 1e-3
    eff_tops = 2.0 * m * n * k / gemm_s / 1e12
    gbytes = gemm_bytes(m, k, n, bits, experts, out_bytes)
    traffic = measured_traffic(workload, bits, kname, out_kind)
    entry = ("w4a4_gemm" if experts == 1 else "w4a4_grouped_gemm") + ("_bf16" if bf16_out else "")
    res = {
        "value": wl.get("tokens", m) / (ms_per_step * 1e-3),
        "ms_per_step": ms_per_step,
        "config": {"workload": "%s: M=%d K=%d N=%d%s, bf16 activations, rotated Q4_0 weights, "
                               "%d-bit activation codes"
                               % (workload, m, k, n,
                                  ", %d experts (grouped)" % experts if experts > 1 else "", bits),
                   "m": m, "k": k, "n": n, "experts": experts, "act_bits": bits,
                   "out": out_kind, "cold_copies": copies},
        "roofline": roofline_of(entry + ": " + kname, m, k, n, bits, experts, gemm_s, traffic,
                                out_bytes),
        "epilogue_valu": epilogue_of(m, k, n, gemm_s),
        "kernel": kname,
        "eff_TOPS": eff_tops,
        "pct_int8_peak": 100.0 * eff_tops / (PEAK_INT8_OPS / 1e12),
        "gemm_us": gemm_ms * 1e3,
        "gemm_us_min_max": [gemm_spread[1], gemm_spread[2]],
        "quant_us": quant_ms * 1e3,
        "step_graph_us": step_graph_ms * 1e3,
        "gemm_in_step_us": (step_graph_ms - quant_ms) * 1e3,
        "step_us": ms_per_step * 1e3,
        "eager_step_us": eager_ms * 1e3,
        "gemm_hbm_GBps": gbytes / gemm_s / 1e9,
        "pct_hbm": 100.0 * gbytes / gemm_s / PEAK_HBM,
        "gemm_algorithmic_bytes": gbytes,
    }
    del imgs, xs, Ws, img0, x0, codes, scales, y
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res, data


def summary(res):
    """The per-workload entry of `configs`."""
    if "kernel_us" in res:
        return {"step_us": res["step_us"], "eager_step_us": res["eager_step_us"],
                "tokens_per_s": res["value"],
                "kernel_us": res["kernel_us"], "roofline": res["roofline"]}
    r = res["roofline"]
    return {"kernel": res["kernel"], "gemm_us": res["gemm_us"],
            "gemm_us_min_max": res["gemm_us_min_max"], "quant_us": res["quant_us"],
            "gemm_in_step_us": res["gemm_in_step_us"],
            "step_us": res["step_us"], "eager_step_us": res["eager_step_us"],
            "tokens_per_s": res["value"],
            "roofline": {"bound": r["bound"], "frac": r["frac"], "achieved": r["achieved"],
                         "unit": r["unit"], "traffic": r["traffic"]},
            "int8_frac": res["pct_int8_peak"] / 100.0, "hbm_frac": res["pct_hbm"] / 100.0,
            "epilogue_valu_frac": res["epilogue_valu"]["frac"]}


def ffn_pair(configs, bits, m=512):
    """The FFN block's prompt rate from its two measured shapes: quantize X1,
    the gate and up products (one shape, measured once), quantize X2, the
    down product; each term the kernel's own graph-timed figure."""
    g, d = configs.get("ffn512_gate/%d" % bits), configs.get("ffn512_down/%d" % bits)
    if g is None or d is None:
        return None
    us = g["quant_us"] + 2.0 * g["gemm_us"] + d["quant_us"] + d["gemm_us"]
    return {"us_per_block": us, "tokens_per_s": m / (us * 1e-6),
            "terms_us": {"quantize_x1": g["quant_us"], "gate": g["gemm_us"],
                         "up": g["gemm_us"], "quantize_x2": d["quant_us"],
                         "down": d["gemm_us"]}}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    from bit_prefill_gemm_amd import binding as bb

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    bb.lib()
    wl = WORKLOADS[args.workload]
    cache = {}
    if wl.get("layer"):
        res, data = run_layer(args.bits, args.steps, args.warmup, args.cold_bytes, cache)
    else:
        res, data = run_gemm(args.workload, args.bits, args.out, args.steps, args.warmup,
                             args.cold_bytes, cache)
    out = {
        "metric": "prompt tokens/s + effective TOPS (% int8 MFMA peak) for rotated W4A4 GEMM, M=512",
        "value": res["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8" if args.bits == 8 else "i4",
        "data": "synthetic",
    }
    out.update({kk: v for kk, v in res.items() if kk not in ("value", "ms_per_step")})
    out["gemm_source_sha256_16"] = source_hash()
    if args.workload == "attn512" and not args.no_configs:
        configs = {}
        for name, bits in CONFIG_RUNS:
            if (name, bits) == (args.workload, args.bits):
                continue
            print("config %s %d-bit" % (name, bits), file=sys.stderr, flush=True)
            if WORKLOADS[name].get("layer"):
                r, _ = run_layer(bits, args.config_steps, args.config_warmup, args.cold_bytes,
                                 cache)
            else:
                r, _ = run_gemm(name, bits, "f32", args.config_steps, args.config_warmup,
                                args.cold_bytes, cache)
            configs["%s/%d" % (name, bits)] = summary(r)
        for bits in (4, 8):
            pair = ffn_pair(configs, bits)
            if pair is not None:
                configs["ffn512_block/%d" % bits] = pair
        out["configs"] = configs
    if not args.no_cpu_baseline:
        if wl.get("layer"):
            out["cpu_baseline"] = cpu_baseline_layer(data, res["routes"][0], res["routes"][1],
                                                     args.bits, args.cpu_seconds)
        else:
            out["cpu_baseline"] = cpu_baseline(data, wl, args.workload, args.bits,
                                               args.cpu_seconds)
    out.pop("routes", None)
    print(json.dumps(out))


def run_layer(bits, steps, warmup, cold_bytes, cache):
    """One step = one expert layer over 512 tokens (moe512: hidden 2048, 128
    experts, top-8, expert intermediate 768)."""
    import torch

    from bit_prefill_gemm_amd import binding as bb
    from bit_prefill_gemm_amd import synth

    data = load_data("moe512", cache)
    c = data["cfg"]
    T, H, E, K8, I = c["tokens"], c["hidden"], c["experts"], c["topk"], c["inter"]
    rows = T * K8
    e_np, w_np = synth.draw_routes(np.random.default_rng(21), T, E, K8)
    dev = torch.device("cuda:0")
    Wgu0 = bb.rotate_pack_weights(data["w_gu"], bb.SRC_Q4_0_ROTATED, 2 * I, H, E)
    Wdn0 = bb.rotate_pack_weights(data["w_dn"], bb.SRC_Q4_0_ROTATED, H, I, E)
    gu_img = torch.from_numpy(Wgu0.image).to(dev)
    dn_img = torch.from_numpy(Wdn0.image).to(dev)
    x0 = torch.from_numpy(data["x_tokens"].view(np.int16)).to(dev).view(torch.bfloat16)
    per_copy = gu_img.numel() + dn_img.numel() + x0.numel() * 2
    copies = max(1, int(math.ceil(cold_bytes / per_copy)))
    Wgu = [bb.Weights(Wgu0.desc, gu_img if j == 0 else gu_img.clone()) for j in range(copies)]
    Wdn = [bb.Weights(Wdn0.desc, dn_img if j == 0 else dn_img.clone()) for j in range(copies)]
    xs = [x0 if j == 0 else x0.clone() for j in range(copies)]
    expert_of = torch.from_numpy(e_np).to(dev)
    weights = torch.from_numpy(w_np).to(dev)
    ab = 2 if bits == 4 else 1
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    row_token = torch.empty(rows, dtype=torch.int32, device=dev)
    slot_of = torch.empty(rows, dtype=torch.int32, device=dev)
    codes = torch.empty((T, H // ab), dtype=torch.uint8, device=dev)
    scales = torch.empty((T, H // 32), dtype=torch.float32, device=dev)
    gu = torch.empty((rows, 2 * I), dtype=torch.float32, device=dev)
    hc = torch.empty((rows, I // ab), dtype=torch.uint8, device=dev)
    hs = torch.empty((rows, I // 32), dtype=torch.float32, device=dev)
    dn = torch.empty((rows, H), dtype=torch.float32, device=dev)
    y = torch.empty((T, H), dtype=torch.float32, device=dev)
    stream = torch.cuda.Stream(device=dev)
    lib = bb.lib()
    sh = bb._stream_handle(stream)

    def check(st, what):
        if st != 0:
            raise bb.BpgError(st, what)

    kernels = {
        "moe_route_sort": lambda j: check(lib.moe_route_sort(
            bb._dptr(expert_of), T, K8, E, bb._dptr(offsets), bb._dptr(row_token),
            bb._dptr(slot_of), sh), "sort"),
        "quantize_act_h32": lambda j: bb.quantize_act_h32(xs[j], bits, codes=codes, scales=scales,
                                                          stream=stream),
        "w4a4_grouped_gemm_gather": lambda j: bb.w4a4_grouped_gemm_gather(
            codes, scales, bits, row_token, offsets, Wgu[j], y=gu, stream=stream),
        "swiglu_quantize_h32": lambda j: bb.swiglu_quantize_h32(gu, I, bits, codes=hc, scales=hs,
                                                                stream=stream),
        "w4a4_grouped_gemm": lambda j: bb.w4a4_grouped_gemm(hc, hs, bits, offsets, Wdn[j], y=dn,
                                                            stream=stream),
        "moe_combine": lambda j: bb.moe_combine(dn, slot_of, weights, T, K8, y=y, stream=stream),
    }

    gate_name = "w4a4_grouped_gemm_gather"

    def step(j):
        for f in kernels.values():
            f(j)

    ms_per_step, eager_ms = timed_steps(torch, stream, step, steps, warmup, copies)
    # each kernel's own duration: a graph replay of back-to-back launches of
    # it alone over the cold copies (every kernel of the step rewrites its
    # outputs from its inputs, so repeating one is the same work each time)
    kernel_us = {name: graph_time_us(torch, stream, lambda i, f=f: f(i % copies))
                 for name, f in kernels.items()}
    gate_s = kernel_us[gate_name] * 1e-6
    kname = bb.w4a4_grouped_gemm_kernel_name(bits, rows, Wgu0, src_rows=T)
    roofline = roofline_of("w4a4_grouped_gemm_gather: " + kname, rows, H, 2 * I, bits, E, gate_s,
                           None)
    res = {
        "value": T / (ms_per_step * 1e-3),
        "ms_per_step": ms_per_step,
        "config": {"workload": "moe512_layer: expert layer over %d tokens, hidden %d, %d experts, "
                               "top-%d, expert intermediate %d, bf16 activations, rotated Q4_0 "
                               "weights, %d-bit activation codes" % (T, H, E, K8, I, bits),
                   "tokens": T, "hidden": H, "experts": E, "topk": K8, "inter": I,
                   "act_bits": bits, "cold_copies": copies},
        "roofline": roofline,
        "kernel_us": kernel_us,
        "step_us": ms_per_step * 1e3,
        "eager_step_us": eager_ms * 1e3,
        "routes": (e_np, w_np),
    }
    del Wgu, Wdn, xs, gu_img, dn_img, x0
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res, data


def cpu_baseline_layer(data, e_np, w_np, bits, seconds):
    """The oracle's expert layer (same steps, fp64 GEMM outputs rounded to fp32
    between steps) on the same 512 tokens."""
    import oracle
    c = data["cfg"]
    T, H, E, K8, I = c["tokens"], c["hidden"], c["experts"], c["topk"], c["inter"]
    gu_dec = [oracle.q4_0_decode(data["w_gu"][e], H) for e in range(E)]
    dn_dec = [oracle.q4_0_decode(data["w_dn"][e], I) for e in range(E)]
    reps, t0 = 0, time.perf_counter()
    while True:
        off, entry, slot = oracle.route_sort(e_np, E)
        q, d, _ = oracle.quantize(data["x_tokens"], bits)
        rt = entry // K8
        qg, dg = q[rt], d[rt]
        gu = np.zeros((T * K8, 2 * I), dtype=np.float32)
        for e in range(E):
            a, b = off[e], off[e + 1]
            if b > a:
                w, dw = gu_dec[e]
                gu[a:b] = oracle.gemm_rect(qg[a:b], dg[a:b], w, dw, 0, b - a, 0, 2 * I)
        hq, hd, _ = oracle.swiglu_quantize(gu, I, bits)
        dn = np.zeros((T * K8, H), dtype=np.float32)
        for e in range(E):
            a, b = off[e], off[e + 1]
            if b > a:
                w, dw = dn_dec[e]
                dn[a:b] = oracle.gemm_rect(hq[a:b], hd[a:b], w, dw, 0, b - a, 0, H)
        oracle.moe_combine(dn, slot, w_np, T, K8)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 20:
            break
    return {"value": reps * T / el, "unit": "tokens/s", "cores": oracle.num_threads(),
            "cpu": cpu_model(), "kind": "oracle",
            "sample": "whole moe512 expert layer (sort, quantize, gate/up, SwiGLU-quantize, "
                      "down, combine), %d repetition(s) in %.1f s" % (reps, el)}


if __name__ == "__main__":
    main()
