"""bench.py's workloads against the synthetic recipes they draw from (host
only: no data is generated)."""
import os
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402
from bit_prefill_gemm_amd import synth  # noqa: E402


@pytest.mark.parametrize("name", sorted(bench.WORKLOADS))
def test_workload_matches_recipe(name):
    wl = bench.WORKLOADS[name]
    cfg = synth.CONFIGS[wl.get("src", "moe512" if wl.get("layer") else name)]
    if wl.get("layer") or wl.get("experts"):
        assert cfg["experts"] == wl["experts"] and cfg["tokens"] == wl["tokens"]
        if not wl.get("layer"):
            # gate/up: K = hidden, N = 2 x intermediate; down: K = intermediate, N = hidden
            gu = (cfg["hidden"], 2 * cfg["inter"])
            dn = (cfg["inter"], cfg["hidden"])
            assert (wl["k"], wl["n"]) in (gu, dn)
            assert wl["m"] == cfg["tokens"] * cfg["topk"]
        return
    if name == "ffn512_down":
        # the down projection maps the FFN width back to the model width
        assert (wl["m"], wl["k"], wl["n"]) == (cfg["m"], cfg["n"], cfg["k"])
        assert wl["x"] == "x2" and wl["w"] == "w_down"
        return
    assert (wl["m"], wl["k"], wl["n"]) == (cfg["m"], cfg["k"], cfg["n"])
    assert wl["k"] % 32 == 0 and wl["n"] % 32 == 0


def test_default_workload_is_the_attention_projection():
    args = sys.argv
    try:
        sys.argv = ["bench.py"]
        assert bench.parse().workload == "attn512"
    finally:
        sys.argv = args


def test_ffn_block_rate_sums_its_kernels():
    # combined rate of the FFN pair: q(X1) + gate + up + q(X2) + down
    configs = {"ffn512_gate/4": {"quant_us": 6.0, "gemm_us": 140.0},
               "ffn512_down/4": {"quant_us": 10.0, "gemm_us": 120.0}}
    pair = bench.ffn_pair(configs, 4)
    assert pair["us_per_block"] == 6.0 + 2 * 140.0 + 10.0 + 120.0
    assert abs(pair["tokens_per_s"] - 512 / 416e-6) < 1e-6
    assert bench.ffn_pair(configs, 8) is None
