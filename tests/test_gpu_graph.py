"""The entry points replayed from a captured HIP graph give the eager results.

bench.py times its steps as one captured graph, so every kernel family it
replays is checked here the same way: the calls are captured once, then the
graph is replayed several times, with the program's own eager work (the same
calls on other buffers, the outputs cleared by fill kernels) and a device
synchronisation between replays, and every replay's codes, scales and outputs
must equal the eager ones bit for bit (the kernels are deterministic).  The
library enqueues kernels only: no memory-set or copy nodes enter a graph.
"""
import numpy as np
import pytest

from bit_prefill_gemm_amd import binding as bb
from bit_prefill_gemm_amd import synth

from gpu_util import act_to_device, torch_mod, weights_to_device

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(scope="module")
def torch():
    t = torch_mod()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    return t


def replay_and_check(torch, capture, eager_work, clear, refs, names, label):
    """Capture `capture()` (which returns its output tensors) on a side stream,
    then replay it REPLAYS times; before each replay run `eager_work()` and
    `clear(outputs)`, after it compare the outputs with `refs` bit for bit."""
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        outputs = capture()
    torch.cuda.synchronize()
    assert len(outputs) == len(refs) == len(names)
    for rep in range(REPLAYS):
        eager_work()
        clear(outputs)
        torch.cuda.synchronize()
        print(label, "replay", rep, flush=True)
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        for name, got, ref in zip(names, outputs, refs):
            a = got.contiguous().view(torch.uint8).cpu().numpy()
            b = ref.contiguous().view(torch.uint8).cpu().numpy()
            assert np.array_equal(a, b), "%s: replay %d: %s differs from the eager result" % (
                label, rep, name)
    del g


def clear_all(torch, tensors):
    """Fill kernels (never memory-set nodes): NaN in float outputs, zeros elsewhere."""
    for t in tensors:
        if t.dtype == torch.float32:
            t.fill_(float("nan"))
        else:
            t.zero_()


DENSE = [
    # m, k, n, bits, kernel
    (16, 1024, 256, 4, "weight-stream"),
    (16, 1024, 256, 8, "weight-stream"),
    (100, 1024, 256, 4, "strip 32x128"),
    (100, 1024, 256, 8, "strip 32x128"),
    (512, 512, 5120, 4, "wide 64x160"),
    (512, 512, 5120, 8, "tiled 64x160"),
    (96, 1024, 320, 4, "tiled 64x32"),
]


@pytest.mark.parametrize("m,k,n,bits,kernel", DENSE,
                         ids=["%dx%dx%d-%d" % c[:4] for c in DENSE])
def test_dense_step_replays(torch, m, k, n, bits, kernel):
    """quantize_act_h32 + w4a4_gemm captured as one step."""
    case = synth.small_dense(m, k, n, seed=m + k + n + bits, dtype="bf16")
    x = act_to_device(case["x"])
    x_other = act_to_device(synth.small_dense(m, k, n, seed=7, dtype="bf16")["x"])
    W = weights_to_device(case["w"], n, k)
    assert bb.w4a4_gemm_kernel_name(bits, m, W) == kernel
    codes_ref, scales_ref = bb.quantize_act_h32(x, bits)
    y_ref = bb.w4a4_gemm(codes_ref, scales_ref, bits, W)
    torch.cuda.synchronize()
    codes = torch.empty_like(codes_ref)
    scales = torch.empty_like(scales_ref)
    y = torch.empty_like(y_ref)
    codes_o, scales_o = torch.empty_like(codes_ref), torch.empty_like(scales_ref)
    y_o = torch.empty_like(y_ref)

    def capture():
        bb.quantize_act_h32(x, bits, codes=codes, scales=scales)
        bb.w4a4_gemm(codes, scales, bits, W, y=y)
        return [codes, scales, y]

    def eager_work():
        bb.quantize_act_h32(x_other, bits, codes=codes_o, scales=scales_o)
        bb.w4a4_gemm(codes_o, scales_o, bits, W, y=y_o)

    replay_and_check(torch, capture, eager_work, lambda outs: clear_all(torch, outs),
                     [codes_ref, scales_ref, y_ref], ["codes", "scales", "y"],
                     "dense %dx%dx%d %d-bit" % (m, k, n, bits))


def expert_setup(torch, tokens, experts, topk, hidden, inter, seed):
    rng = np.random.default_rng(seed)
    e, w = synth.draw_routes(rng, tokens, experts, topk)
    x = synth.bf16_bits(rng.standard_normal((tokens, hidden)).astype(np.float32))
    w_gu = synth.draw_q4_0(rng, (experts, 2 * inter), hidden, 0.005, 0.05)
    w_dn = synth.draw_q4_0(rng, (experts, hidden), inter, 0.005, 0.05)
    Wgu = weights_to_device(w_gu.reshape(experts * 2 * inter, hidden // 32, 18), 2 * inter,
                            hidden, experts)
    Wdn = weights_to_device(w_dn.reshape(experts * hidden, inter // 32, 18), hidden, inter,
                            experts)
    ed = torch.from_numpy(e.astype(np.int32)).cuda()
    wd = torch.from_numpy(w.astype(np.float32)).cuda()
    return act_to_device(x), ed, wd, Wgu, Wdn


@pytest.mark.parametrize("bits,kernel", [(4, "expert-slot"), (8, "grouped 32x128")])
def test_expert_layer_replays(torch, bits, kernel):
    """The whole expert layer (sort, token quantize, gathered gate/up,
    SwiGLU-quantize, down, combine) captured as one step."""
    T, E, K8, H, I = 96, 16, 4, 256, 128
    x, ed, wd, Wgu, Wdn = expert_setup(torch, T, E, K8, H, I, seed=bits)
    assert bb.w4a4_grouped_gemm_kernel_name(bits, T * K8, Wgu, src_rows=T) == kernel

    def layer():
        off, row_token, slot_of = bb.moe_route_sort(ed, T, K8, E)
        codes, scales = bb.quantize_act_h32(x, bits)
        gu = bb.w4a4_grouped_gemm_gather(codes, scales, bits, row_token, off, Wgu)
        hc, hs = bb.swiglu_quantize_h32(gu, I, bits)
        dn = bb.w4a4_grouped_gemm(hc, hs, bits, off, Wdn)
        y = bb.moe_combine(dn, slot_of, wd, T, K8)
        return [off, row_token, slot_of, codes, scales, gu, hc, hs, dn, y]

    names = ["offsets", "row_token", "slot_of", "codes", "scales", "gate/up", "h codes",
             "h scales", "down", "y"]
    refs = layer()
    torch.cuda.synchronize()
    # the captured calls allocate their outputs from the graph's own pool
    replay_and_check(torch, layer, layer, lambda outs: clear_all(torch, outs), refs, names,
                     "expert layer %d-bit" % bits)
