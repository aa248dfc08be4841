"""Entry points called concurrently: two host threads, each issuing products on
its own stream, give the same results as the same calls one after the other
(the library keeps no per-call state; its one process-wide cache, the device
check, is written once and atomically)."""
import threading

import numpy as np
import pytest

from bit_prefill_gemm_amd import binding as bb
from bit_prefill_gemm_amd import synth

from gpu_util import act_to_device, torch_mod, weights_to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    t = torch_mod()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    return t


def test_two_threads_two_streams(torch):
    cases = [(16, 1024, 256, 4), (200, 1056, 1280, 4), (100, 1024, 256, 8)]
    work = []
    for i, (m, k, n, bits) in enumerate(cases):
        case = synth.small_dense(m, k, n, seed=90 + i, dtype="bf16")
        x = act_to_device(case["x"])
        W = weights_to_device(case["w"], n, k)
        codes, scales = bb.quantize_act_h32(x, bits)
        ref = bb.w4a4_gemm(codes, scales, bits, W)
        work.append((x, W, bits, codes, scales, ref))
    torch.cuda.synchronize()
    refs = [(c.cpu().numpy(), s.cpu().numpy(), r.cpu().numpy()) for _, _, _, c, s, r in work]

    errors = []

    def run(tid):
        try:
            stream = torch.cuda.Stream()
            order = list(range(len(work)))[tid::2] + list(range(len(work)))[1 - tid::2]
            outs = []
            with torch.cuda.stream(stream):
                for rep in range(20):
                    for idx in order:
                        x, W, bits = work[idx][:3]
                        c, s = bb.quantize_act_h32(x, bits, stream=stream)
                        y = bb.w4a4_gemm(c, s, bits, W, stream=stream)
                        outs.append((idx, c, s, y))
            stream.synchronize()
            for j, (idx, c, s, y) in enumerate(outs):
                rc, rs, ry = refs[idx]
                if not (np.array_equal(c.cpu().numpy(), rc) and
                        np.array_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32)) and
                        np.array_equal(y.cpu().numpy().view(np.uint32), ry.view(np.uint32))):
                    errors.append("thread %d call %d (case %d) differs" % (tid, j, idx))
                    return
        except Exception as e:  # reported below, on the main thread
            errors.append("thread %d: %r" % (tid, e))

    threads = [threading.Thread(target=run, args=(t,)) for t in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
