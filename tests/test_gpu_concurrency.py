"""Calls on several streams and host threads at once: every call owns its workspace and
outputs, so the results must equal the same calls made one after another, bit for bit (the
library keeps no state between calls other than per-thread error and timing-hook slots and
per-device attribute flags)."""
import threading

import pytest

import moe_synth as S
from tests import gpu_cases as C

pytestmark = pytest.mark.gpu

# one decode layer on the VALU GEMV, one prefill-size layer on the ring GEMM (different
# kernels in flight at once), and the fp32 layer
CASES = [(S.OLMOE_BF16, 8, 0), (S.DEEPSEEK_BF16, 300, 1), (S.TINY_F32, 40, 2)]


def test_threads_on_their_own_streams_match_serial_calls():
    from grouped_expert_ffn_amd import DeviceLayer, to_device
    t = C.torch()
    jobs = []
    for wl, T, seed in CASES:
        gl = C.GpuLayer(wl)
        d = gl.dev
        # a layer object per thread: DeviceLayer keeps one workspace per object
        mine = DeviceLayer(gl.desc, d.w_router, d.bias, d.w_gate, d.w_up, d.w_down, d.s_gate,
                           d.s_up, d.s_down)
        x = to_device(S.make_tokens(wl, T, seed=seed))
        jobs.append((mine, x))
    ref = [layer.forward(x) for layer, x in jobs]
    t.cuda.synchronize()

    reps = 20
    out = [None] * len(jobs)
    errors = []

    def run(i):
        try:
            layer, x = jobs[i]
            s = t.cuda.Stream()
            with t.cuda.stream(s):
                y = None
                for _ in range(reps):
                    y = layer.forward(x)
                s.synchronize()
            out[i] = y
        except Exception as e:  # noqa: BLE001 - reported below
            errors.append(repr(e))

    threads = [threading.Thread(target=run, args=(i,)) for i in range(len(jobs))]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads), "a thread did not finish"
    assert not errors, errors
    t.cuda.synchronize()
    for (wl, T, _), y, r in zip(CASES, out, ref):
        assert t.equal(y, r), f"{wl.name} T={T}: concurrent result differs from the serial one"
