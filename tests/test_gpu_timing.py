"""The per-kernel timing hook (moe_time_next_launch) that bench.py's roofline figures rest
on: every kernel of a forward gets a positive time, the times fit inside the step, the hook
fires once, and the multi-launch sort (past one workgroup's rows) is bracketed as a whole."""
import pytest

import moe_synth as S
from tests import gpu_cases as C

pytestmark = pytest.mark.gpu


def _events(t, n):
    evs = [(t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in evs:  # torch creates the HIP events on their first record
        a.record()
        b.record()
    t.cuda.synchronize()
    return evs


def _layer(wl, T):
    from grouped_expert_ffn_amd import to_device
    gl = C.GpuLayer(wl)
    return gl, to_device(S.make_tokens(wl, T))


# T=8: the down projection and the combine run as one launch (decode sizes); T=64: separate
@pytest.mark.parametrize("T,fused", [(8, True), (64, False)])
def test_every_kernel_of_a_forward_is_timed_inside_the_step(T, fused):
    from grouped_expert_ffn_amd import abi
    t = C.torch()
    wl = S.OLMOE_BF16
    gl, x = _layer(wl, T)
    gl.dev.forward(x)
    t.cuda.synchronize()
    kernels = [abi.MOE_KERNEL_ROUTER, abi.MOE_KERNEL_PERMUTE, abi.MOE_KERNEL_GATE_UP,
               abi.MOE_KERNEL_DOWN, abi.MOE_KERNEL_COMBINE]
    evs = _events(t, len(kernels))
    step = _events(t, 1)[0]
    for kern, (a, b) in zip(kernels, evs):
        abi.moe_time_next_launch(kern, a, b)
    step[0].record()
    gl.dev.forward(x)
    step[1].record()
    t.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in evs]
    total = step[0].elapsed_time(step[1])
    print("kernel ms", [round(m, 4) for m in ms], "step ms", round(total, 4))
    assert all(m > 0 for m in ms), ms
    if fused:
        # the combine's hook brackets the launch whose own window the down projection's holds
        assert ms[4] >= ms[3] * 0.999, ms
        assert sum(ms[:4]) <= total * 1.001, (ms, total)
    else:
        assert sum(ms) <= total * 1.001, (ms, total)
    # the weight-streaming GEMVs dominate the decode layer
    assert ms[2] > ms[0] and ms[2] > ms[1] and ms[2] > ms[4]


def test_hook_fires_once():
    from grouped_expert_ffn_amd import abi
    t = C.torch()
    gl, x = _layer(S.OLMOE_BF16, 8)
    (a, b), (c, d) = _events(t, 2)
    abi.moe_time_next_launch(abi.MOE_KERNEL_GATE_UP, a, b)
    gl.dev.forward(x)
    t.cuda.synchronize()
    first = a.elapsed_time(b)
    # a second forward must not record the (now disarmed) events again: arm a fresh pair for
    # the down kernel only and check the gate/up pair still holds the first launch's time
    abi.moe_time_next_launch(abi.MOE_KERNEL_DOWN, c, d)
    gl.dev.forward(x)
    t.cuda.synchronize()
    assert a.elapsed_time(b) == first
    assert c.elapsed_time(d) > 0


@pytest.mark.parametrize("T", [600, 8300])  # 5 chunks (two launches); 65 chunks (three)
def test_multi_launch_sort_is_bracketed(T):
    # T*k past one workgroup's rows: the sort is a histogram launch, past 64 chunks a scan,
    # and the sort launch, and the hook brackets them all
    from grouped_expert_ffn_amd import abi
    t = C.torch()
    gl, x = _layer(S.OLMOE_BF16, T)
    gl.dev.forward(x)
    t.cuda.synchronize()
    (a, b), (c, d) = _events(t, 2)
    abi.moe_time_next_launch(abi.MOE_KERNEL_PERMUTE, a, b)
    abi.moe_time_next_launch(abi.MOE_KERNEL_GATE_UP, c, d)
    gl.dev.forward(x)
    t.cuda.synchronize()
    assert a.elapsed_time(b) > 0 and c.elapsed_time(d) > 0
