"""moe_forward_noalloc (the entry point that allocates nothing, its workspace a static
scratch array in the library) against moe_forward with a caller workspace: bit for bit, on
two calls in a row, the second with fewer tokens, through the C ABI."""
import numpy as np
import pytest

import moe_synth as S

import gpu_cases as C

pytestmark = pytest.mark.gpu


def _bits(t):
    import torch
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


@pytest.mark.parametrize("wl,Ts", [(S.OLMOE_BF16, (300, 5)), (S.DEEPSEEK_I8, (512, 16)),
                                   (S.TINY_F32, (200, 16))], ids=lambda v: getattr(v, "name", str(v)))
def test_noalloc_matches_forward_on_two_calls(wl, Ts):
    import torch
    from grouped_expert_ffn_amd import abi, to_device
    gl = C.GpuLayer(wl)
    dev = gl.dev
    for i, T in enumerate(Ts):
        print(f"no-alloc {wl.name} call {i} T={T}", flush=True)
        x = to_device(S.make_tokens(wl, T, seed=10 + i))
        res = to_device(S.make_tokens(wl, T, seed=20 + i))
        ids_a = torch.empty((T, wl.k), dtype=torch.int32, device="cuda")
        w_a = torch.empty((T, wl.k), dtype=torch.float32, device="cuda")
        y_a = dev.forward(x, residual=res, topk_ids=ids_a, topk_w=w_a)
        ids_b = torch.full((T, wl.k), -7, dtype=torch.int32, device="cuda")
        w_b = torch.full((T, wl.k), -7.0, dtype=torch.float32, device="cuda")
        y_b = torch.full_like(x, 3.0)
        abi.moe_forward_noalloc(dev.desc, T, x, dev.w_router, dev.bias, dev.weights, res, y_b,
                                ids_b, w_b)
        torch.cuda.synchronize()
        assert torch.equal(ids_a, ids_b)
        assert torch.equal(w_a, w_b)
        assert torch.equal(_bits(y_a), _bits(y_b)), f"{wl.name} T={T}: outputs differ"
        assert np.all(np.isfinite(C.widen_dev(y_b)))


# The callers it is for include code under HIP graph capture: the call captured in a graph
# (nothing to allocate while capturing) replays the eager result bit for bit, with eager calls
# of the same entry point between the replays.
@pytest.mark.parametrize("wl,T", [(S.OLMOE_BF16, 8), (S.DEEPSEEK_BF16, 300)],
                         ids=lambda v: getattr(v, "name", str(v)))
def test_noalloc_under_graph_capture_matches_eager(wl, T):
    import torch
    from grouped_expert_ffn_amd import abi, to_device
    gl = C.GpuLayer(wl)
    dev = gl.dev
    print(f"no-alloc graph {wl.name} T={T}", flush=True)
    x = to_device(S.make_tokens(wl, T, seed=30))
    x_other = to_device(S.make_tokens(wl, T, seed=31))
    y_ref = torch.empty_like(x)
    abi.moe_forward_noalloc(dev.desc, T, x, dev.w_router, dev.bias, dev.weights, None, y_ref,
                            None, None)
    torch.cuda.synchronize()
    y = torch.empty_like(x)
    y_other = torch.empty_like(x)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        abi.moe_forward_noalloc(dev.desc, T, x, dev.w_router, dev.bias, dev.weights, None, y,
                                None, None, stream=torch.cuda.current_stream().cuda_stream)
    for _ in range(3):
        y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(y), _bits(y_ref))
        abi.moe_forward_noalloc(dev.desc, T, x_other, dev.w_router, dev.bias, dev.weights, None,
                                y_other, None, None)  # eager use of the same scratch between
        torch.cuda.synchronize()
    del g
