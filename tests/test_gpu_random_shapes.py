"""Seeded random layer shapes and options through moe_forward, against the fp64 oracle.

Each case draws the activation and weight types, d and I (multiples of 16, so both the
ring GEMM and the general GEMM for K % 32 != 0 are reached), E, k, shared experts, T,
routing (uniform or Zipf), renormalisation, the RMSNorm prologue, a residual and a capacity
factor.  The expert choice is checked against the oracle's (ties within the pre-registered
margin may differ) and the output, with the oracle using the GPU's choice, to the usual
tolerance on a token sample.
"""
import numpy as np
import pytest

import moe_synth as S
from oracle import moe_oracle as O
from tests import gpu_cases as C

pytestmark = pytest.mark.gpu

N_CASES = 32


def draw_case(i: int):
    g = np.random.default_rng(9000 + i)
    act, wdt = [("f32", "f32"), ("bf16", "bf16"), ("bf16", "i8")][int(g.integers(3))]
    E = int(g.choice([1, 2, 3, 5, 8, 17, 40, 64, 100, 256]))
    k = int(g.integers(1, min(E, 16) + 1))
    n_shared = int(g.choice([0, 0, 1, 2, 8]))
    # keep the layer's weights small enough for a quick fp64 oracle
    cap_dim = 640 if E + n_shared <= 24 else (256 if E + n_shared <= 72 else 128)
    d = 16 * int(g.integers(1, cap_dim // 16 + 1))
    I = 16 * int(g.integers(1, cap_dim // 16 + 1))
    T = int(g.choice([1, 2, 3, 7, 8, 9, 16, 17, 40, 130, 300]))
    zipf = bool(g.integers(2))
    cf = float(g.choice([0.0, 0.0, 0.75, 1.25, 2.0]))
    wl = S.Workload(f"rand{i}", 300 + i, d=d, E=E, k=k, I=I, S=n_shared,
                    renormalize=bool(g.integers(2)), act=act, wdt=wdt,
                    routing="zipf" if zipf else "uniform", zipf_alpha=1.2 if zipf else 0.0,
                    pre_norm=bool(g.integers(2)), tokens=(T,))
    return wl, T, cf, bool(g.integers(2))


CASES = [draw_case(i) for i in range(N_CASES)]


def case_name(c):
    wl, T, cf, res = c
    return (f"{wl.name}-{wl.act}-{wl.wdt}-d{wl.d}-I{wl.I}-E{wl.E}-k{wl.k}-S{wl.S}-T{T}"
            f"-cf{cf}{'-norm' if wl.pre_norm else ''}{'-res' if res else ''}")


@pytest.mark.parametrize("case", CASES, ids=[case_name(c) for c in CASES])
def test_random_layer_matches_oracle(case):
    from grouped_expert_ffn_amd import DTYPES, DeviceLayer, make_desc, to_device
    t = C.torch()
    wl, T, cf, use_res = case
    host = S.make_layer(wl, 0)
    desc = make_desc(wl.d, wl.E, wl.k, wl.I, wl.S, wl.renormalize, DTYPES[wl.act], DTYPES[wl.wdt],
                     wl.pre_norm, wl.norm_eps, capacity_factor=cf)
    dl = DeviceLayer(desc, host.w_router, host.bias, host.w_gate, host.w_up, host.w_down,
                     host.s_gate, host.s_up, host.s_down)
    x = S.make_tokens(wl, T)
    xd = to_device(x)
    ids = t.empty((T, wl.k), dtype=t.int32, device="cuda")
    y = dl.forward(xd, residual=xd if use_res else None, topk_ids=ids)
    t.cuda.synchronize()
    ids_g = ids.cpu().numpy()
    # the oracle's view of the router input
    if wl.pre_norm:
        xn = O.stack_layer_input(x, wl.norm_eps) if wl.act == "bf16" else O.rmsnorm(x, wl.norm_eps)
        delta = C.TIE_DELTA_STACK if wl.act == "bf16" else C.TIE_DELTA
    else:
        xn, delta = x, C.TIE_DELTA
    logits = O.router_logits(xn, host.w_router, host.bias)
    C.check_routing_against_oracle(ids_g, logits, wl.k, delta)
    w_ref = O.gate_weights_for(logits, ids_g, wl.renormalize)
    keep = O.kept_slots(ids_g, wl.E, O.capacity(cf, T, wl.k, wl.E))
    tok = list(range(T)) if T <= 40 else sorted(set(range(0, T, max(1, T // 24))) | {T - 1})
    y_ref = O.moe_layer(xn, O.Experts.from_layer(host), ids_g, w_ref, wl.S, wl.E,
                        residual=x if use_res else None, tokens=tok, keep=keep)
    C.assert_close(C.widen_dev(y)[tok], y_ref, wl.act, case_name(case))


# Decode sizes (T = 1-9), where moe_forward runs the down projection and the combine in one
# launch whenever the rows fit one workgroup's LDS: the forward against the separate C-ABI
# steps, bit for bit, over random shapes, options, residuals and capacity factors.
N_DECODE = 60


def draw_decode(i: int):
    g = np.random.default_rng(20000 + i)
    act, wdt = [("f32", "f32"), ("bf16", "bf16"), ("bf16", "i8")][int(g.integers(3))]
    E = int(g.choice([1, 2, 3, 5, 8, 17, 40, 64, 100, 256]))
    k = int(g.integers(1, min(E, 16) + 1))
    n_shared = int(g.choice([0, 0, 1, 2, 8]))
    cap_dim = 640 if E + n_shared <= 24 else (256 if E + n_shared <= 72 else 128)
    d = 16 * int(g.integers(1, cap_dim // 16 + 1))
    I = 16 * int(g.integers(1, cap_dim // 16 + 1))
    T = int(g.integers(1, 10))
    cf = float(g.choice([0.0, 0.0, 0.5, 1.0, 2.0]))
    wl = S.Workload(f"rd{i}", 700 + i, d=d, E=E, k=k, I=I, S=n_shared, renormalize=bool(g.integers(2)),
                    act=act, wdt=wdt, routing="zipf" if g.integers(2) else "uniform", zipf_alpha=1.2,
                    tokens=(T,))
    return wl, T, cf, bool(g.integers(2))


DECODE_CASES = [draw_decode(i) for i in range(N_DECODE)]


@pytest.mark.parametrize("case", DECODE_CASES, ids=[case_name(c) for c in DECODE_CASES])
def test_random_decode_forward_matches_steps(case):
    from grouped_expert_ffn_amd import DTYPES, DeviceLayer, make_desc, to_device
    t = C.torch()
    wl, T, cf, use_res = case
    host = S.make_layer(wl, 0)
    desc = make_desc(wl.d, wl.E, wl.k, wl.I, wl.S, wl.renormalize, DTYPES[wl.act], DTYPES[wl.wdt],
                     capacity_factor=cf)
    dl = DeviceLayer(desc, host.w_router, host.bias, host.w_gate, host.w_up, host.w_down,
                     host.s_gate, host.s_up, host.s_down)
    xd = to_device(S.make_tokens(wl, T))
    res = to_device(S.make_tokens(wl, T, seed=3)) if use_res else None
    y = dl.forward(xd, residual=res)

    class Layer:  # run_steps needs the workload, the descriptor and the device weights
        pass
    gl = Layer()
    gl.wl, gl.desc, gl.dev = wl, desc, dl
    steps = C.run_steps(gl, xd, T, desc=desc, residual=res)
    t.cuda.synchronize()
    assert t.equal(y, steps["y"]), case_name(case)
