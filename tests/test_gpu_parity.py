"""GPU parity of every step of the path against the fp64 oracle, through the C ABI.

Routing (in logits-input mode), expert counts and the permutation are compared bit for
bit; floating-point outputs to rel-L2 <= 1e-5 (fp32) / 1e-2 (bf16, int8 weights) and
max-abs <= 2e-2 * max|y|, on the same rounded inputs.
"""
import dataclasses

import numpy as np
import pytest

import moe_synth as S
from oracle import moe_oracle as O
from tests import gpu_cases as C

pytestmark = pytest.mark.gpu


def T_():
    return C.torch()


# ----------------------------------------------------------------------------------------
# step 1: top-k on given logits is bit-exact
# ----------------------------------------------------------------------------------------
def logits_case(kind, T, E, seed):
    g = np.random.default_rng(seed)
    if kind == "normal":
        return g.standard_normal((T, E)).astype(np.float32)
    if kind == "ties":
        return g.integers(-3, 3, size=(T, E)).astype(np.float32)
    if kind == "specials":
        a = g.standard_normal((T, E)).astype(np.float32)
        a[g.random((T, E)) < 0.05] = np.inf
        a[g.random((T, E)) < 0.05] = -np.inf
        a[g.random((T, E)) < 0.05] = np.nan
        a[g.random((T, E)) < 0.1] = -0.0
        a[g.random((T, E)) < 0.1] = 0.0
        return a
    raise ValueError(kind)


@pytest.mark.parametrize("E,k,renorm", [(8, 2, True), (64, 8, False), (64, 6, True), (256, 16, False),
                                        (64, 1, False), (5, 5, True), (130, 3, True)])
@pytest.mark.parametrize("kind", ["normal", "ties", "specials"])
def test_topk_on_given_logits_is_bit_exact(E, k, renorm, kind):
    from grouped_expert_ffn_amd import make_desc, moe_route, to_device
    t = T_()
    T = 37
    lg = logits_case(kind, T, E, seed=E * 100 + k)
    desc = make_desc(64, E, k, 64, renormalize=renorm)
    ids = t.empty((T, k), dtype=t.int32, device="cuda")
    w = t.empty((T, k), dtype=t.float32, device="cuda")
    lin = to_device(lg)
    moe_route(desc, T, None, None, None, lin, None, ids, w)
    t.cuda.synchronize()
    ref_ids, ref_w = O.route(lg.astype(np.float64), k, renorm)
    np.testing.assert_array_equal(ids.cpu().numpy(), ref_ids)
    finite = np.nonzero(np.all(np.isfinite(lg), axis=1))[0]
    C.assert_gate_weights(w.cpu().numpy(), ref_w, lg, E, renorm, k, rows=finite)


# ----------------------------------------------------------------------------------------
# step 1: router GEMM
# ----------------------------------------------------------------------------------------
# a bf16 router whose expert count is not a multiple of the 16-expert MFMA tile
ROUTER_E40 = S.Workload("router_e40", 94, d=320, E=40, k=4, I=32, renormalize=True,
                        routing="zipf", router_std=320 ** -0.5, zipf_alpha=1.2, tokens=(77,))
ROUTE_CASES = [(S.TINY_F32, 16), (S.OLMOE_BF16, 1), (S.OLMOE_BF16, 64), (S.OLMOE_BF16, 65),
               (S.DEEPSEEK_BF16, 2048), (ROUTER_E40, 77), (ROUTER_E40, 1000)]


@pytest.mark.parametrize("wl,T", ROUTE_CASES, ids=lambda v: getattr(v, "name", str(v)))
def test_router_logits_and_choice(wl, T):
    from grouped_expert_ffn_amd import from_device, moe_route, to_device
    t = T_()
    gl = C.GpuLayer(wl)
    x = S.make_tokens(wl, T)
    xd = to_device(x)
    lg = t.empty((T, wl.E), dtype=t.float32, device="cuda")
    ids = t.empty((T, wl.k), dtype=t.int32, device="cuda")
    w = t.empty((T, wl.k), dtype=t.float32, device="cuda")
    moe_route(gl.desc, T, xd, gl.dev.w_router, gl.dev.bias, None, lg, ids, w)
    t.cuda.synchronize()
    ref = O.router_logits(x, gl.host.w_router, gl.host.bias)
    got = lg.cpu().numpy()
    assert C.rel_l2(got, ref) <= 1e-5
    # the choice on the GPU's own fp32 logits is the oracle's, bit for bit
    ids_g = ids.cpu().numpy()
    ref_ids, ref_w = O.route(got.astype(np.float64), wl.k, wl.renormalize)
    np.testing.assert_array_equal(ids_g, ref_ids)
    C.assert_gate_weights(w.cpu().numpy(), ref_w, got, wl.E, wl.renormalize, wl.k)
    # against fp64 logits, only pre-registered near-ties may differ
    C.check_routing_against_oracle(ids_g, ref, wl.k)


# ----------------------------------------------------------------------------------------
# step 2: permutation is bit-exact
# ----------------------------------------------------------------------------------------
def ids_case(kind, T, E, k, seed):
    g = np.random.default_rng(seed)
    if kind == "uniform":
        return np.stack([g.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    if kind == "same":  # every token picks the same k experts
        return np.tile(np.arange(k, dtype=np.int32)[::-1], (T, 1))
    if kind == "zipf":
        p = 1.0 / np.arange(1, E + 1) ** 1.2
        p /= p.sum()
        return np.stack([g.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    raise ValueError(kind)


# T*k up to 64 takes the one-wavefront sort (1-64 rows, up to 256 experts and 8 shared),
# beyond the workgroup sort, past 4096 rows the chunked one (chunks of 1024 rows: up to 64
# chunks the sort blocks sum their own bases, 65528 rows at T=8191; beyond, a scan launch
# does, 65600 rows at T=8200)
@pytest.mark.parametrize("T,E,k,S_", [(1, 8, 2, 0), (16, 8, 2, 0), (1, 64, 8, 0), (8, 64, 8, 0),
                                      (10, 64, 6, 2), (64, 8, 1, 0), (9, 256, 7, 8), (37, 64, 6, 2),
                                      (64, 64, 8, 0), (300, 256, 16, 1), (2048, 64, 8, 0),
                                      (2048, 64, 6, 2), (1000, 3, 1, 0), (513, 64, 8, 8),
                                      (2100, 64, 8, 0), (8191, 64, 8, 0), (8200, 64, 8, 2)])
@pytest.mark.parametrize("kind", ["uniform", "same", "zipf"])
def test_permute_is_bit_exact(T, E, k, S_, kind):
    _permute_case(T, E, k, S_, kind, d=64)


# layers whose FFN at these sizes is the GEMM, so the plan carries its M-tile list (d = 48 is
# not a multiple of the matrix-core GEMV's 64): one-wavefront sort (40 and 64 rows) and
# workgroup sort (65 rows)
@pytest.mark.parametrize("T,E,k,S_", [(40, 8, 1, 1), (32, 4, 2, 2), (65, 8, 1, 0)])
@pytest.mark.parametrize("kind", ["uniform", "zipf"])
def test_permute_tile_list_is_bit_exact(T, E, k, S_, kind):
    from grouped_expert_ffn_amd import abi, make_desc
    assert abi.moe_ffn_kernel(make_desc(48, E, k, 48, n_shared=S_), T) == abi.MOE_FFN_GEMM
    _permute_case(T, E, k, S_, kind, d=48)


def _permute_case(T, E, k, S_, kind, d):
    from grouped_expert_ffn_amd import (MOE_WS_PERMUTE, alloc_workspace, make_desc, moe_permute,
                                        moe_workspace_bytes, to_device)
    t = T_()
    ids = ids_case(kind, T, E, k, seed=T + E + k)
    desc = make_desc(d, E, k, d, n_shared=S_)
    dev = "cuda"
    counts = t.full((E,), -7, dtype=t.int32, device=dev)
    offsets = t.full((E + S_ + 1,), -7, dtype=t.int32, device=dev)
    perm = t.full((T * k,), -7, dtype=t.int32, device=dev)
    inv = t.full((T * k,), -7, dtype=t.int32, device=dev)
    pb = moe_workspace_bytes(desc, T, MOE_WS_PERMUTE)
    plan = alloc_workspace(pb)
    moe_permute(desc, T, to_device(ids), counts, offsets, perm, inv, plan, pb)
    t.cuda.synchronize()
    c_ref, o_ref, p_ref, i_ref = O.permute(ids, E)
    np.testing.assert_array_equal(counts.cpu().numpy(), c_ref)
    o_full = np.concatenate([o_ref, T * k + T * np.arange(1, S_ + 1)])
    np.testing.assert_array_equal(offsets.cpu().numpy(), o_full)
    np.testing.assert_array_equal(perm.cpu().numpy(), p_ref)
    np.testing.assert_array_equal(inv.cpu().numpy(), i_ref)
    # plan: touched groups ascending, then the shared ones; M-tiles cover every row once
    pl = plan.view(t.int32).cpu().numpy()
    touched = [e for e in range(E) if c_ref[e] > 0] + [E + s for s in range(S_)]
    assert pl[0] == len(touched)
    assert pl[4:4 + len(touched)].tolist() == touched
    tm = pl[2]
    if tm > 0:
        tiles = pl[4 + E + S_: 4 + E + S_ + 2 * pl[1]].reshape(-1, 2)
        expect = [(g, m0) for g in touched for m0 in range(0, c_ref[g] if g < E else T, tm)]
        assert [tuple(x) for x in tiles.tolist()] == expect
    else:
        assert d == 64


# ----------------------------------------------------------------------------------------
# steps 3-5 and the whole layer
# ----------------------------------------------------------------------------------------
# a small bf16 layer whose MFMA tiles have ragged edges in every dimension: d not a
# multiple of the 64-wide K step, I not a multiple of the 64-channel N tile, groups not
# multiples of the 128-row M tile
SMALL_RAGGED = S.Workload("small_ragged", 90, d=272, E=8, k=2, I=208, S=1, renormalize=True,
                          tokens=(100,))
SMALL_RAGGED_I8 = dataclasses.replace(SMALL_RAGGED, name="small_ragged_i8", cid=91, wdt="i8")
SMALL_ZIPF = dataclasses.replace(SMALL_RAGGED, name="small_zipf", cid=92, routing="zipf",
                                 zipf_alpha=2.0, router_std=0.05, tokens=(300,))
# bf16 layer on the LDS-ring MFMA path (d and I multiples of 32) whose N-tiles are ragged in
# both GEMMs (I=352 is not a multiple of 128 channels, d=288 not of 256)
SMALL_RING = S.Workload("small_ring", 93, d=288, E=8, k=2, I=352, S=1, renormalize=True,
                        tokens=(300,))
# the same with d and I multiples of 64 (the full-line weight-block ring), N-tiles ragged in
# both GEMMs (I=448 is 3.5 gate/up tiles of 128 channels, d=320 is 1.25 down tiles of 256)
SMALL_RING64 = S.Workload("small_ring64", 99, d=320, E=8, k=2, I=448, S=1, renormalize=True,
                          tokens=(300,))
# int8 weights on both ring kernels: the 32-deep ring serves K % 64 == 32 (SMALL_RING's
# d=288 and I=352), the 64-deep blocks K % 64 == 0
SMALL_RING_I8 = dataclasses.replace(SMALL_RING, name="small_ring_i8", cid=88, wdt="i8")
SMALL_RING64_I8 = dataclasses.replace(SMALL_RING64, name="small_ring64_i8", cid=89, wdt="i8")

# the matrix-core GEMV (bf16 activations, d and I multiples of 64): routed experts only under
# Zipf routing, so the busiest groups span two 16-token chunks (T=32: 64 rows over 8 experts);
# T=12 is the last size on the VALU GEMV (mean 3 rows per group), T=13 the first on this one
SMALL_MFV = S.Workload("small_mfv", 86, d=320, E=8, k=2, I=448, S=0, renormalize=True,
                       routing="zipf", zipf_alpha=2.0, router_std=0.05, tokens=(32,))
SMALL_MFV_I8 = dataclasses.replace(SMALL_MFV, name="small_mfv_i8", cid=85, wdt="i8")

# the limits of the descriptor: 256 experts, top-16, 8 shared experts, and the smallest
# dimensions (d = I = 16; neither a multiple of the 32-wide K step of the ring GEMM)
EDGE_MAX = S.Workload("edge_max", 95, d=48, E=256, k=16, I=48, S=8, renormalize=True,
                      tokens=(40,))
EDGE_MIN = S.Workload("edge_min", 96, d=16, E=3, k=1, I=16, S=1, tokens=(40,))

FULL_CASES = [  # every row checked
    (EDGE_MAX, 4), (EDGE_MAX, 40), (EDGE_MIN, 5), (EDGE_MIN, 40), (S.TINY_F32, 200),
    (S.TINY_F32, 16), (SMALL_RAGGED, 100), (SMALL_RAGGED, 7), (SMALL_RAGGED_I8, 100),
    (SMALL_RAGGED_I8, 5), (SMALL_ZIPF, 300), (SMALL_RING, 300), (SMALL_RING, 40),
    (SMALL_RING64, 300), (SMALL_RING64, 40), (SMALL_RING_I8, 300), (SMALL_RING64_I8, 300),
    (S.OLMOE_BF16, 1), (S.OLMOE_BF16, 8),
    # speculative-decode verify batches (draft length + 1 tokens), both on the VALU GEMV
    (S.OLMOE_BF16, 3), (S.OLMOE_BF16, 9),
    (S.OLMOE_I8, 1), (S.OLMOE_I8, 8), (S.DEEPSEEK_BF16, 1), (S.OLMOE_I8_ZIPF, 8),
    # the matrix-core GEMV: ragged Zipf groups (bf16 and int8), its lower edge, and with a
    # shared expert (T = 8-16; the shared group is one full chunk at T=16)
    (SMALL_MFV, 32), (SMALL_MFV, 13), (SMALL_MFV, 12), (SMALL_MFV_I8, 24), (SMALL_RING64, 12),
    (SMALL_RING64_I8, 16),
]
SAMPLED_CASES = [  # rows sampled (tile edges, segment ends, random)
    (S.OLMOE_BF16, 64), (S.OLMOE_I8, 64), (S.OLMOE_I8_ZIPF, 64), (S.DEEPSEEK_BF16, 16),
    (S.DEEPSEEK_BF16, 128), (S.DEEPSEEK_BF16, 512), (S.DEEPSEEK_BF16, 2048), (S.DEEPSEEK_I8, 16),
    (S.DEEPSEEK_I8, 512),
    # the tuned tile widths (bf16: gate/up 128 at T = 17-48, down 128 at T = 64-128; int8:
    # gate/up 128 at T = 25-32, down 128 at T = 9-512): bf16 gate/up 128 + down 256, gate/up
    # 256 + down 128, both 256; int8 gate/up 256 + down 128, both 128
    (S.DEEPSEEK_BF16, 40), (S.DEEPSEEK_BF16, 100), (S.DEEPSEEK_BF16, 450), (S.DEEPSEEK_I8, 24),
    (S.DEEPSEEK_I8, 30), (S.DEEPSEEK_I8, 100),
    # the VALU GEMV at its largest sizes (routed experts only: groups of several 4-row chunks)
    (S.OLMOE_BF16, 24), (S.OLMOE_I8, 16),
    # the matrix-core GEMV on the production shapes (OLMoE bf16 T = 25-64, int8 17-48;
    # DeepSeek T = 8-16; OLMOE_BF16 64 and DEEPSEEK 16 above)
    (S.OLMOE_BF16, 32), (S.OLMOE_I8, 48), (S.OLMOE_I8_ZIPF, 24), (S.DEEPSEEK_BF16, 8),
    (S.DEEPSEEK_BF16, 9), (S.DEEPSEEK_BF16, 12), (S.DEEPSEEK_I8, 8),
    # the sweep's largest points on the other shapes (64-deep weight blocks, bf16 and int8)
    (S.OLMOE_BF16, 2048), (S.OLMOE_I8, 2048), (S.DEEPSEEK_I8, 2048),
]


def case_id(v):
    return getattr(v, "name", str(v))


def _steps_and_check(wl, T, sampled):
    from grouped_expert_ffn_amd import to_device
    gl = C.GpuLayer(wl)
    x = S.make_tokens(wl, T)
    out = C.run_steps(gl, to_device(x), T)
    ids = out["ids"].cpu().numpy()
    counts = out["counts"].cpu().numpy()
    offsets = out["offsets"].cpu().numpy()
    perm = out["perm"].cpu().numpy()
    inv = out["inv_perm"].cpu().numpy()
    # permutation of the GPU's own routing is the oracle's, bit for bit
    c_ref, o_ref, p_ref, i_ref = O.permute(ids, wl.E)
    np.testing.assert_array_equal(counts, c_ref)
    np.testing.assert_array_equal(offsets[:wl.E + 1], o_ref)
    np.testing.assert_array_equal(perm, p_ref)
    np.testing.assert_array_equal(inv, i_ref)
    R = T * wl.k + wl.S * T
    rows_g = C.widen_dev(out["rows"])
    if sampled:
        sel = C.sample_rows(offsets, wl.E + wl.S, R, n_random=24)
    else:
        sel = list(range(R))
    rows_ref = C.oracle_sorted_rows(x, gl.experts, ids, perm, wl.S, wl.E, sel)
    C.assert_close(rows_g[sel], rows_ref, wl.act, f"{wl.name} T={T} grouped FFN rows")
    # combine of the GPU's rows: only the final rounding of y differs from fp64
    w_g = out["w"].cpu().numpy().astype(np.float64)
    y_g = C.widen_dev(out["y"])
    tok = sorted(set(range(T)) if not sampled else set(range(0, T, max(1, T // 24))) | {T - 1})
    from grouped_expert_ffn_amd import from_device
    rows_stored = from_device(out["rows"])
    y_ref = O.combine(rows_stored, inv, w_g, wl.S)
    tol = 2.0 ** -8 if wl.act == "bf16" else 1e-6
    np.testing.assert_allclose(y_g, y_ref, rtol=tol, atol=tol * np.max(np.abs(y_ref)))
    # the layer end to end, the oracle using the GPU's expert choice
    logits_ref = O.router_logits(x, gl.host.w_router, gl.host.bias)
    C.check_routing_against_oracle(ids, logits_ref, wl.k)
    w_ref = O.gate_weights_for(logits_ref, ids, wl.renormalize)
    y_full = C.oracle_layer(x, gl.experts, ids, w_ref, wl.S, wl.E, tok)
    C.assert_close(y_g[tok], y_full, wl.act, f"{wl.name} T={T} layer output")


@pytest.mark.parametrize("wl,T", FULL_CASES, ids=case_id)
def test_steps_full(wl, T):
    _steps_and_check(wl, T, sampled=False)


@pytest.mark.parametrize("wl,T", SAMPLED_CASES, ids=case_id)
def test_steps_sampled(wl, T):
    _steps_and_check(wl, T, sampled=True)


# Every row of the grouped FFN and every token of the layer at the largest prefill size
# of the DeepSeek-shaped workload (64-deep weight-block ring GEMM, 2 shared experts, Zipf load)
@pytest.mark.timeout(900)
def test_steps_every_row_deepseek_2048():
    _steps_and_check(S.DEEPSEEK_BF16, 2048, sampled=False)


# moe_forward against the five step-by-step calls, bit for bit, at decode and prefill sizes
# (the forward fuses the top-k into the sort; the steps sort given ids: up to 64 rows both
# with the one-wavefront sort, from 65 rows with the workgroup sort)
TINY_F32_SHARED = dataclasses.replace(S.TINY_F32, name="tiny_f32_shared", cid=83, S=1)
FORWARD_CASES = [
    (S.TINY_F32, 16), (SMALL_RAGGED, 100), (S.OLMOE_BF16, 8), (S.OLMOE_BF16, 1), (S.OLMOE_BF16, 2),
    (S.OLMOE_BF16, 9), (S.DEEPSEEK_BF16, 4), (S.DEEPSEEK_BF16, 1), (S.DEEPSEEK_BF16, 7),
    (S.DEEPSEEK_BF16, 8), (S.DEEPSEEK_I8, 3), (S.OLMOE_I8, 8), (S.OLMOE_I8, 1), (S.TINY_F32, 5),
    (TINY_F32_SHARED, 8), (TINY_F32_SHARED, 9), (SMALL_RAGGED, 7), (SMALL_RAGGED_I8, 5),
    (EDGE_MIN, 5), (EDGE_MAX, 4), (EDGE_MAX, 5), (SMALL_RING64, 8), (S.DEEPSEEK_BF16, 512),
    (S.OLMOE_I8, 64)]


@pytest.mark.parametrize("wl,T", FORWARD_CASES, ids=case_id)
def test_forward_matches_steps_and_is_deterministic(wl, T):
    from grouped_expert_ffn_amd import to_device
    t = T_()
    gl = C.GpuLayer(wl)
    x = S.make_tokens(wl, T)
    xd = to_device(x)
    steps = C.run_steps(gl, xd, T)
    ids = t.empty((T, wl.k), dtype=t.int32, device="cuda")
    w = t.empty((T, wl.k), dtype=t.float32, device="cuda")
    y1 = gl.dev.forward(xd, topk_ids=ids, topk_w=w)
    y2 = gl.dev.forward(xd)
    t.cuda.synchronize()
    assert t.equal(y1.view(t.int16) if y1.dtype == t.bfloat16 else y1,
                   y2.view(t.int16) if y2.dtype == t.bfloat16 else y2)
    assert t.equal(ids, steps["ids"]) and t.equal(w, steps["w"])
    assert t.equal(y1, steps["y"])


# moe_forward with a residual and a capacity limit against the separate calls, bit for bit.
# At decode sizes (OLMoE shapes through T=9, DeepSeek shapes through T=6) the forward sums a
# token's rows inside the down projection's launch; T=64 and T=7 take the two launches.
RESID_CASES = [(S.OLMOE_BF16, 1, 0.0), (S.OLMOE_BF16, 8, 1.0), (S.OLMOE_BF16, 9, 0.0),
               (S.DEEPSEEK_BF16, 5, 0.0), (S.DEEPSEEK_BF16, 6, 0.5), (S.DEEPSEEK_I8, 3, 0.5),
               (S.OLMOE_I8, 2, 0.0), (TINY_F32_SHARED, 9, 0.0), (S.TINY_F32, 3, 1.0),
               (SMALL_RAGGED_I8, 5, 0.5), (EDGE_MAX, 5, 0.0), (S.DEEPSEEK_BF16, 7, 0.0),
               (S.OLMOE_BF16, 64, 0.0)]


@pytest.mark.parametrize("wl,T,cf", RESID_CASES, ids=case_id)
def test_forward_with_residual_and_capacity_matches_steps(wl, T, cf):
    from grouped_expert_ffn_amd import DTYPES, DeviceLayer, make_desc, to_device
    t = T_()
    gl = C.GpuLayer(wl)
    desc = make_desc(wl.d, wl.E, wl.k, wl.I, wl.S, wl.renormalize, DTYPES[wl.act], DTYPES[wl.wdt],
                     capacity_factor=cf)
    dl = DeviceLayer(desc, gl.dev.w_router, gl.dev.bias, gl.dev.w_gate, gl.dev.w_up, gl.dev.w_down,
                     gl.dev.s_gate, gl.dev.s_up, gl.dev.s_down)
    xd = to_device(S.make_tokens(wl, T))
    res = to_device(S.make_tokens(wl, T, seed=11))
    y = dl.forward(xd, residual=res)
    steps = C.run_steps(gl, xd, T, desc=desc, residual=res)
    t.cuda.synchronize()
    if cf and cf <= 0.5:
        assert (steps["inv_perm"] < 0).any(), "the case is meant to drop rows"
    assert t.equal(y, steps["y"])


@pytest.mark.parametrize("T", [4, 16])  # the decode GEMV and the prefill GEMM
def test_forward_residual_and_power_of_two_scaling(T):
    from grouped_expert_ffn_amd import DeviceLayer, to_device
    t = T_()
    wl = S.DEEPSEEK_BF16
    gl = C.GpuLayer(wl)
    xd = to_device(S.make_tokens(wl, T))
    y = gl.dev.forward(xd)
    d2 = DeviceLayer(gl.desc, gl.dev.w_router, gl.dev.bias, gl.dev.w_gate, gl.dev.w_up,
                     gl.dev.w_down * 2)
    y2 = d2.forward(xd)
    t.cuda.synchronize()
    assert t.equal(y2, y * 2), "doubling W_down (routed and shared) must double y exactly"
    res = to_device(S.make_tokens(wl, T, seed=5))
    yr = gl.dev.forward(xd, residual=res)
    t.cuda.synchronize()
    got = C.widen_dev(yr)
    exp = C.widen_dev(y).astype(np.float64) + C.widen_dev(res)
    np.testing.assert_allclose(got, exp, rtol=2.0 ** -7, atol=2.0 ** -7 * np.max(np.abs(exp)))


def test_identical_experts_make_output_independent_of_routing():
    from grouped_expert_ffn_amd import DeviceLayer, to_device
    t = T_()
    wl = dataclasses.replace(SMALL_RAGGED, S=0)
    h = S.make_layer(wl)
    rep = lambda a: np.repeat(a[:1], wl.E, axis=0)  # noqa: E731
    outs = []
    for seed in (1, 2):
        wr = S.make_layer(dataclasses.replace(wl, cid=200 + seed)).w_router
        dl = DeviceLayer(C.desc_of(wl), wr, None, rep(h.w_gate), rep(h.w_up), rep(h.w_down))
        outs.append(C.widen_dev(dl.forward(to_device(S.make_tokens(wl, 100)))))
    x = S.make_tokens(wl, 100)
    one = O.Experts(h.w_gate[:1], h.w_up[:1], h.w_down[:1])
    ref = O.moe_layer(x, one, np.zeros((100, 1), dtype=np.int64), np.ones((100, 1)), 0, 1)
    for y in outs:
        C.assert_close(y, ref, "bf16", "identical experts")


# ----------------------------------------------------------------------------------------
# the 16-layer prefill stack, checked layer by layer (each layer's oracle is fed the GPU's
# bf16 input of that layer)
# ----------------------------------------------------------------------------------------
@pytest.mark.timeout(600)
def test_stack_staged_per_layer():
    from grouped_expert_ffn_amd import DeviceLayer, to_device
    t = T_()
    wl = S.OLMOE_STACK16
    T = wl.tokens[0]
    h = to_device(S.make_tokens(wl, T))
    ids = t.empty((T, wl.k), dtype=t.int32, device="cuda")
    tok = list(range(0, T, 97)) + [T - 1]
    skews = []
    flips = 0
    # unstaged: the oracle's own fp64 residual stream for the sampled tokens, routed by the
    # oracle's own choices through all 16 layers (reported, not gated: near-tied routing
    # choices may differ from the GPU's and then the streams part)
    h_o = O.widen(S.make_tokens(wl, T)[tok])
    for layer in range(wl.n_layers):
        host = S.make_layer(wl, layer)
        dl = DeviceLayer(C.desc_of(wl), host.w_router, host.bias, host.w_gate, host.w_up, host.w_down)
        h_in = C.widen_dev(h)
        h_next = dl.forward(h, residual=h, topk_ids=ids)
        t.cuda.synchronize()
        ids_g = ids.cpu().numpy()
        counts = np.bincount(ids_g.ravel(), minlength=wl.E)
        skews.append(counts.max() / (T * wl.k / wl.E))
        from grouped_expert_ffn_amd import from_device
        h_in_bits = from_device(h)
        xn = O.stack_layer_input(h_in_bits[tok], wl.norm_eps)
        logits = O.router_logits(xn, host.w_router, host.bias)
        flips += C.check_routing_against_oracle(ids_g[tok], logits, wl.k, C.TIE_DELTA_STACK)
        w_ref = O.gate_weights_for(logits, ids_g[tok], wl.renormalize)
        ex = O.Experts.from_layer(host)
        y = O.moe_layer(xn, ex, ids_g[tok], w_ref, 0, wl.E, residual=h_in[tok])
        C.assert_close(C.widen_dev(h_next)[tok], y, "bf16", f"stack layer {layer}")
        xo = O.rmsnorm(h_o, wl.norm_eps)
        _, ids_o, w_o = O.full_route(xo, host.w_router, host.bias, wl.k, wl.renormalize)
        h_o = h_o + O.moe_layer(xo, ex, ids_o, w_o, 0, wl.E)
        h = h_next
        del dl, host, ex
    print(f"stack: busiest/mean per layer {[round(float(s), 2) for s in skews]}, tie flips {flips}")
    h_gpu = C.widen_dev(h)[tok]
    print(f"stack unstaged after {wl.n_layers} layers: rel-L2 {C.rel_l2(h_gpu, h_o):.3e} "
          f"(max-abs {float(np.max(np.abs(h_gpu - h_o))):.3e}, max |h| {float(np.max(np.abs(h_o))):.3e})")
    # the tuned skew holds on layer 0 (later layers drift)
    assert 3.9 <= skews[0] <= 4.1, skews


# One full layer of the stack, every token: RMSNorm prologue, Zipf routing with the busiest
# expert at about four times the mean, residual epilogue, at T = 2048
@pytest.mark.timeout(900)
def test_stack_layer_every_token():
    from grouped_expert_ffn_amd import DeviceLayer, from_device, to_device
    t = T_()
    wl = S.OLMOE_STACK16
    T = wl.tokens[0]
    layer = 3
    x_bits = S.make_tokens(wl, T, layer=layer)
    host = S.make_layer(wl, layer)
    dl = DeviceLayer(C.desc_of(wl), host.w_router, host.bias, host.w_gate, host.w_up, host.w_down)
    h = to_device(x_bits)
    ids = t.empty((T, wl.k), dtype=t.int32, device="cuda")
    y = dl.forward(h, residual=h, topk_ids=ids)
    t.cuda.synchronize()
    ids_g = ids.cpu().numpy()
    xn = O.stack_layer_input(x_bits, wl.norm_eps)
    logits = O.router_logits(xn, host.w_router, host.bias)
    C.check_routing_against_oracle(ids_g, logits, wl.k, C.TIE_DELTA_STACK)
    w_ref = O.gate_weights_for(logits, ids_g, wl.renormalize)
    ref = C.oracle_layer(xn, O.Experts.from_layer(host), ids_g, w_ref, 0, wl.E, range(T),
                         residual=O.widen(x_bits))
    C.assert_close(C.widen_dev(y), ref, "bf16", f"stack layer {layer}, every token")


# RMSNorm prologue at every register width of its kernel (1, 2, 4, 8 and 16 chunks of 16
# bytes per thread, whole and with a partial last round) for both activation types
PRE_NORM_CASES = [("bf16", 48), ("bf16", 4096), ("bf16", 6144), ("bf16", 16384),
                  ("f32", 48), ("f32", 2048), ("f32", 12288), ("f32", 16384)]


@pytest.mark.parametrize("act,d", PRE_NORM_CASES, ids=[f"{a}-d{d}" for a, d in PRE_NORM_CASES])
def test_forward_pre_norm_widths(act, d):
    from grouped_expert_ffn_amd import DeviceLayer, to_device
    t = T_()
    T = 6
    wl = S.Workload(f"pre_norm_{act}_{d}", 97, d=d, E=4, k=2, I=16, act=act, wdt=act,
                    pre_norm=True, tokens=(T,))
    host = S.make_layer(wl, 0)
    dl = DeviceLayer(C.desc_of(wl), host.w_router, host.bias, host.w_gate, host.w_up, host.w_down)
    x_host = S.make_tokens(wl, T)
    ids = t.empty((T, wl.k), dtype=t.int32, device="cuda")
    y = dl.forward(to_device(x_host), topk_ids=ids)
    t.cuda.synchronize()
    if act == "bf16":
        xn, delta = O.stack_layer_input(x_host, wl.norm_eps), C.TIE_DELTA_STACK
    else:
        xn, delta = O.rmsnorm(x_host, wl.norm_eps), C.TIE_DELTA
    logits = O.router_logits(xn, host.w_router, host.bias)
    ids_g = ids.cpu().numpy()
    C.check_routing_against_oracle(ids_g, logits, wl.k, delta)
    w_ref = O.gate_weights_for(logits, ids_g, wl.renormalize)
    ref = O.moe_layer(xn, O.Experts.from_layer(host), ids_g, w_ref, 0, wl.E)
    C.assert_close(C.widen_dev(y), ref, act, f"pre_norm {act} d={d}")


# ----------------------------------------------------------------------------------------
# option: capacity-factor dropping
# ----------------------------------------------------------------------------------------
@pytest.mark.parametrize("T,E,k,S_", [(16, 8, 2, 0), (300, 8, 2, 1), (1000, 64, 6, 2),
                                      (2048, 64, 8, 0), (2100, 64, 6, 2)])
@pytest.mark.parametrize("cf", [0.5, 1.0, 2.0])
def test_permute_with_capacity_is_bit_exact(T, E, k, S_, cf):
    from grouped_expert_ffn_amd import (MOE_WS_PERMUTE, alloc_workspace, make_desc, moe_permute,
                                        moe_workspace_bytes, to_device)
    t = T_()
    ids = ids_case("zipf", T, E, k, seed=T + E + k + 7)
    desc = make_desc(64, E, k, 64, n_shared=S_, capacity_factor=cf)
    counts = t.full((E,), -7, dtype=t.int32, device="cuda")
    offsets = t.full((E + S_ + 1,), -7, dtype=t.int32, device="cuda")
    perm = t.full((T * k,), -7, dtype=t.int32, device="cuda")
    inv = t.full((T * k,), -7, dtype=t.int32, device="cuda")
    pb = moe_workspace_bytes(desc, T, MOE_WS_PERMUTE)
    plan = alloc_workspace(pb)
    moe_permute(desc, T, to_device(ids), counts, offsets, perm, inv, plan, pb)
    t.cuda.synchronize()
    cap = O.capacity(cf, T, k, E)
    c_ref, o_ref, p_ref, i_ref = O.permute_with_capacity(ids, E, cap)
    np.testing.assert_array_equal(counts.cpu().numpy(), c_ref)
    np.testing.assert_array_equal(offsets.cpu().numpy()[:E + 1], o_ref)
    np.testing.assert_array_equal(perm.cpu().numpy(), p_ref)
    np.testing.assert_array_equal(inv.cpu().numpy(), i_ref)
    assert (i_ref < 0).any() or cf == 2.0
    pl = plan.view(t.int32).cpu().numpy()
    assert pl[3] == min(cap, T)
    tm = pl[2]
    if tm > 0:
        touched = [e for e in range(E) if c_ref[e] > 0] + [E + s for s in range(S_)]
        rows = {g: (min(c_ref[g], cap) if g < E else T) for g in touched}
        tiles = pl[4 + E + S_: 4 + E + S_ + 2 * pl[1]].reshape(-1, 2)
        assert [tuple(x) for x in tiles.tolist()] == [(g, m0) for g in touched
                                                      for m0 in range(0, rows[g], tm)]


CAP_CASES = [(SMALL_ZIPF, 300, 1.0), (SMALL_RING, 300, 1.0), (SMALL_RING, 40, 0.5),
             (S.OLMOE_BF16, 8, 1.0), (S.OLMOE_I8_ZIPF, 8, 1.0), (S.DEEPSEEK_BF16, 2048, 1.0),
             (S.DEEPSEEK_BF16, 16, 2.0), (SMALL_MFV, 32, 1.0), (S.DEEPSEEK_BF16, 6, 0.5),
             (SMALL_ZIPF, 8, 0.5)]


@pytest.mark.parametrize("wl,T,cf", CAP_CASES, ids=case_id)
def test_forward_with_capacity(wl, T, cf):
    from grouped_expert_ffn_amd import DeviceLayer, make_desc, to_device, DTYPES
    t = T_()
    gl = C.GpuLayer(wl)
    desc = make_desc(wl.d, wl.E, wl.k, wl.I, wl.S, wl.renormalize, DTYPES[wl.act], DTYPES[wl.wdt],
                     capacity_factor=cf)
    dl = DeviceLayer(desc, gl.dev.w_router, gl.dev.bias, gl.dev.w_gate, gl.dev.w_up, gl.dev.w_down,
                     gl.dev.s_gate, gl.dev.s_up, gl.dev.s_down)
    x = S.make_tokens(wl, T)
    ids = t.empty((T, wl.k), dtype=t.int32, device="cuda")
    y = dl.forward(to_device(x), topk_ids=ids)
    t.cuda.synchronize()
    ids_g = ids.cpu().numpy()
    cap = O.capacity(cf, T, wl.k, wl.E)
    keep = O.kept_slots(ids_g, wl.E, cap)
    if cf <= 1.0:
        assert (~keep).any(), "the case is meant to drop rows"
    logits = O.router_logits(x, gl.host.w_router, gl.host.bias)
    C.check_routing_against_oracle(ids_g, logits, wl.k)
    w_ref = O.gate_weights_for(logits, ids_g, wl.renormalize)
    tok = list(range(T)) if T <= 300 else sorted(set(range(0, T, 97)) | {T - 1})
    y_ref = O.moe_layer(x, gl.experts, ids_g, w_ref, wl.S, wl.E, tokens=tok, keep=keep)
    C.assert_close(C.widen_dev(y)[tok], y_ref, wl.act, f"{wl.name} T={T} cf={cf}")


# ----------------------------------------------------------------------------------------
# the layer captured in a HIP graph: every replay equals the eager result bit for bit
# ----------------------------------------------------------------------------------------
@pytest.mark.parametrize("wl,T", [(S.OLMOE_BF16, 8), (SMALL_RING, 300), (S.DEEPSEEK_BF16, 16),
                                  (S.DEEPSEEK_BF16, 4)],
                         ids=case_id)
def test_forward_graph_replay_matches_eager(wl, T):
    from grouped_expert_ffn_amd import abi, to_device
    t = T_()
    gl = C.GpuLayer(wl)
    x = to_device(S.make_tokens(wl, T))
    x_other = to_device(S.make_tokens(wl, T, seed=5))
    y_eager = gl.dev.forward(x)
    t.cuda.synchronize()
    ws = gl.dev.workspace(T)
    y_graph = t.empty_like(y_eager)
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        abi.moe_forward(gl.desc, T, x, gl.dev.w_router, gl.dev.bias, gl.dev.weights, None, y_graph,
                        None, None, ws, ws.numel())
    for _ in range(4):
        y_graph.zero_()
        t.cuda.synchronize()
        g.replay()
        t.cuda.synchronize()
        assert t.equal(y_graph, y_eager)
        gl.dev.forward(x_other)  # eager work on the same workspace between replays
        t.cuda.synchronize()
    del g


# Several forwards in one graph, alternating two weight copies and two token batches over one
# shared workspace (the form bench.py times): every output equals its eager result bit for bit
# on each replay.
@pytest.mark.parametrize("wl,T", [(S.OLMOE_BF16, 8), (S.OLMOE_BF16, 1), (S.DEEPSEEK_BF16, 300)],
                         ids=case_id)
def test_graph_of_several_forwards_matches_eager(wl, T):
    from grouped_expert_ffn_amd import DeviceLayer, abi, to_device
    t = T_()
    gl = C.GpuLayer(wl)
    d = gl.dev
    twin = DeviceLayer(gl.desc, d.w_router, d.bias, d.w_gate.clone(), d.w_up.clone(), d.w_down.clone(),
                       None if d.s_gate is None else d.s_gate.clone(),
                       None if d.s_up is None else d.s_up.clone(),
                       None if d.s_down is None else d.s_down.clone())
    xs = [to_device(S.make_tokens(wl, T, seed=s)) for s in (0, 7)]
    eager = [d.forward(x) for x in xs]
    t.cuda.synchronize()
    ws = d.workspace(T)
    ys = [t.empty_like(e) for e in eager]
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        for i in range(6):
            L = (d, twin)[i % 2]
            abi.moe_forward(gl.desc, T, xs[(i // 2) % 2], L.w_router, L.bias, L.weights, None,
                            ys[(i // 2) % 2], None, None, ws, ws.numel())
    for _ in range(3):
        for y in ys:
            y.zero_()
        t.cuda.synchronize()
        g.replay()
        t.cuda.synchronize()
        for y, e in zip(ys, eager):
            assert t.equal(y, e)
        d.forward(xs[1])  # eager work on the same workspace between replays
        t.cuda.synchronize()
    del g


# In place: y may alias x and the residual may alias either (moe.h).  The same layer run
# out of place and in place gives the same bits, on the fused decode launch (OLMoE T=1, 8,
# DeepSeek T=4), the matrix-core GEMV (OLMoE T=64), the GEMM (DeepSeek T=300) and with the
# RMSNorm prologue.
INPLACE_CASES = [(S.OLMOE_BF16, 1), (S.OLMOE_BF16, 8), (S.DEEPSEEK_BF16, 4), (S.OLMOE_BF16, 64),
                 (S.DEEPSEEK_BF16, 300), (S.OLMOE_I8, 8),
                 (dataclasses.replace(S.OLMOE_BF16, name="olmoe_bf16_prenorm", pre_norm=True), 8)]


@pytest.mark.parametrize("wl,T", INPLACE_CASES, ids=case_id)
def test_forward_in_place_matches_out_of_place(wl, T):
    from grouped_expert_ffn_amd import to_device
    t = T_()
    gl = C.GpuLayer(wl)
    x = to_device(S.make_tokens(wl, T))
    ref = gl.dev.forward(x.clone(), residual=x.clone())
    buf = x.clone()
    out = gl.dev.forward(buf, residual=buf, y=buf)
    t.cuda.synchronize()
    assert out.data_ptr() == buf.data_ptr()
    assert t.equal(buf, ref)
    assert not t.equal(buf, x)  # the layer did write its output over the input


@pytest.mark.parametrize("wl,T", [(S.OLMOE_BF16, 8), (S.DEEPSEEK_BF16, 300), (S.TINY_F32, 16)], ids=case_id)
def test_combine_with_the_residual_in_y(wl, T):
    # moe_combine's residual may be the output buffer itself
    from grouped_expert_ffn_amd import moe_combine, to_device
    t = T_()
    gl = C.GpuLayer(wl)
    xd = to_device(S.make_tokens(wl, T))
    st = C.run_steps(gl, xd, T)
    res = to_device(S.make_tokens(wl, T, seed=9))
    ref = t.empty_like(res)
    moe_combine(gl.desc, T, st["rows"], st["inv_perm"], st["w"], res, ref)
    buf = res.clone()
    moe_combine(gl.desc, T, st["rows"], st["inv_perm"], st["w"], buf, buf)
    t.cuda.synchronize()
    assert t.equal(buf, ref)
