"""Shared helpers of the GPU parity tests: upload seeded layers, run the C-ABI steps, and
compare with the fp64 oracle."""
from __future__ import annotations

import functools
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import moe_synth as S
from oracle import moe_oracle as O

# Output tolerances: relative L2 error (fp32 path 1e-5; bf16 and int8-weight paths 1e-2),
# and max-abs error <= 2e-2 * max|reference|.
REL_L2 = {"f32": 1e-5, "bf16": 1e-2}
MAX_ABS_FRAC = 2e-2
# Pre-registered routing tie margin: a token whose k-th and (k+1)-th oracle logits are
# closer than this may be routed differently by the fp32 GPU router; any other
# difference is a failure.
TIE_DELTA = 1e-4
# In the stacked workload the router input is the bf16-rounded RMSNorm output; the GPU
# normalises in fp32, so one element may round to the neighbouring bf16 value, which moves
# a logit by up to about one bf16 ulp of |x| <= 4 times a router weight (~6e-4).
TIE_DELTA_STACK = 1e-3


def torch():
    import torch as t
    return t


def desc_of(wl: S.Workload):
    from grouped_expert_ffn_amd import DTYPES, make_desc
    return make_desc(wl.d, wl.E, wl.k, wl.I, wl.S, wl.renormalize, DTYPES[wl.act], DTYPES[wl.wdt],
                     wl.pre_norm, wl.norm_eps)


@functools.lru_cache(maxsize=4)
def host_layer(wl: S.Workload, layer: int = 0, seed: int = 0) -> S.Layer:
    return S.make_layer(wl, layer, seed)


class GpuLayer:
    def __init__(self, wl: S.Workload, layer: int = 0, seed: int = 0, host: S.Layer = None):
        from grouped_expert_ffn_amd import DeviceLayer
        self.wl = wl
        self.host = host if host is not None else host_layer(wl, layer, seed)
        h = self.host
        self.desc = desc_of(wl)
        self.dev = DeviceLayer(self.desc, h.w_router, h.bias, h.w_gate, h.w_up, h.w_down,
                               h.s_gate, h.s_up, h.s_down)
        self.experts = O.Experts.from_layer(h)


def rel_l2(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))


def assert_close(got, ref, act: str, what: str):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    r = rel_l2(got, ref)
    m = float(np.max(np.abs(got - ref))) if got.size else 0.0
    lim = MAX_ABS_FRAC * float(np.max(np.abs(ref))) if ref.size else 0.0
    assert r <= REL_L2[act], f"{what}: rel-L2 {r:.3e} > {REL_L2[act]:.0e}"
    assert m <= lim, f"{what}: max-abs {m:.3e} > {lim:.3e}"
    return r, m


def widen_dev(t) -> np.ndarray:
    from grouped_expert_ffn_amd import from_device
    return O.widen(from_device(t))


def check_routing_against_oracle(ids_gpu, logits_ref, k, delta=TIE_DELTA):
    """GPU ids vs the oracle's choice on fp64 logits; returns the number of tie flips.

    A token whose choice differs must have an oracle margin l_(k) - l_(k+1) below
    TIE_DELTA, else the test fails."""
    ids_ref, _ = O.route(logits_ref, k, False)
    flips = 0
    for t in range(ids_ref.shape[0]):
        if list(ids_gpu[t]) != list(ids_ref[t]):
            srt = np.sort(logits_ref[t])[::-1]
            margin = srt[k - 1] - srt[k] if k < len(srt) else np.inf
            # a difference in slot order alone also needs a near-tie among the chosen
            gaps = np.diff(srt[:k + 1])
            tight = margin < delta or (np.min(np.abs(gaps)) < delta if len(gaps) else False)
            assert tight, f"token {t}: GPU {list(ids_gpu[t])} vs oracle {list(ids_ref[t])}, margin {margin:.3e}"
            flips += 1
    return flips


def sample_rows(offsets: np.ndarray, n_groups: int, R: int, n_random: int, seed: int = 0):
    """Rows to check one by one: both ends and tile edges of every group, plus random rows."""
    rows = set()
    for g in range(n_groups):
        a, b = int(offsets[g]), int(offsets[g + 1])
        if b <= a:
            continue
        for r in (a, a + 1, b - 1, b - 2, a + 127, a + 128, a + 255, a + 256):
            if a <= r < b:
                rows.add(r)
    g = np.random.default_rng(seed)
    rows.update(int(r) for r in g.integers(0, R, size=n_random))
    return sorted(rows)


def run_steps(gl: GpuLayer, x_dev, T: int, logits_in=None, desc=None, residual=None):
    """Route, permute, grouped FFN and combine through the separate C-ABI calls (with the
    layer's own descriptor unless `desc` is given, and `residual` added in the combine)."""
    import torch as t
    from grouped_expert_ffn_amd import (MOE_WS_GROUPED_FFN, MOE_WS_PERMUTE, alloc_workspace,
                                        moe_combine, moe_grouped_ffn, moe_permute, moe_route,
                                        moe_workspace_bytes)
    wl, d = gl.wl, (desc if desc is not None else gl.desc)
    dev = x_dev.device
    k, E, S_ = wl.k, wl.E, wl.S
    R = T * k + S_ * T
    out = {}
    out["logits"] = t.empty((T, E), dtype=t.float32, device=dev)
    out["ids"] = t.empty((T, k), dtype=t.int32, device=dev)
    out["w"] = t.empty((T, k), dtype=t.float32, device=dev)
    moe_route(d, T, x_dev, gl.dev.w_router, gl.dev.bias, logits_in, out["logits"], out["ids"], out["w"])
    out["counts"] = t.empty(E, dtype=t.int32, device=dev)
    out["offsets"] = t.empty(E + S_ + 1, dtype=t.int32, device=dev)
    out["perm"] = t.empty(T * k, dtype=t.int32, device=dev)
    out["inv_perm"] = t.empty(T * k, dtype=t.int32, device=dev)
    pb = moe_workspace_bytes(d, T, MOE_WS_PERMUTE)
    out["plan"] = alloc_workspace(pb, dev)
    moe_permute(d, T, out["ids"], out["counts"], out["offsets"], out["perm"], out["inv_perm"],
                out["plan"], pb)
    adt = x_dev.dtype
    out["rows"] = t.empty((R, wl.d), dtype=adt, device=dev)
    wb = moe_workspace_bytes(d, T, MOE_WS_GROUPED_FFN)
    ws = alloc_workspace(wb, dev)
    moe_grouped_ffn(d, T, x_dev, gl.dev.weights, out["offsets"], out["perm"], out["plan"], out["rows"],
                    ws, wb)
    out["y"] = t.empty((T, wl.d), dtype=adt, device=dev)
    moe_combine(d, T, out["rows"], out["inv_perm"], out["w"], residual, out["y"])
    t.cuda.synchronize()
    return out


# ----------------------------------------------------------------------------------------
# the oracle over many rows or tokens: contiguous chunks in threads (NumPy's matrix-vector
# products release the GIL), each chunk an ordinary oracle call
# ----------------------------------------------------------------------------------------
def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _chunks(items, n):
    items = list(items)
    step = max(1, math.ceil(len(items) / n))
    return [items[i:i + step] for i in range(0, len(items), step)]


def oracle_sorted_rows(x, experts, ids, perm, n_shared, n_experts, rows):
    """O.sorted_rows over `rows`, split across threads; returns the expert outputs."""
    parts = _chunks(rows, 4 * _threads())
    with ThreadPoolExecutor(_threads()) as ex:
        outs = list(ex.map(lambda r: O.sorted_rows(x, experts, ids, perm, n_shared, n_experts,
                                                   rows=r)[1], parts))
    return np.concatenate(outs)


def oracle_layer(x, experts, ids, w, n_shared, n_experts, tokens, residual=None):
    """O.moe_layer over `tokens`, split across threads."""
    parts = _chunks(tokens, 4 * _threads())
    with ThreadPoolExecutor(_threads()) as ex:
        outs = list(ex.map(lambda tk: O.moe_layer(x, experts, ids, w, n_shared, n_experts,
                                                  residual=residual, tokens=tk), parts))
    return np.concatenate(outs)


# ----------------------------------------------------------------------------------------
# gate weights: the bound of the GPU's fp32 softmax against the oracle on the same logits
# ----------------------------------------------------------------------------------------
U = 2.0 ** -24  # unit roundoff of fp32


def gate_weight_rtol(logits32: np.ndarray, E: int) -> np.ndarray:
    """Per-token relative bound of a gate weight computed in fp32 as
    expf(l - m) / sum_e expf(l_e - m), against the exact value on the same fp32 logits.

    First-order terms: the subtraction l - m rounds with relative error u, i.e. an absolute
    error |l - m| u in the exponent (at most the token's logit spread s); expf is taken to be
    within 2 ulp (4u); the denominator repeats both for each of its terms and adds the
    rounding of its summation tree (depth 6 over the wavefront, plus 3 sequential additions
    in a lane when E > 64); the division adds u.  Sum:
    (s + 4) u + (s + 4 + depth) u + u = (2 s + 9 + depth) u.  The renormalising division by
    the sum of the k chosen terms has the same form with a shallower tree, so the bound holds
    for it as well."""
    lg = np.asarray(logits32, dtype=np.float64)
    fin = np.where(np.isfinite(lg), lg, np.nan)
    spread = np.nanmax(fin, axis=1) - np.nanmin(fin, axis=1)
    depth = 6 + (3 if E > 64 else 0)
    return (2.0 * spread + 9 + depth) * U


def assert_gate_weights(got_w, ref_w, logits32, E, renorm, k, rows=None):
    """GPU gate weights against the oracle's (computed on the same fp32 logits): within the
    per-token bound above; with renormalisation the k weights of a token sum to 1 within
    k u (each of the k quotients rounds once, the sum of k positive terms at most k - 1 times)."""
    got = np.asarray(got_w, dtype=np.float64)
    ref = np.asarray(ref_w, dtype=np.float64)
    rt = gate_weight_rtol(logits32, E)
    sel = np.arange(got.shape[0]) if rows is None else np.asarray(rows)
    err = np.abs(got[sel] - ref[sel]) / np.abs(ref[sel])
    assert np.all(err <= rt[sel, None]), \
        f"gate weight off by {np.max(err / rt[sel, None]):.2f}x its bound"
    if renorm:
        dev = np.abs(got[sel].sum(1) - 1.0)
        assert np.all(dev <= k * U * (1 + 1e-6)), f"renormalised sum off by {dev.max():.3e}"
