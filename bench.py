#!/usr/bin/env python3
"""Throughput of the MoE dispatch layer on one MI355X.

One step = one ``moe_forward`` (router, top-k, sort, grouped gate/up + SwiGLU,
grouped down, combine) over one batch of seeded synthetic tokens whose weights
and inputs are already resident in HBM.  The headline workload is the
OLMoE-shaped decode layer (d=2048, E=64, k=8, I=1024, bf16) at T=8 tokens.

Before a point is timed its output must be finite and bit-identical over two
runs, and a few of its tokens must agree with the fp64 CPU oracle (routing up
to pre-registered near-ties, outputs within the parity tolerance); a point that
fails is refused and no JSON line is printed.  The CPU-baseline leg runs the
oracle over worker processes on the headline tokens and further tokens of the
same workload, and compares its outputs with the GPU's for the headline tokens.

The expert weights are replicated ``--copies`` times and the steps rotate over
the copies, so the 256 MiB Infinity Cache cannot serve the weights of the next
step (``copies_plateau`` shows the time no longer falls with more copies).

Timed steps run inside one HIP graph: the K timed forwards (rotating over the
weight copies) are captured once into a single graph, which is replayed three
times with the output cleared, eager work and a synchronisation in between and
must reproduce the eager output bit for bit; the timed region is then one
replay of the K steps, after the warm-up steps.  Launched this way, no step
waits on the host: eager launches fetch their kernel arguments from host memory
on machines whose runtime keeps them there (about 1.1 us per launch, four or
five launches per layer), and a graph of one forward per replay pays about 5 us
of launch latency per replay.  The eager time is reported beside the graph time
(``eager_ms_per_layer``).  The dominant kernel (grouped gate/up) is
additionally timed per launch with HIP events through the library's one-shot
timing hook (eager launches; the events bracket the kernel itself), for the
roofline.

After the headline, the other workload points are timed (``--sweep``; each the
median of three windows of at least 5 ms of steps), then the 16-layer prefill stack (RMSNorm + MoE + residual per layer, T=2048, Zipf
routing with the busiest expert at about 4x the mean), then the oracle on the
host cores as a reported CPU baseline.

    python bench.py [--gpus 1] [--steps 50] [--warmup 5] [--workload olmoe_bf16 --tokens 8]
Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 matrix peak, TFLOP/s
PROFILES = os.path.join(ROOT, "profiles")

# the curve over T = 1, 2, 4, ..., 2048 on the OLMoE-shaped (uniform) and DeepSeek-shaped
# (Zipf) layers, the speculative-verify size T = 9, and the int8 points
_POW2 = (1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048)
DEFAULT_SWEEP = ",".join([f"olmoe_bf16:{t}" for t in sorted(set(_POW2) - {8} | {9})] +
                         ["olmoe_i8:1", "olmoe_i8:8", "olmoe_i8:64", "olmoe_i8_zipf:8"] +
                         [f"deepseek_bf16:{t}" for t in _POW2])


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=16,
                   help="untimed steps before the timed ones (the default touches each of the 8 "
                        "weight copies twice: a copy's first pass pays page-table walks, and the "
                        "clocks settle)")
    p.add_argument("--workload", default="olmoe_bf16")
    p.add_argument("--tokens", type=int, default=8)
    p.add_argument("--copies", type=int, default=8, help="weight replicas rotated over (cache defeat)")
    p.add_argument("--sweep", default=DEFAULT_SWEEP,
                   help="extra workload:T points timed after the headline ('' or none for none)")
    p.add_argument("--sweep-steps", type=int, default=20)
    p.add_argument("--no-stack", action="store_true", help="skip the 16-layer prefill stack")
    p.add_argument("--capacity", default="deepseek_bf16:2048@1.0,deepseek_bf16:2048@2.0,"
                   "olmoe_stack16:2048@1.0,olmoe_stack16:2048@2.0",
                   help="workload:T@capacity_factor points with token dropping ('' or none for none)")
    p.add_argument("--stack-steps", type=int, default=5, help="timed passes over the 16 layers")
    p.add_argument("--no-extras", action="store_true",
                   help="skip the step percentiles, copies plateau and copy ceiling")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="oracle CPU baseline budget")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--counters-pass", action="store_true",
                   help="for rocprofv3 --pmc runs: a 256 MiB device copy (the counters' "
                        "calibration), then the headline steps only; prints no JSON")
    return p.parse_args()


# ------------------------------------------------------------------------------------------
# algorithmic work of one layer (bytes that must move, flops that must be done)
# ------------------------------------------------------------------------------------------
def layer_work(wl, T, n_touched_routed):
    """Bytes and flops per kernel of one layer, from the GPU's own routing.

    Weight bytes count each touched expert once (and the int8 scales); activations
    count each tensor the kernel must read or write once."""
    bw = {"f32": 4, "bf16": 2, "i8": 1}[wl.wdt]
    ba = {"f32": 4, "bf16": 2}[wl.act]
    G = n_touched_routed + wl.S
    R = T * wl.k + wl.S * T
    sc_gu = 2 * wl.I * 4 if wl.wdt == "i8" else 0
    sc_d = wl.d * 4 if wl.wdt == "i8" else 0
    gate_up = G * (2 * wl.I * wl.d * bw + sc_gu) + T * wl.d * ba + R * wl.I * ba
    down = G * (wl.d * wl.I * bw + sc_d) + R * wl.I * ba + R * wl.d * ba
    router = wl.E * wl.d * ba + T * wl.d * ba + T * wl.E * 4
    combine = R * wl.d * ba + T * wl.d * ba + T * wl.k * 8
    return {
        "gate_up_bytes": gate_up, "down_bytes": down,
        "layer_bytes": gate_up + down + router + combine,
        "gate_up_flops": 2.0 * R * wl.d * 2 * wl.I, "down_flops": 2.0 * R * wl.I * wl.d,
        "layer_flops": 2.0 * R * wl.d * 3 * wl.I + 2.0 * T * wl.d * wl.E,
        "touched_groups": G,
    }


def mfma_bound(wl, T, work):
    """Whether a layer's gate/up kernel is bound by the matrix cores rather than by HBM:
    its flops at the bf16 peak take longer than its algorithmic bytes at the HBM peak."""
    return (wl.act == "bf16" and work["gate_up_flops"] / (MFMA_BF16_PEAK_TFS * 1e12)
            > work["gate_up_bytes"] / (HBM_PEAK_GBS * 1e9))


# ------------------------------------------------------------------------------------------
# timing helpers (all on torch's current stream, which is the stream the library launches on)
# ------------------------------------------------------------------------------------------
def _events(n):
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in evs:  # torch creates the HIP events on first record
        a.record()
        b.record()
    torch.cuda.synchronize()
    return evs


def time_steps(step, steps, warmup):
    """Mean ms of one step over exactly `steps` steps bracketed by synchronisations."""
    import torch
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for i in range(steps):
        step(i)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return ev0.elapsed_time(ev1) / steps, wall


def warm_up(step, copies, min_s=0.05):
    """Untimed steps for the sweep and capacity points: two rotations over the weight copies,
    then more until at least `min_s` seconds of GPU work have run (the first passes over a
    copy pay page-table walks, and the clocks take tens of ms to settle).  Returns the count
    and the ms of one step measured on the way."""
    import torch
    n = 2 * copies
    for i in range(n):
        step(i)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for i in range(copies):
        step(i)
    ev1.record()
    torch.cuda.synchronize()
    n += copies
    per_step = max(ev0.elapsed_time(ev1) / copies * 1e-3, 1e-6)
    extra = max(0, int(min_s / per_step) - n)
    for i in range(extra):
        step(i)
    return n + extra, per_step * 1e3


def time_steps_median(step, steps, per_step_ms, windows=3, min_window_ms=5.0):
    """The sweep and capacity points: the median of `windows` timed windows, each of at least
    `steps` steps and `min_window_ms` of GPU work, so that one slow step in a short window
    (a decode layer takes 30 µs) does not move the point."""
    n = window_steps(steps, per_step_ms, min_window_ms)
    runs = sorted(time_steps(step, n, 0) for _ in range(windows))
    return runs[len(runs) // 2]


def step_percentiles(step, n):
    """p10 / median / p90 of single steps, each bracketed by its own event pair."""
    import numpy as np
    import torch
    evs = _events(n)
    for i, (a, b) in enumerate(evs):
        a.record()
        step(i)
        b.record()
    torch.cuda.synchronize()
    d = np.array([a.elapsed_time(b) for a, b in evs])
    return {"p10": round(float(np.percentile(d, 10)), 5), "p50": round(float(np.median(d)), 5),
            "p90": round(float(np.percentile(d, 90)), 5)}


def time_kernel(kernel, launch, launches):
    """Average duration (ms) of one kernel, bracketed by HIP events that the library records
    on the kernel's own stream around its next launch; `launch(i)` runs one layer."""
    import torch

    from grouped_expert_ffn_amd import abi
    evs = _events(launches)
    for i, (a, b) in enumerate(evs):
        abi.moe_time_next_launch(kernel, a, b)
        launch(i)
    torch.cuda.synchronize()
    ds = [a.elapsed_time(b) for a, b in evs]
    return sum(ds) / len(ds), min(ds)


def capture_graphs(captures, y, reference, checks=3):
    """One HIP graph per entry of `captures` (each `capture(stream)` records its launches on
    the capture stream it is handed).  Every graph is replayed `checks` times, with `y`
    cleared, eager work and a synchronisation between replays, and must reproduce
    `reference` bit for bit, else the point is refused.  Returns the graphs."""
    import torch
    graphs = []
    torch.cuda.synchronize()
    for capture in captures:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            capture(torch.cuda.current_stream().cuda_stream)
        graphs.append(g)
    for g in graphs:
        for _ in range(checks):
            y.zero_()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            if not torch.equal(y, reference):
                raise SystemExit("graph replay differs from the eager result; refusing to time it")
    return graphs


def time_graph(g, n_steps, warm=None, warmup=0):
    """ms of one step when one replay of `g` runs `n_steps` steps, after `warmup` untimed
    calls of `warm(i)`; the replay is bracketed by synchronisations."""
    import torch
    for i in range(warmup):
        warm(i)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    g.replay()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return ev0.elapsed_time(ev1) / n_steps, wall


def time_graph_median(g, n_steps, windows=3):
    """The median of `windows` replays (each `n_steps` steps), as ms per step."""
    runs = sorted(time_graph(g, n_steps) for _ in range(windows))
    return runs[len(runs) // 2]


def window_steps(steps, per_step_ms, min_window_ms=5.0):
    """Steps in a timed window of a sweep or capacity point: at least `steps` and at least
    `min_window_ms` of GPU work."""
    return max(steps, int(min_window_ms / max(per_step_ms, 1e-3)) + 1)


def copy_ceiling_gbs(mib=1024, reps=10):
    """Read + write bandwidth of a plain device-to-device copy (context for the peak)."""
    import torch
    a = torch.empty(mib << 20, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(reps):
        b.copy_(a)
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / reps
    del a, b
    torch.cuda.empty_cache()
    return round(2 * (mib << 20) / (ms * 1e-3) / 1e9, 1)


# ------------------------------------------------------------------------------------------
# HBM traffic from a committed rocprofv3 PMC summary, valid only for the kernel source it
# was taken on
# ------------------------------------------------------------------------------------------
def _sources_digest(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def read_traffic(summary_name):
    """Bytes per launch = FETCH_SIZE * fetch_scale + WRITE_SIZE * write_scale (KiB), from
    `profiles/<summary_name>`; None when the summary is missing or its kernel sources have
    changed since the counters were taken."""
    path = os.path.join(PROFILES, summary_name)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if "=" in line:
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    try:
        srcs = [s.strip() for s in kv["sources"].split(",")]
        if _sources_digest(srcs) != kv["sources_sha256"]:
            return None
        kib = (float(kv["fetch_kib_per_dispatch"]) * float(kv["fetch_scale"])
               + float(kv["write_kib_per_dispatch"]) * float(kv["write_scale"]))
    except (KeyError, ValueError, OSError):
        return None
    return int(kib * 1024)


# ------------------------------------------------------------------------------------------
# one workload point on the GPU
# ------------------------------------------------------------------------------------------
_HOST = {}


def host_layer(wl, seed=0):
    import moe_synth as S
    key = (wl.name, seed)
    if key not in _HOST:
        _HOST.clear()
        _HOST[key] = S.make_layer(wl, 0, seed)
    return _HOST[key]


def _forward_args(desc, T, x, L, residual, y, ws, stream):
    import ctypes
    ptr = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    return (ctypes.byref(desc), T, x.data_ptr(), L.w_router.data_ptr(), ptr(L.bias),
            ctypes.byref(L.weights), ptr(residual), y.data_ptr(), None, None, ws.data_ptr(),
            ws.numel(), stream)


def _call(lib, args):
    st = lib.moe_forward(*args)
    if st != 0:
        from grouped_expert_ffn_amd import abi
        raise abi.MoeError(st, "moe_forward", abi.last_error())


class Point:
    """One layer at T tokens, its weights replicated `copies` times on the GPU (layer 0 of the
    workload; `cf` > 0 turns on capacity-factor dropping)."""

    def __init__(self, wl, T, copies, seed=0, cf=0.0):
        import torch

        import moe_synth as S
        from grouped_expert_ffn_amd import DTYPES, DeviceLayer, abi, make_desc, to_device
        self.wl, self.T = wl, T
        self.host = host_layer(wl, seed)
        self.x_host = S.make_tokens(wl, T, seed)
        self.cf = cf
        self.desc = make_desc(wl.d, wl.E, wl.k, wl.I, wl.S, wl.renormalize, DTYPES[wl.act],
                              DTYPES[wl.wdt], wl.pre_norm, wl.norm_eps, cf)
        h = self.host
        base = DeviceLayer(self.desc, h.w_router, h.bias, h.w_gate, h.w_up, h.w_down, h.s_gate,
                           h.s_up, h.s_down)
        self.layers = [base]
        c = lambda t: None if t is None else t.clone()  # noqa: E731
        for _ in range(copies - 1):
            self.layers.append(DeviceLayer(self.desc, base.w_router, base.bias, c(base.w_gate),
                                           c(base.w_up), c(base.w_down), c(base.s_gate),
                                           c(base.s_up), c(base.s_down)))
        self.x = to_device(self.x_host)
        self.y = torch.empty_like(self.x)
        self.ids = torch.empty((T, wl.k), dtype=torch.int32, device="cuda")
        self.ws = base.workspace(T)
        # pre-marshalled ctypes arguments: the timed loop is one C call per step
        self.lib = abi.lib()
        self.args = [self.args_for(L, torch.cuda.current_stream().cuda_stream) for L in self.layers]

    def args_for(self, L, stream):
        return _forward_args(self.desc, self.T, self.x, L, None, self.y, self.ws, stream)

    def step(self, i):
        _call(self.lib, self.args[i % len(self.args)])

    def routing(self):
        import torch
        self.layers[0].forward(self.x, y=self.y, topk_ids=self.ids)
        torch.cuda.synchronize()
        return self.ids.cpu().numpy()

    def sanity_gate(self):
        """Refuse to time a layer whose output is not finite or not bit-identical over two
        runs; keeps the output and routing of the checked run."""
        import torch

        from grouped_expert_ffn_amd import from_device
        ids = self.routing()
        y1 = from_device(self.y).copy()
        ids2 = self.routing()
        y2 = from_device(self.y)
        yf = self.y.float()
        if not (bool(torch.isfinite(yf).all()) and (y1 == y2).all() and (ids == ids2).all()):
            raise SystemExit(f"{self.wl.name} T={self.T}: output not finite or not deterministic; "
                             "refusing to time")
        self.y_host, self.ids_host = y1, ids
        return ids

    def graph_of(self, n):
        """`n` forwards, step i on weight copy i % copies, captured in one graph and checked
        against the eager output."""
        import torch
        for i in range(len(self.args)):
            self.step(i)
        torch.cuda.synchronize()
        ref = self.y.clone()
        lib, args_for, layers = self.lib, self.args_for, self.layers

        def capture(stream):
            for i in range(n):
                _call(lib, args_for(layers[i % len(layers)], stream))
        self.graphs = capture_graphs([capture], self.y, ref)
        return self.graphs[0]

    def free(self):
        import torch
        self.graphs = None
        self.layers.clear()
        self.args.clear()
        torch.cuda.empty_cache()


DTYPE_CODES = {"f32": 0, "bf16": 1, "i8": 2}  # moe_dtype_t


def roofline_for(wl, T, work, kern_ms, traffic=None):
    """Roofline of the gate/up kernel: its algorithmic bytes against the HBM peak and its
    flops against the bf16 matrix peak; the bound is whichever takes longer at peak, and
    frac is that time over the measured launch time."""
    from grouped_expert_ffn_amd import abi
    desc = abi.make_desc(wl.d, wl.E, wl.k, wl.I, wl.S, wl.renormalize, DTYPE_CODES[wl.act],
                         DTYPE_CODES[wl.wdt])
    family = abi.moe_ffn_kernel(desc, T)  # the library's own choice for this layer and T
    name = "grouped gate/up + SwiGLU (" + {abi.MOE_FFN_GEMV: "GEMV", abi.MOE_FFN_GEMV_MFMA: "matrix-core GEMV",
                                          abi.MOE_FFN_GEMM: "MFMA GEMM"}[family] + ")"
    hbm = work["gate_up_bytes"] / (kern_ms * 1e-3) / 1e9
    mfma = work["gate_up_flops"] / (kern_ms * 1e-3) / 1e12
    common = {"kernel": name, "traffic": traffic, "bytes_per_launch": work["gate_up_bytes"],
              "flops_per_launch": work["gate_up_flops"], "avg_launch_ms": round(kern_ms, 5),
              "hbm_frac": round(hbm / HBM_PEAK_GBS, 4), "mfma_frac": round(mfma / MFMA_BF16_PEAK_TFS, 4)}
    if mfma_bound(wl, T, work):
        return {"bound": "mfma", "achieved": round(mfma, 1), "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
                "frac": round(mfma / MFMA_BF16_PEAK_TFS, 4), **common}
    return {"bound": "hbm", "achieved": round(hbm, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(hbm / HBM_PEAK_GBS, 4), **common}


def _fracs(work, ms):
    return (round(work["layer_bytes"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            round(work["layer_flops"] / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS, 4))


def measure(wl, T, steps, warmup, copies, extras=False):
    """warmup: untimed steps before the timed ones, or None for warm_up()'s count."""
    import numpy as np

    from grouped_expert_ffn_amd import abi
    pt = Point(wl, T, copies)
    ids = pt.sanity_gate()
    gate = oracle_gate(wl, pt.host, pt.x_host, pt.y_host, ids, gate_tokens(T), what=f"{wl.name} T={T}")
    n_touched = int(np.count_nonzero(np.bincount(ids.ravel(), minlength=wl.E)))
    work = layer_work(wl, T, n_touched)
    if warmup is None:  # a sweep point
        _, per_step = warm_up(pt.step, copies)
        n = window_steps(steps, per_step)
        ms, wall = time_graph_median(pt.graph_of(n), n)
        eager_ms, _ = time_steps_median(pt.step, steps, per_step)
    else:
        ms, wall = time_graph(pt.graph_of(steps), steps, pt.step, warmup)
        eager_ms, _ = time_steps(pt.step, steps, warmup)
    launches = 50  # the average over 50 launches, as rocprofv3's kernel statistics report it
    gu_ms, _ = time_kernel(abi.MOE_KERNEL_GATE_UP, pt.step, launches)
    dn_ms, _ = time_kernel(abi.MOE_KERNEL_DOWN, pt.step, launches)
    hbm, mfma = _fracs(work, ms)
    res = {
        "workload": wl.name, "tokens": T, "ms_per_layer": round(ms, 5),
        "tokens_per_s": round(T / (ms * 1e-3), 1),
        "layer_hbm_frac": hbm, "layer_mfma_frac": mfma,
        "gate_up_ms": round(gu_ms, 5), "down_ms": round(dn_ms, 5),
        "gate_up_hbm_frac": round(work["gate_up_bytes"] / (gu_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "down_hbm_frac": round(work["down_bytes"] / (dn_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "touched_experts": n_touched,
        "eager_ms_per_layer": round(eager_ms, 5),
        "oracle_gate": gate,
    }
    if T > 8 and wl.act == "bf16":
        res["gate_up_mfma_frac"] = round(work["gate_up_flops"] / (gu_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS, 4)
        res["down_mfma_frac"] = round(work["down_flops"] / (dn_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS, 4)
    if extras:
        res["eager_step_ms_percentiles"] = step_percentiles(pt.step, steps)
    roof = roofline_for(wl, T, work, gu_ms)
    # the whole layer (every launch of the step) against the same HBM peak, beside the one
    # kernel's fraction: at small T the fixed cost of the other launches is what separates them
    roof["layer_hbm_frac"] = hbm
    roof["layer_ms"] = round(ms, 5)
    checked = (pt.x_host, pt.y_host, pt.ids_host)
    pt.free()
    return res, roof, ms, wall, work, checked


def copies_plateau(wl, T, counts=(1, 2, 4, 8, 16), steps=50):
    """Layer time against the number of weight copies rotated over: it falls while the
    Infinity Cache still holds the next step's weights, then stays flat.  Timed like the
    headline (warm-up of at least two rotations and 16 steps, then one graph of the steps)."""
    out = {}
    for n in counts:
        pt = Point(wl, T, n)
        ms, _ = time_graph(pt.graph_of(steps), steps, pt.step, max(16, 2 * n))
        out[str(n)] = round(ms, 5)
        pt.free()
    return out


# ------------------------------------------------------------------------------------------
# the 16-layer prefill stack: h <- h + MoE_l(RMSNorm(h)), l = 0..15, every pass from the same
# input (layers ping-pong between two buffers, so no copy is timed)
# ------------------------------------------------------------------------------------------
class Stack:
    def __init__(self, wl, T):
        import torch

        import moe_synth as S
        from grouped_expert_ffn_amd import DTYPES, DeviceLayer, abi, make_desc, to_device
        self.wl, self.T = wl, T
        self.desc = make_desc(wl.d, wl.E, wl.k, wl.I, wl.S, wl.renormalize, DTYPES[wl.act],
                              DTYPES[wl.wdt], wl.pre_norm, wl.norm_eps)
        self.x_host = S.make_tokens(wl, T)
        self.layers = []
        for layer in range(wl.n_layers):
            h = S.make_layer(wl, layer)
            self.layers.append(DeviceLayer(self.desc, h.w_router, h.bias, h.w_gate, h.w_up, h.w_down))
            if layer == 0:
                self.host0 = h  # for the oracle gate
            del h
        self.x0 = to_device(self.x_host)
        self.buf = [torch.empty_like(self.x0), torch.empty_like(self.x0)]
        self.ids = torch.empty((T, wl.k), dtype=torch.int32, device="cuda")
        self.ws = self.layers[0].workspace(T)
        self.lib = abi.lib()
        stream = torch.cuda.current_stream().cuda_stream
        self.args = []
        for i, L in enumerate(self.layers):
            src = self.x0 if i == 0 else self.buf[(i - 1) % 2]
            self.args.append(_forward_args(self.desc, T, src, L, src, self.buf[i % 2], self.ws, stream))

    def step(self, _i=0):
        for a in self.args:
            _call(self.lib, a)

    def layer(self, i):
        _call(self.lib, self.args[i % len(self.args)])

    def graph_of(self, passes):
        """`passes` whole passes captured in one graph, checked against the eager pass."""
        import torch
        self.step()
        torch.cuda.synchronize()
        out = self.buf[(len(self.layers) - 1) % 2]
        ref = out.clone()

        def capture(stream):
            for _ in range(passes):
                for i, L in enumerate(self.layers):
                    src = self.x0 if i == 0 else self.buf[(i - 1) % 2]
                    _call(self.lib, _forward_args(self.desc, self.T, src, L, src, self.buf[i % 2],
                                                  self.ws, stream))
        self.graphs = capture_graphs([capture], out, ref)
        return self.graphs[0]

    def sanity_gate(self):
        """Layer 0 twice: the output must be finite and bit-identical; records the busiest
        expert's load over the mean."""
        import numpy as np
        import torch

        wl, T = self.wl, self.T
        outs = []
        for _ in range(2):
            self.layers[0].forward(self.x0, residual=self.x0, y=self.buf[0], topk_ids=self.ids)
            torch.cuda.synchronize()
            outs.append(self.buf[0].clone())
        if not (bool(torch.isfinite(outs[0].float()).all()) and torch.equal(outs[0], outs[1])):
            raise SystemExit("stack layer 0: output not finite or not deterministic; refusing to time")
        from grouped_expert_ffn_amd import from_device
        ids = self.ids.cpu().numpy()
        self.gate = oracle_gate(wl, self.host0, self.x_host, from_device(outs[0]), ids, gate_tokens(T),
                                residual=self.x_host, what="stack layer 0")
        counts = np.bincount(ids.ravel(), minlength=wl.E)
        self.skew0 = float(counts.max() / (T * wl.k / wl.E))

    def free(self):
        import torch
        self.graphs = None
        self.layers.clear()
        self.args.clear()
        self.host0 = None
        torch.cuda.empty_cache()


def measure_stack(wl, steps):
    from grouped_expert_ffn_amd import abi
    st = Stack(wl, wl.tokens[0])
    st.sanity_gate()
    T, n = st.T, wl.n_layers
    warm_up(st.step, 1)
    ms, _ = time_graph(st.graph_of(steps), steps)
    eager_ms, _ = time_steps(st.step, steps, 0)
    gu_ms, _ = time_kernel(abi.MOE_KERNEL_GATE_UP, st.layer, 2 * n)
    dn_ms, _ = time_kernel(abi.MOE_KERNEL_DOWN, st.layer, 2 * n)
    work = layer_work(wl, T, wl.E)  # every expert is touched at T=2048
    per_layer = ms / n
    hbm, mfma = _fracs(work, per_layer)
    res = {
        "workload": wl.name, "tokens": T, "layers": n, "ms_per_stack": round(ms, 4),
        "ms_per_layer": round(per_layer, 5), "tokens_per_s_per_layer": round(T / (per_layer * 1e-3), 1),
        "layer_hbm_frac": hbm, "layer_mfma_frac": mfma,
        "gate_up_ms": round(gu_ms, 5), "down_ms": round(dn_ms, 5),
        "gate_up_mfma_frac": round(work["gate_up_flops"] / (gu_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS, 4),
        "down_mfma_frac": round(work["down_flops"] / (dn_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS, 4),
        "eager_ms_per_stack": round(eager_ms, 4),
        "busiest_over_mean_layer0": round(st.skew0, 3),
        "oracle_gate_layer0": st.gate,
    }
    st.free()
    return res


def drop_stats(ids, E, cf):
    """Rows per routed expert C = ceil(cf*T*k/E) (the library's rule) and which (token, slot)
    pairs fall past the first C of their expert, the pairs reaching experts in flat order."""
    import numpy as np
    T, k = ids.shape
    cap = int(np.ceil(float(np.float32(cf)) * T * k / E)) if cf > 0 else 0
    flat = ids.ravel()
    order = np.argsort(flat, kind="stable")
    starts = np.searchsorted(flat[order], np.arange(E))
    rank = np.empty(flat.size, dtype=np.int64)
    rank[order] = np.arange(flat.size) - starts[flat[order]]
    dropped = (rank >= cap).reshape(T, k) if cap > 0 else np.zeros((T, k), dtype=bool)
    return cap, dropped


def measure_capacity(wl, T, cf, steps, copies):
    """Layer time with capacity-factor dropping, and how much is dropped (the GPU's own
    routing)."""
    import numpy as np
    pt = Point(wl, T, copies, cf=cf)
    ids = pt.sanity_gate()
    cap, dropped = drop_stats(ids, wl.E, cf)
    gate = capacity_gate(wl, pt, ids, cf, dropped)
    _, per_step = warm_up(pt.step, copies)
    n = window_steps(steps, per_step)
    ms, _ = time_graph_median(pt.graph_of(n), n)
    eager_ms, _ = time_steps_median(pt.step, steps, per_step)
    pt.free()
    counts = np.bincount(ids.ravel(), minlength=wl.E)
    return {"workload": wl.name, "tokens": T, "capacity_factor": cf, "capacity_rows": cap,
            "ms_per_layer": round(ms, 5), "tokens_per_s": round(T / (ms * 1e-3), 1),
            "eager_ms_per_layer": round(eager_ms, 5),
            "dropped_pairs_frac": round(float(dropped.mean()), 4),
            "tokens_with_a_drop_frac": round(float(dropped.any(axis=1).mean()), 4),
            "busiest_over_mean": round(float(counts.max() / (T * wl.k / wl.E)), 3),
            "oracle_gate": gate}


def capacity_gate(wl, pt, ids, cf, dropped):
    """The oracle check of a capacity point: sampled tokens, among them tokens that lost a
    slot, with the dropped slots left out of the oracle's sum."""
    import numpy as np

    from oracle import moe_oracle as O
    T = pt.T
    lost = np.nonzero(dropped.any(axis=1))[0]
    tokens = sorted(set(gate_tokens(T)) | set(lost[:2].tolist()))
    xs, _ = layer_input(wl, pt.x_host[tokens])
    logits = O.router_logits(xs, pt.host.w_router, pt.host.bias)
    ids_g = ids[tokens]
    w = O.gate_weights_for(logits, ids_g, wl.renormalize)
    keep = O.kept_slots(ids, wl.E, O.capacity(cf, T, wl.k, wl.E))[tokens]
    ref = O.moe_layer(xs, O.Experts.from_layer(pt.host), ids_g, w, wl.S, wl.E, keep=keep)
    got = O.widen(pt.y_host[tokens])
    rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    mx = float(np.max(np.abs(got - ref)) / np.max(np.abs(ref)))
    if not (rel <= 1e-2 and mx <= 2e-2):
        raise SystemExit(f"{wl.name} T={T} cf={cf}: oracle disagrees (rel-L2 {rel:.3e}, "
                         f"max-abs/max {mx:.3e}); refusing to time")
    return {"tokens": len(tokens), "rel_l2": float(f"{rel:.3e}"), "max_abs_over_max": float(f"{mx:.3e}")}


# ------------------------------------------------------------------------------------------
# parity gate of every timed point: sampled tokens against the fp64 oracle
# ------------------------------------------------------------------------------------------
TIE_DELTA = 1e-4        # pre-registered routing tie margin (fp64 logits)
TIE_DELTA_NORM = 1e-3   # the router input is a bf16 rounding of an fp32 RMSNorm


def layer_input(wl, xs):
    """What the router and the experts see (the RMSNorm of the stacked workload, stored in the
    activation type), and the tie margin that goes with it."""
    from oracle import moe_oracle as O
    if not wl.pre_norm:
        return xs, TIE_DELTA
    xn = O.stack_layer_input(xs, wl.norm_eps) if wl.act == "bf16" else O.rmsnorm(xs, wl.norm_eps)
    return xn, TIE_DELTA_NORM


def oracle_gate(wl, host, x_host, y_bits, ids_gpu, tokens, residual=None, what=""):
    """Refuse to time a point whose sampled tokens disagree with the oracle: a routing choice
    may differ from the oracle's only on a pre-registered near-tie, and the layer output,
    computed by the oracle for the GPU's own choice, must be within rel-L2 1e-2 (1e-5 for
    fp32) and max-abs 2e-2 * max|y|.  `x_host` is the layer input as the router sees it."""
    import numpy as np

    from oracle import moe_oracle as O
    tokens = list(tokens)
    xs, delta = layer_input(wl, x_host[tokens])
    logits = O.router_logits(xs, host.w_router, host.bias)
    ids_o, _ = O.route(logits, wl.k, False)
    ids_g = ids_gpu[tokens]
    for i in range(len(tokens)):
        if list(ids_g[i]) != list(ids_o[i]):
            srt = np.sort(logits[i])[::-1]
            margin = srt[wl.k - 1] - srt[wl.k] if wl.k < wl.E else np.inf
            gaps = np.abs(np.diff(srt[:wl.k + 1]))
            if not (margin < delta or (len(gaps) and np.min(gaps) < delta)):
                raise SystemExit(f"{what}: token {tokens[i]} routed {list(ids_g[i])}, oracle "
                                 f"{list(ids_o[i])} (margin {margin:.2e}); refusing to time")
    w = O.gate_weights_for(logits, ids_g, wl.renormalize)
    res = None if residual is None else O.widen(residual[tokens])
    ref = O.moe_layer(xs, O.Experts.from_layer(host), ids_g, w, wl.S, wl.E, residual=res)
    got = O.widen(y_bits[tokens])
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    mx = float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-300))
    lim = 1e-5 if wl.act == "f32" else 1e-2
    if not (rel <= lim and mx <= 2e-2):
        raise SystemExit(f"{what}: oracle disagrees on tokens {tokens}: rel-L2 {rel:.3e}, "
                         f"max-abs/max {mx:.3e}; refusing to time")
    return {"tokens": len(tokens), "rel_l2": float(f"{rel:.3e}"), "max_abs_over_max": float(f"{mx:.3e}")}


def gate_tokens(T, n=3):
    """A few tokens spread over the batch (first, middle, last)."""
    return sorted({0, T // 2, T - 1})[:n]


# ------------------------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, in worker processes over distinct tokens
# ------------------------------------------------------------------------------------------
def cpu_workers() -> int:
    """Worker processes for the oracle: the host cores this process may use, at most the
    thread budget the environment sets (OMP_NUM_THREADS) and at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    try:
        n = min(n, int(os.environ.get("OMP_NUM_THREADS", n)))
    except ValueError:
        pass
    return max(1, min(16, n))


def _oracle_worker(name, head_T, n_extra, lo, hi, budget_s, barrier, out_q):
    """One worker of the CPU baseline: tokens [lo, hi) of (the headline tokens, then n_extra
    further tokens of the same workload), one token at a time through the oracle, until done
    or out of time.  Weights are widened once per expert (the oracle's lazy cache)."""
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # pragma: no cover
        pass
    import numpy as np

    import moe_synth as S
    from oracle import moe_oracle as O
    wl = S.WORKLOADS[name]
    host = S.make_layer(wl, 0, 0, threads=1)
    xs = np.concatenate([S.make_tokens(wl, head_T), S.make_tokens(wl, n_extra, seed=1)])
    ex = O.Experts.from_layer(host)
    barrier.wait()
    t0 = time.perf_counter()
    done, head = 0, []
    for t in range(lo, hi):
        xt = xs[t:t + 1]
        _, ids, w = O.full_route(xt, host.w_router, host.bias, wl.k, wl.renormalize)
        y = O.moe_layer(xt, ex, ids, w, wl.S, wl.E)
        if t < head_T:
            head.append((t, ids[0], y[0]))
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    out_q.put((done, time.perf_counter() - t0, head))


def cpu_baseline(wl, T, budget_s, checked):
    """The fp64 oracle as it stands, spread over worker processes on distinct tokens of the
    same workload (the headline tokens first), for about `budget_s` seconds.  Its outputs for
    the headline tokens are compared with the GPU's (`checked`: tokens, output bits and routing
    of the run the sanity gate kept) wherever the oracle picked the same experts; none in
    common, or a disagreement, withholds the bench line."""
    import multiprocessing as mp

    import numpy as np

    from oracle import moe_oracle as O
    x_host, y_gpu, ids_gpu = checked
    n = cpu_workers()
    per = 48                                  # tokens per worker at most (the bounded sample)
    total = n * per
    n_extra = max(0, total - T)
    ctx = mp.get_context("spawn")             # fresh interpreters: no GPU state is inherited
    barrier, q = ctx.Barrier(n + 1), ctx.Queue()
    bounds = [(i * total // n, (i + 1) * total // n) for i in range(n)]
    procs = [ctx.Process(target=_oracle_worker, args=(wl.name, T, n_extra, lo, hi, budget_s, barrier, q))
             for lo, hi in bounds]
    for p in procs:
        p.start()
    try:
        barrier.wait(timeout=600)             # every worker has its weights and tokens
        t0 = time.perf_counter()
        results = [q.get(timeout=budget_s + 600) for _ in procs]
        wall = time.perf_counter() - t0
    except Exception as e:                    # a worker died or stalled: no baseline
        for p in procs:
            p.kill()
        raise SystemExit(f"CPU baseline workers failed ({type(e).__name__}); no bench line")
    for p in procs:
        p.join()
    done = sum(r[0] for r in results)
    head = sorted([h for r in results for h in r[2]], key=lambda h: h[0])
    out = {"value": round(done / wall, 3), "unit": "tokens/s", "cores": n, "kind": "oracle",
           "sample": f"{done} distinct tokens of {wl.name} (the {T} headline tokens, then further "
                     f"seeded tokens), {n} worker processes, fp64 per-token per-expert loop "
                     f"incl. weight widening, {wall:.1f} s"}
    same = [(t, y) for t, ids, y in head if np.array_equal(ids, ids_gpu[t])]
    if not same:
        raise SystemExit(f"oracle and GPU share no routing on the {T} headline tokens; no bench line")
    ref = np.array([y for _, y in same])
    got = O.widen(y_gpu[[t for t, _ in same]])
    rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    mx = float(np.max(np.abs(got - ref)) / np.max(np.abs(ref)))
    out["parity"] = {"tokens": len(head), "same_routing": len(same),
                     "rel_l2": float(f"{rel:.3e}"), "max_abs_over_max": float(f"{mx:.3e}")}
    lim = 1e-5 if wl.act == "f32" else 1e-2
    if not (rel <= lim and mx <= 2e-2):
        raise SystemExit(f"oracle disagrees with the GPU on {wl.name} T={T}: rel-L2 {rel:.3e}, "
                         f"max-abs/max {mx:.3e}; no bench line")
    return out


def counters_pass(wl, T, steps, warmup, copies):
    """What a rocprofv3 --pmc run profiles: the copy kernel whose FETCH_SIZE / WRITE_SIZE
    calibrate the counters (256 MiB read, 256 MiB written per dispatch), then the steps."""
    import torch
    a = torch.ones(256 << 20, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    del a, b
    pt = Point(wl, T, copies)
    pt.sanity_gate()
    time_steps(pt.step, steps, warmup)
    pt.free()
    print(f"counters pass done: {wl.name} T={T}, {steps} steps", flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "the library runs on one GPU; --gpus must be 1 "
                          "(the path has no multi-GPU sharding or collectives)"}), flush=True)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    import moe_synth as S
    wl = S.WORKLOADS[args.workload]
    if args.counters_pass:
        counters_pass(wl, args.tokens, args.steps, args.warmup, args.copies)
        return
    res, roof, ms, wall, work, checked = measure(wl, args.tokens, args.steps, args.warmup, args.copies,
                                                 extras=not args.no_extras)
    kind = "gemm" if "GEMM" in roof["kernel"] else "gemv"
    roof["traffic"] = read_traffic(f"{kind}_gateup_{wl.name}_T{args.tokens}.pmc.txt")
    print(f"# headline {wl.name} T={args.tokens}: {ms:.4f} ms/layer", file=sys.stderr, flush=True)
    extras = {}
    if not args.no_extras:
        extras["copies_plateau_ms"] = copies_plateau(wl, args.tokens)
        extras["copy_ceiling_gbs"] = copy_ceiling_gbs()
    sweep = []
    for item in [s for s in args.sweep.split(",") if s.strip() and s.strip() != "none"]:
        name, t = item.split(":")
        if name == wl.name and int(t) == args.tokens:
            continue
        r, rf, *_ = measure(S.WORKLOADS[name], int(t), args.sweep_steps, None, args.copies)
        r["roofline_frac"] = rf["frac"]
        r["roofline_bound"] = rf["bound"]
        sweep.append(r)
        print(f"# sweep {name} T={t}: {r['ms_per_layer']:.4f} ms/layer, {r['tokens_per_s']:.0f} tok/s, "
              f"{rf['bound']} frac {rf['frac']:.3f}", file=sys.stderr, flush=True)
    stack = None
    if not args.no_stack:
        stack = measure_stack(S.OLMOE_STACK16, args.stack_steps)
        print(f"# stack: {stack['ms_per_stack']:.3f} ms / {stack['layers']} layers", file=sys.stderr,
              flush=True)
    capacity = []
    for item in [c for c in args.capacity.split(",") if c.strip() and c.strip() != "none"]:
        point, cf = item.split("@")
        name, t = point.split(":")
        r = measure_capacity(S.WORKLOADS[name], int(t), float(cf), args.sweep_steps, args.copies)
        capacity.append(r)
        print(f"# capacity {name} T={t} cf={cf}: {r['ms_per_layer']:.4f} ms/layer, "
              f"{100 * r['dropped_pairs_frac']:.1f}% of pairs dropped", file=sys.stderr, flush=True)
    cpu = None if args.no_cpu_baseline else cpu_baseline(wl, args.tokens, args.cpu_seconds, checked)
    out = {
        "metric": "MoE-layer tokens/s (one MoE layer forward, T tokens per step)",
        "value": res["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": res["ms_per_layer"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16"}[wl.act] + ("+i8w" if wl.wdt == "i8" else ""),
        "data": "synthetic (seeded N(0,1) tokens, N(0,0.02) weights)",
        "config": {"workload": wl.name, "tokens": args.tokens, "d_model": wl.d, "experts": wl.E,
                   "top_k": wl.k, "d_ff": wl.I, "shared": wl.S, "weight_copies": args.copies,
                   "parallelism": "single GPU"},
        "detail": res,
        "roofline": roof,
        "cpu_baseline": cpu,
        "extras": extras,
        "sweep": sweep,
        "stack": stack,
        "capacity": capacity,
        "wall_s_timed": round(wall, 3),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
