#!/usr/bin/env python3
"""Throughput of the MoE dispatch layer on one MI355X.

One step = one ``moe_forward`` (router, top-k, sort, grouped gate/up + SwiGLU,
grouped down, combine) over one batch of seeded synthetic tokens whose weights
and inputs are already resident in HBM.  The headline workload is the
OLMoE-shaped decode layer (d=2048, E=64, k=8, I=1024, bf16) at T=8 tokens.

Before anything is timed, the layer's output on sampled tokens is checked
against the fp64 CPU oracle; a disagreeing build is refused, not timed.

The expert weights are replicated ``--copies`` times and the steps rotate over
the copies, so the 256 MiB Infinity Cache cannot serve the weights of the next
step.  The dominant kernel (grouped gate/up) is additionally timed per launch
with HIP events through the library's one-shot timing hook, for the roofline.

    python bench.py [--gpus 1] [--steps 50] [--warmup 5] [--workload olmoe_bf16 --tokens 8]
Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 matrix peak, TFLOP/s


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="olmoe_bf16")
    p.add_argument("--tokens", type=int, default=8)
    p.add_argument("--copies", type=int, default=8, help="weight replicas rotated over (cache defeat)")
    p.add_argument("--sweep", default="olmoe_bf16:1,olmoe_bf16:64,olmoe_i8:1,olmoe_i8:8,"
                   "deepseek_bf16:1,deepseek_bf16:16,deepseek_bf16:2048",
                   help="extra workload:T points timed after the headline ('' for none)")
    p.add_argument("--sweep-steps", type=int, default=20)
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="oracle CPU baseline budget")
    p.add_argument("--no-cpu-baseline", action="store_true")
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


class Point:
    def __init__(self, wl, T, copies, seed=0):
        import torch

        import moe_synth as S
        from grouped_expert_ffn_amd import DTYPES, DeviceLayer, make_desc, to_device
        self.wl, self.T = wl, T
        self.host = host_layer(wl, seed)
        self.x_host = S.make_tokens(wl, T, seed)
        self.desc = make_desc(wl.d, wl.E, wl.k, wl.I, wl.S, wl.renormalize, DTYPES[wl.act],
                              DTYPES[wl.wdt], wl.pre_norm, wl.norm_eps)
        h = self.host
        base = DeviceLayer(self.desc, h.w_router, h.bias, h.w_gate, h.w_up, h.w_down, h.s_gate,
                           h.s_up, h.s_down)
        self.layers = [base]
        for _ in range(copies - 1):
            c = lambda t: None if t is None else t.clone()  # noqa: E731
            self.layers.append(DeviceLayer(self.desc, base.w_router, base.bias, c(base.w_gate),
                                           c(base.w_up), c(base.w_down), c(base.s_gate),
                                           c(base.s_up), c(base.s_down)))
        self.x = to_device(self.x_host)
        self.y = torch.empty_like(self.x)
        self.ids = torch.empty((T, wl.k), dtype=torch.int32, device="cuda")
        ws = base.workspace(T)
        self.ws = ws
        # pre-marshalled ctypes arguments: the timed loop is one C call per step
        import ctypes

        from grouped_expert_ffn_amd import abi
        self.lib = abi.lib()
        self.stream = torch.cuda.current_stream().cuda_stream
        self.args = []
        for L in self.layers:
            self.args.append((ctypes.byref(self.desc), T, self.x.data_ptr(), L.w_router.data_ptr(),
                              None if L.bias is None else L.bias.data_ptr(), ctypes.byref(L.weights),
                              None, self.y.data_ptr(), None, None, ws.data_ptr(), ws.numel(),
                              self.stream))

    def step(self, i):
        st = self.lib.moe_forward(*self.args[i % len(self.args)])
        if st != 0:
            from grouped_expert_ffn_amd import abi
            raise abi.MoeError(st, "moe_forward", abi.last_error())

    def routing(self):
        import torch
        self.layers[0].forward(self.x, y=self.y, topk_ids=self.ids)
        torch.cuda.synchronize()
        return self.ids.cpu().numpy()

    def parity_gate(self, n_tokens=8):
        """Check sampled tokens against the fp64 oracle; raise if they disagree."""
        import numpy as np

        from grouped_expert_ffn_amd import from_device
        from oracle import moe_oracle as O
        ids = self.routing()
        y = O.widen(from_device(self.y))
        T = self.T
        tok = sorted(set(np.linspace(0, T - 1, min(T, n_tokens)).astype(int).tolist()))
        logits = O.router_logits(self.x_host[tok], self.host.w_router, self.host.bias)
        w = O.gate_weights_for(logits, ids[tok], self.wl.renormalize)
        ref = O.moe_layer(self.x_host[tok], O.Experts.from_layer(self.host), ids[tok], w,
                          self.wl.S, self.wl.E)
        got = y[tok]
        rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
        mx = float(np.max(np.abs(got - ref)) / np.max(np.abs(ref)))
        lim = 1e-5 if self.wl.act == "f32" else 1e-2
        if not (rel <= lim and mx <= 2e-2):
            raise SystemExit(f"parity gate FAILED for {self.wl.name} T={T}: rel-L2 {rel:.3e}, "
                             f"max-abs/max {mx:.3e}; refusing to time")
        return rel

    def time_steps(self, steps, warmup):
        import torch
        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        ev0.record()
        for i in range(steps):
            self.step(i)
        ev1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return ev0.elapsed_time(ev1) / steps, wall

    def time_kernel(self, kernel, launches):
        """Average duration (ms) of one kernel, bracketed by HIP events on its stream."""
        import torch

        from grouped_expert_ffn_amd import abi
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(launches)]
        for a, b in evs:  # torch creates the HIP events on first record
            a.record()
            b.record()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(evs):
            abi.moe_time_next_launch(kernel, a, b)
            self.step(i)
        torch.cuda.synchronize()
        ds = [a.elapsed_time(b) for a, b in evs]
        return sum(ds) / len(ds), min(ds)

    def free(self):
        import torch
        self.layers.clear()
        self.args.clear()
        torch.cuda.empty_cache()


def roofline_for(pt, work, kern_ms):
    if pt.T >= 512 and pt.wl.act == "bf16":
        achieved = work["gate_up_flops"] / (kern_ms * 1e-3) / 1e12
        return {"bound": "mfma", "kernel": "grouped gate/up + SwiGLU (MFMA)", "achieved": round(achieved, 1),
                "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFS, 4),
                "traffic": None, "flops_per_launch": work["gate_up_flops"],
                "avg_launch_ms": round(kern_ms, 5)}
    achieved = work["gate_up_bytes"] / (kern_ms * 1e-3) / 1e9
    return {"bound": "hbm", "kernel": "grouped gate/up + SwiGLU (GEMV)", "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None, "bytes_per_launch": work["gate_up_bytes"], "avg_launch_ms": round(kern_ms, 5)}


def measure(wl, T, steps, warmup, copies):
    import numpy as np

    from grouped_expert_ffn_amd import abi
    pt = Point(wl, T, copies)
    rel = pt.parity_gate()
    ids = pt.routing()
    n_touched = int(np.count_nonzero(np.bincount(ids.ravel(), minlength=wl.E)))
    work = layer_work(wl, T, n_touched)
    ms, wall = pt.time_steps(steps, warmup)
    launches = max(10, min(steps, 50))
    gu_ms, gu_min = pt.time_kernel(abi.MOE_KERNEL_GATE_UP, launches)
    dn_ms, _ = pt.time_kernel(abi.MOE_KERNEL_DOWN, launches)
    res = {
        "workload": wl.name, "tokens": T, "ms_per_layer": round(ms, 5),
        "tokens_per_s": round(T / (ms * 1e-3), 1),
        "layer_hbm_frac": round(work["layer_bytes"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "layer_mfma_frac": round(work["layer_flops"] / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS, 4),
        "gate_up_ms": round(gu_ms, 5), "down_ms": round(dn_ms, 5),
        "gate_up_hbm_frac": round(work["gate_up_bytes"] / (gu_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "down_hbm_frac": round(work["down_bytes"] / (dn_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "touched_experts": n_touched, "parity_rel_l2": float(f"{rel:.3e}"),
    }
    roof = roofline_for(pt, work, gu_ms)
    pt.free()
    return res, roof, ms, wall, work


def cpu_baseline(wl, T, budget_s):
    """The fp64 oracle as it stands, on a bounded sample of the same workload."""
    import numpy as np

    import moe_synth as S
    from oracle import moe_oracle as O
    host = host_layer(wl)
    x = S.make_tokens(wl, T)
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = 1
    done, passes = 0, 0
    t0 = time.perf_counter()
    while True:
        ex = O.Experts.from_layer(host)  # every pass widens the stored weights again
        for t in range(T):
            xt = x[t:t + 1]
            logits, ids, w = O.full_route(xt, host.w_router, host.bias, wl.k, wl.renormalize)
            O.moe_layer(xt, ex, ids, w, wl.S, wl.E)
            done += 1
            if time.perf_counter() - t0 > budget_s:
                break
        passes += 1
        if time.perf_counter() - t0 > budget_s * 0.66 or done >= 64 * T:
            break
    el = time.perf_counter() - t0
    return {"value": round(done / el, 3), "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{done} tokens of {wl.name} T={T} ({passes} pass(es), fp64 per-token "
                      f"per-expert loop incl. weight widening), {el:.1f} s"}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1 "
                          "(the path has no multi-GPU sharding or collectives)"}), flush=True)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    import moe_synth as S
    wl = S.WORKLOADS[args.workload]
    res, roof, ms, wall, work = measure(wl, args.tokens, args.steps, args.warmup, args.copies)
    sweep = []
    for item in [s for s in args.sweep.split(",") if s.strip()]:
        name, t = item.split(":")
        if name == wl.name and int(t) == args.tokens:
            continue
        r, rf, *_ = measure(S.WORKLOADS[name], int(t), args.sweep_steps, 3, args.copies)
        r["roofline_frac"] = rf["frac"]
        r["roofline_bound"] = rf["bound"]
        sweep.append(r)
        print(f"# sweep {name} T={t}: {r['ms_per_layer']:.4f} ms/layer, {r['tokens_per_s']:.0f} tok/s, "
              f"{rf['bound']} frac {rf['frac']:.3f}", file=sys.stderr, flush=True)
    cpu = None if args.no_cpu_baseline else cpu_baseline(wl, args.tokens, args.cpu_seconds)
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
        "sweep": sweep,
        "wall_s_timed": round(wall, 3),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
