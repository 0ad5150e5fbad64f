"""Seeded synthetic inputs for the MoE token-dispatch layer.

This module only *makes inputs*: random draws, bf16 round-to-nearest-even
storage and the per-output-channel int8 weight format.  It holds none of the
layer's arithmetic (no routing, no softmax, no expert FFN, no combine), so the
CPU oracle and the GPU path can both take their inputs from here without
sharing any of the method.

Workloads stand in for the models the source pages measure (dispatch README,
"Stack": DeepSeek-MoE-16B, shared + routed experts; switchyard page, hero:
OLMoE-1B-7B, 8 of 64 experts per token; switchyard §03 "Load balance": 2,048
tokens per GPU with the busiest expert at 4.0x the mean load).  Trained weights
and WikiText-2 are not used: every tensor is drawn from a seeded PCG64 stream.

Stream layout: tensor ``tag`` of expert ``e`` in layer ``l`` of workload
``cfg.cid`` draws from ``PCG64(SeedSequence([seed, cid, l, tag, e]))`` (``e`` is
0 for per-layer tensors), always in float32, then rounded to bf16 where the
workload is bf16.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Optional

import numpy as np

# tensor tags of the seed streams
TAG_X = 0
TAG_ROUTER = 1
TAG_RANKING = 2
TAG_GATE = 3
TAG_UP = 4
TAG_DOWN = 5
TAG_LOGITS = 6


# --------------------------------------------------------------------------
# storage formats
# --------------------------------------------------------------------------
def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even).

    Returns the 16-bit patterns as ``uint16``.  NaN stays a quiet NaN.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        r[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x0040)).astype(np.uint16)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (``uint16``) to float32 exactly."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def quantize_int8_rows(w: np.ndarray):
    """Symmetric int8 weight-only format, one fp32 scale per output channel.

    ``w`` is ``[..., out, in]`` float32 (already bf16-representable).  For each
    output channel ``n``: ``scale[n] = max_c |w[n, c]| / 127`` in fp32, and
    ``q[n, c] = clamp(rint(w[n, c] / scale[n]), -127, 127)`` with rint rounding
    half to even.  A channel that is all zero gets scale 0 and q 0.

    The format (int8 values + fp32 per-output-channel scales) is the one whose
    storage saving matches the 49.89% expert-memory reduction the dispatch
    README reports for its int8 weight-only kernel ("What has been measured",
    phase 5a); tests/golden/int8_memory_reduction.txt derives that figure.
    """
    w = np.asarray(w, dtype=np.float32)
    amax = np.max(np.abs(w), axis=-1)
    scale = (amax / np.float32(127.0)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    q = np.rint(w / safe[..., None]).astype(np.float32)
    q = np.clip(q, -127, 127).astype(np.int8)
    q[scale == 0] = 0
    return q, scale


# --------------------------------------------------------------------------
# workload descriptions
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    cid: int                 # stream id of the workload
    d: int                   # hidden size
    E: int                   # routed experts
    k: int                   # experts per token
    I: int                   # expert intermediate size
    S: int = 0               # always-on shared experts (intermediate I each)
    renormalize: bool = False
    act: str = "bf16"        # "f32" | "bf16"
    wdt: str = "bf16"        # "f32" | "bf16" | "i8"
    routing: str = "uniform"  # "uniform" | "zipf"
    router_std: float = 0.02
    zipf_alpha: float = 0.0
    w_std: float = 0.02
    n_layers: int = 1
    pre_norm: bool = False
    norm_eps: float = 1e-5
    tokens: tuple = (16,)


# Zipf exponent of the 16-layer prefill stack.  Written by
# oracle/tune_zipf_alpha.py (bisection on layer 0 of the stack with the
# oracle's routing) so that the busiest expert of layer 0 receives 4.0x the
# mean load; rerun that script if the stack's recipe changes.
STACK_ZIPF_ALPHA = 0.32421875  # busiest expert of layer 0: 4.0039x the mean

TINY_F32 = Workload("tiny_f32", 1, d=256, E=8, k=2, I=512, renormalize=True,
                    act="f32", wdt="f32", tokens=(16,))
OLMOE_BF16 = Workload("olmoe_bf16", 2, d=2048, E=64, k=8, I=1024,
                      tokens=(1, 8, 64))
DEEPSEEK_BF16 = Workload("deepseek_bf16", 3, d=2048, E=64, k=6, I=1408, S=2,
                         renormalize=True, routing="zipf",
                         router_std=2048 ** -0.5, zipf_alpha=1.2,
                         tokens=(1, 16, 128, 512, 2048))
OLMOE_I8 = Workload("olmoe_i8", 4, d=2048, E=64, k=8, I=1024, wdt="i8",
                    tokens=(1, 8, 64))
OLMOE_I8_ZIPF = dataclasses.replace(OLMOE_I8, name="olmoe_i8_zipf",
                                    routing="zipf", zipf_alpha=1.2)
DEEPSEEK_I8 = dataclasses.replace(DEEPSEEK_BF16, name="deepseek_i8", cid=6, wdt="i8")
OLMOE_STACK16 = Workload("olmoe_stack16", 5, d=2048, E=64, k=8, I=1024,
                         routing="zipf", zipf_alpha=STACK_ZIPF_ALPHA,
                         n_layers=16, pre_norm=True, norm_eps=1e-5,
                         tokens=(2048,))

WORKLOADS = {w.name: w for w in (TINY_F32, OLMOE_BF16, DEEPSEEK_BF16, OLMOE_I8,
                                  OLMOE_I8_ZIPF, DEEPSEEK_I8, OLMOE_STACK16)}


# --------------------------------------------------------------------------
# draws
# --------------------------------------------------------------------------
def _rng(seed: int, cid: int, layer: int, tag: int, sub: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, cid, layer, tag, sub])))


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _normal(seed, cid, layer, tag, sub, shape, std) -> np.ndarray:
    g = _rng(seed, cid, layer, tag, sub)
    a = g.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def _store(a: np.ndarray, dt: str) -> np.ndarray:
    """float32 draw -> stored array (float32, or bf16 bit patterns)."""
    if dt == "f32":
        return a
    return bf16_bits(a)


@dataclasses.dataclass
class Layer:
    """One MoE layer's weights in the layouts the C ABI takes.

    Matrices are ``[out, in]`` with ``in`` contiguous: ``w_router [E, d]``,
    ``w_gate``/``w_up`` ``[E+S, I, d]``, ``w_down [E+S, d, I]``; experts
    ``E..E+S-1`` are the shared ones.  bf16 arrays hold ``uint16`` bit
    patterns; int8 weights come with fp32 scales ``s_gate``/``s_up [E+S, I]``
    and ``s_down [E+S, d]``.
    """
    wl: Workload
    layer: int
    w_router: np.ndarray
    bias: Optional[np.ndarray]
    w_gate: np.ndarray
    w_up: np.ndarray
    w_down: np.ndarray
    s_gate: Optional[np.ndarray] = None
    s_up: Optional[np.ndarray] = None
    s_down: Optional[np.ndarray] = None


def zipf_bias(wl: Workload, seed: int, layer: int) -> np.ndarray:
    """Per-expert router bias ``alpha * ln(1/rank)`` over a seeded ranking.

    The ranking is a seeded random permutation of the routed experts; rank 1
    gets bias 0, rank E gets ``-alpha * ln(E)``.
    """
    g = _rng(seed, wl.cid, layer, TAG_RANKING)
    rank = g.permutation(wl.E) + 1
    return (np.float32(wl.zipf_alpha) * -np.log(rank.astype(np.float32))).astype(np.float32)


def make_layer(wl: Workload, layer: int = 0, seed: int = 0, threads: Optional[int] = None) -> Layer:
    """Draw one layer's router and expert weights.

    Expert ``e`` of each matrix draws from its own stream, so the draws run in
    parallel threads and any single expert can be redrawn on its own.
    """
    G = wl.E + wl.S
    wdt_store = "f32" if wl.wdt == "f32" else "bf16"
    w_router = _store(_normal(seed, wl.cid, layer, TAG_ROUTER, 0, (wl.E, wl.d), wl.router_std),
                      "f32" if wl.act == "f32" else "bf16")
    bias = zipf_bias(wl, seed, layer) if wl.routing == "zipf" else None

    def expert(e):
        g = _normal(seed, wl.cid, layer, TAG_GATE, e, (wl.I, wl.d), wl.w_std)
        u = _normal(seed, wl.cid, layer, TAG_UP, e, (wl.I, wl.d), wl.w_std)
        dn = _normal(seed, wl.cid, layer, TAG_DOWN, e, (wl.d, wl.I), wl.w_std)
        if wl.wdt == "i8":
            outs = []
            for a in (g, u, dn):
                q, s = quantize_int8_rows(bf16_bits_to_f32(bf16_bits(a)))
                outs.append((q, s))
            return outs
        return [(_store(a, wdt_store), None) for a in (g, u, dn)]

    with ThreadPoolExecutor(threads or _threads()) as ex:
        parts = list(ex.map(expert, range(G)))
    stack = lambda i: np.stack([p[i][0] for p in parts])  # noqa: E731
    out = Layer(wl, layer, w_router, bias, stack(0), stack(1), stack(2))
    if wl.wdt == "i8":
        out.s_gate = np.stack([p[0][1] for p in parts])
        out.s_up = np.stack([p[1][1] for p in parts])
        out.s_down = np.stack([p[2][1] for p in parts])
    return out


def make_tokens(wl: Workload, T: int, seed: int = 0, layer: int = 0) -> np.ndarray:
    """Input activations ``x [T, d]`` drawn from N(0, 1) (float32 or bf16 bits)."""
    a = _normal(seed, wl.cid, layer, TAG_X, T, (T, wl.d), 1.0)
    return _store(a, wl.act)


def make_logits(T: int, E: int, seed: int = 0, cid: int = 0) -> np.ndarray:
    """Router logits ``[T, E]`` drawn from N(0, 1), float32 (for the logits-input mode)."""
    return _normal(seed, cid, 0, TAG_LOGITS, T, (T, E), 1.0)


def stored_to_f32(a: np.ndarray) -> np.ndarray:
    """Stored array -> float32 (bf16 bit patterns are widened exactly)."""
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a)
    return np.asarray(a, dtype=np.float32)
