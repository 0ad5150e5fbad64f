"""CPU oracle of one MoE layer's token-dispatch path, in float64.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library or its binding; both sides only take their inputs from ``moe_synth``.

It is deliberately plain and slow: a per-token, per-expert loop with NumPy's
matrix-vector product as the only library primitive.  Every input arrives in
its stored form (float32, bf16 bit patterns, or int8 + fp32 scales) and is
widened exactly to float64 before any arithmetic; nothing is rounded on the
way, so the oracle is the exact answer up to float64 rounding order.

What the layer computes, from the pages:

* routing -- each token is sent to ``k`` of ``E`` experts by top-k gating
  (dispatch README, intro and "Why this project"; switchyard page, hero:
  OLMoE routes each token to 8 of its 64 experts, and §02 "Route and sort");
* the rows routed to an expert are grouped together, sorted by expert
  (switchyard §02 "Route and sort");
* each expert is a SwiGLU feed-forward block (switchyard §02 "One launch for
  all experts"; "What switchyard adds", item 1);
* the expert outputs are combined back per token, weighted by the gate, with a
  unique answer that does not depend on where the experts ran (switchyard hero,
  statistics: expert-parallel output equal to one GPU bit for bit, and §02
  "Kernels and dispatch": no atomics);
* DeepSeek-style layers add always-on shared experts to the routed ones
  (dispatch README, "Stack");
* int8 weight-only experts are per-channel quantised and dequantised inside
  the kernel (dispatch README, "What has been measured", phase 5a);
* no token is dropped by default (switchyard §03 "Load balance": dropless);
  as an option, a capacity limit drops the rows an expert has no room for
  (the same section, "What dropping tokens costs": capacity factors 2.0 and
  1.0 against dropless).

Readings taken where the pages are silent:
softmax over all E logits, then top-k, then optional renormalisation; the
selection is made on the logits (softmax is strictly increasing, so this is
the same set), largest first, equal logits going to the lower expert id, NaN
ranking below every number; shared experts carry weight 1 and come after the
routed slots; the RMSNorm of the stacked workload has no learned scale; with a
capacity factor cf each routed expert keeps ceil(cf*T*k/E) rows, the earliest
(token, slot) pairs in flat order t*k+j, a dropped pair contributes nothing
(the remaining gate weights are not rescaled) and shared experts never drop.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np


# --------------------------------------------------------------------------
# decoding of stored inputs (exact widening to float64)
# --------------------------------------------------------------------------
def widen(a: np.ndarray) -> np.ndarray:
    """Stored array -> float64.  ``uint16`` arrays are bf16 bit patterns."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        f32 = (a.astype(np.uint32) << np.uint32(16)).view(np.float32)
        return f32.astype(np.float64)
    return a.astype(np.float64)


def dequantize(q: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """int8 weight-only format: ``w[n, c] = q[n, c] * scale[n]`` (scale per output channel)."""
    return np.asarray(q, dtype=np.float64) * np.asarray(scale, dtype=np.float64)[..., None]


# --------------------------------------------------------------------------
# step 1: router
# --------------------------------------------------------------------------
def router_logits(x: np.ndarray, w_router: np.ndarray, bias: Optional[np.ndarray] = None) -> np.ndarray:
    """``l[t, e] = sum_c x[t, c] * W_r[e, c] + b[e]`` in float64.

    ``W_r`` is stored ``[E, d]`` (one row per expert).
    """
    xf = widen(x)
    wf = widen(w_router)
    T, E = xf.shape[0], wf.shape[0]
    out = np.empty((T, E), dtype=np.float64)
    for t in range(T):
        out[t] = wf @ xf[t]
    if bias is not None:
        out += widen(bias)[None, :]
    return out


def _rank_key(value: float, e: int):
    """Total order used by the selection: larger value first, NaN last, lower id on ties."""
    if math.isnan(value):
        return (1, 0.0, e)
    return (0, -value, e)


def select_experts(logits_row: Sequence[float], k: int) -> list:
    """The k experts with the largest logits, largest first.

    Equal logits (IEEE equality, so -0.0 equals +0.0) go to the lower expert
    id; NaN ranks below every number, NaNs among themselves by id.
    """
    order = sorted(range(len(logits_row)), key=lambda e: _rank_key(float(logits_row[e]), e))
    return order[:k]


def softmax_row(logits_row: np.ndarray) -> np.ndarray:
    """``p_e = exp(l_e - m) / sum_e' exp(l_e' - m)`` with ``m = max_e l_e``."""
    l = np.asarray(logits_row, dtype=np.float64)
    m = np.max(l)
    z = np.exp(l - m)
    return z / np.sum(z)


def route(logits: np.ndarray, k: int, renormalize: bool):
    """Top-k gating of every token.

    Returns ``ids [T, k]`` (int64, slot order = selection order) and the gate
    weights ``w [T, k]`` (float64): the softmax probability over all E experts
    of each chosen expert, divided by their sum over the k slots when
    ``renormalize`` is set.
    """
    logits = np.asarray(logits, dtype=np.float64)
    T = logits.shape[0]
    ids = np.empty((T, k), dtype=np.int64)
    w = np.empty((T, k), dtype=np.float64)
    for t in range(T):
        chosen = select_experts(logits[t], k)
        p = softmax_row(logits[t])
        wt = np.array([p[e] for e in chosen], dtype=np.float64)
        if renormalize:
            wt = wt / np.sum(wt)
        ids[t] = chosen
        w[t] = wt
    return ids, w


def gate_weights_for(logits: np.ndarray, ids: np.ndarray, renormalize: bool) -> np.ndarray:
    """Gate weights of a given expert choice (used when the choice comes from elsewhere)."""
    logits = np.asarray(logits, dtype=np.float64)
    T, k = ids.shape
    w = np.empty((T, k), dtype=np.float64)
    for t in range(T):
        p = softmax_row(logits[t])
        wt = np.array([p[int(e)] for e in ids[t]], dtype=np.float64)
        if renormalize:
            wt = wt / np.sum(wt)
        w[t] = wt
    return w


# --------------------------------------------------------------------------
# step 2: sort of token rows by expert
# --------------------------------------------------------------------------
def permute(ids: np.ndarray, n_experts: int):
    """Group the ``T*k`` (token, slot) rows by expert.

    Flat index ``f = t*k + j``.  Returns
    ``counts[e]`` = rows routed to expert e,
    ``offsets`` = exclusive prefix sum of counts (E+1 entries),
    ``perm[r]`` = flat index of sorted row r (a stable sort on the expert id,
    so rows of one expert keep ascending token order), and
    ``inv_perm[f]`` = the sorted position of flat index f.
    """
    flat = np.asarray(ids, dtype=np.int64).ravel()
    counts = np.bincount(flat, minlength=n_experts).astype(np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    perm = np.argsort(flat, kind="stable").astype(np.int64)
    inv_perm = np.empty_like(perm)
    inv_perm[perm] = np.arange(perm.size, dtype=np.int64)
    return counts, offsets, perm, inv_perm


# --------------------------------------------------------------------------
# option: capacity-factor dropping (switchyard §03 "Load balance", "What
# dropping tokens costs")
# --------------------------------------------------------------------------
def capacity(capacity_factor: float, T: int, k: int, n_experts: int) -> int:
    """Rows each routed expert may keep: ``ceil(cf * T * k / E)``; 0 = no limit.

    The factor is taken as the float32 value the library receives, and the
    product is formed in double precision in the order ((cf * T) * k) / E."""
    cf = float(np.float32(capacity_factor))
    if not cf > 0.0:
        return 0
    return int(math.ceil(cf * T * k / n_experts))


def kept_slots(ids: np.ndarray, n_experts: int, cap: int) -> np.ndarray:
    """``keep[t, j]``: whether slot j of token t finds room in its expert.

    The (token, slot) pairs are visited in flat order ``t*k + j`` and each
    expert accepts the first ``cap`` pairs that reach it (no limit if cap is 0).
    """
    ids = np.asarray(ids)
    T, k = ids.shape
    keep = np.ones((T, k), dtype=bool)
    if cap <= 0:
        return keep
    seen = [0] * n_experts
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            keep[t, j] = seen[e] < cap
            seen[e] += 1
    return keep


def permute_with_capacity(ids: np.ndarray, n_experts: int, cap: int):
    """``permute`` of all rows, with ``inv_perm[f] = -1`` for every dropped pair.

    Dropped pairs keep their place in the sort (they are the tail of their
    expert's segment), so counts, offsets and perm are those of ``permute``."""
    counts, offsets, perm, inv_perm = permute(ids, n_experts)
    keep = kept_slots(ids, n_experts, cap).ravel()
    inv_perm = np.where(keep, inv_perm, -1)
    return counts, offsets, perm, inv_perm


# --------------------------------------------------------------------------
# step 3/4: the expert feed-forward block
# --------------------------------------------------------------------------
def silu(z: np.ndarray) -> np.ndarray:
    """``silu(z) = z / (1 + exp(-z))``."""
    return z / (1.0 + np.exp(-z))


class Experts:
    """Expert weights of one layer, widened to float64 one expert at a time.

    ``w_gate``/``w_up`` are ``[G, I, d]`` and ``w_down`` is ``[G, d, I]``
    (``G = E + S``, output rows, input contiguous); with int8 storage the
    per-output-channel scales multiply each row.
    """

    def __init__(self, w_gate, w_up, w_down, s_gate=None, s_up=None, s_down=None):
        self.w_gate, self.w_up, self.w_down = w_gate, w_up, w_down
        self.s_gate, self.s_up, self.s_down = s_gate, s_up, s_down
        self._cache = {}

    @classmethod
    def from_layer(cls, layer) -> "Experts":
        return cls(layer.w_gate, layer.w_up, layer.w_down, layer.s_gate, layer.s_up, layer.s_down)

    def get(self, e: int):
        if e not in self._cache:
            if self.s_gate is not None:
                wg = dequantize(self.w_gate[e], self.s_gate[e])
                wu = dequantize(self.w_up[e], self.s_up[e])
                wd = dequantize(self.w_down[e], self.s_down[e])
            else:
                wg, wu, wd = widen(self.w_gate[e]), widen(self.w_up[e]), widen(self.w_down[e])
            self._cache[e] = (wg, wu, wd)
        return self._cache[e]


def expert_ffn(x_t: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray):
    """SwiGLU block for one token: ``W_down (silu(W_gate x) * (W_up x))``.

    Returns the output ``o [d]`` and the intermediate ``h [I]``.
    """
    g = wg @ x_t
    u = wu @ x_t
    h = silu(g) * u
    return wd @ h, h


# --------------------------------------------------------------------------
# the layer, written as the plain per-token, per-expert loop
# --------------------------------------------------------------------------
def moe_layer(x: np.ndarray, experts: Experts, ids: np.ndarray, w: np.ndarray,
              n_shared: int, n_experts: int, residual: Optional[np.ndarray] = None,
              tokens: Optional[Sequence[int]] = None,
              keep: Optional[np.ndarray] = None) -> np.ndarray:
    """``y[t] = sum_j w[t,j] FFN_{ids[t,j]}(x_t) + sum_s FFN_{E+s}(x_t) (+ residual[t])``.

    ``tokens`` restricts the loop to a subset of tokens (rows of the result
    follow that subset's order).  ``keep[t, j]`` False drops slot j of token t
    (the capacity option); the sum then skips it.
    """
    xf = widen(x)
    T = xf.shape[0]
    sel = range(T) if tokens is None else list(tokens)
    res = None if residual is None else widen(residual)
    out = np.zeros((len(sel), xf.shape[1]), dtype=np.float64)
    for i, t in enumerate(sel):
        acc = np.zeros(xf.shape[1], dtype=np.float64)
        for j in range(ids.shape[1]):
            if keep is not None and not keep[t, j]:
                continue
            o, _ = expert_ffn(xf[t], *experts.get(int(ids[t, j])))
            acc += w[t, j] * o
        for s in range(n_shared):
            o, _ = expert_ffn(xf[t], *experts.get(n_experts + s))
            acc += o
        if res is not None:
            acc += res[t]
        out[i] = acc
    return out


def moe_layer_dense(x: np.ndarray, experts: Experts, ids: np.ndarray, w: np.ndarray,
                    n_shared: int, n_experts: int, residual: Optional[np.ndarray] = None) -> np.ndarray:
    """Second formulation of the same layer: every token through every expert.

    ``y = sum_e G[:, e] * FFN_e(x)`` with the gate matrix ``G [T, E]`` equal to
    the gate weight where the expert was chosen and zero elsewhere, plus the
    shared experts with gate 1.  Used only to cross-check ``moe_layer``.
    """
    xf = widen(x)
    T, d = xf.shape
    G = np.zeros((T, n_experts), dtype=np.float64)
    for t in range(T):
        for j in range(ids.shape[1]):
            G[t, int(ids[t, j])] += w[t, j]
    y = np.zeros((T, d), dtype=np.float64)
    for e in range(n_experts + n_shared):
        wg, wu, wd = experts.get(e)
        gate = np.ones(T) if e >= n_experts else G[:, e]
        H = silu(xf @ wg.T) * (xf @ wu.T)
        y += gate[:, None] * (H @ wd.T)
    if residual is not None:
        y += widen(residual)
    return y


def sorted_rows(x: np.ndarray, experts: Experts, ids: np.ndarray, perm: np.ndarray,
                n_shared: int, n_experts: int, rows: Optional[Sequence[int]] = None):
    """Expert outputs in sorted-row order (the grouped FFN's result).

    Row ``r < T*k`` belongs to flat index ``f = perm[r]`` (token ``f // k``,
    expert ``ids.flat[f]``); row ``T*k + s*T + t`` is shared expert ``s`` on
    token ``t``.  Returns ``(h, out)`` for the requested rows: the SwiGLU
    intermediate ``h [n, I]`` and the expert output ``out [n, d]``.
    """
    xf = widen(x)
    T, k = ids.shape
    R = T * k + n_shared * T
    sel = range(R) if rows is None else list(rows)
    hs, outs = [], []
    flat = np.asarray(ids).ravel()
    for r in sel:
        if r < T * k:
            f = int(perm[r])
            t, e = f // k, int(flat[f])
        else:
            s, t = divmod(r - T * k, T)
            e = n_experts + s
        o, h = expert_ffn(xf[t], *experts.get(e))
        hs.append(h)
        outs.append(o)
    return np.array(hs), np.array(outs)


def combine(rows: np.ndarray, inv_perm: np.ndarray, w: np.ndarray, n_shared: int,
            residual: Optional[np.ndarray] = None) -> np.ndarray:
    """``y[t] = sum_j w[t,j] rows[inv_perm[t*k+j]] + sum_s rows[T*k + s*T + t] (+ residual[t])``.

    A pair with ``inv_perm < 0`` was dropped by the capacity option and adds nothing."""
    rf = widen(rows)
    T, k = w.shape
    out = np.zeros((T, rf.shape[1]), dtype=np.float64)
    res = None if residual is None else widen(residual)
    for t in range(T):
        acc = np.zeros(rf.shape[1], dtype=np.float64)
        for j in range(k):
            r = int(inv_perm[t * k + j])
            if r >= 0:
                acc += w[t, j] * rf[r]
        for s in range(n_shared):
            acc += rf[T * k + s * T + t]
        if res is not None:
            acc += res[t]
        out[t] = acc
    return out


# --------------------------------------------------------------------------
# stacked workload: RMSNorm before each layer, residual after
# --------------------------------------------------------------------------
def rmsnorm(h: np.ndarray, eps: float) -> np.ndarray:
    """``h / sqrt(mean_c h_c^2 + eps)`` per token (no learned scale)."""
    hf = widen(h)
    return hf / np.sqrt(np.mean(hf * hf, axis=-1, keepdims=True) + eps)


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Nearest bf16 value (ties to even) of float64 values, returned as float64.

    Rounds the float64 significand directly to 8 bits (no float32 step)."""
    a = np.asarray(a, dtype=np.float64)
    m, e = np.frexp(a)                     # a = m * 2**e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 256.0), e - 8)  # rint: half to even


def stack_layer_input(h: np.ndarray, eps: float) -> np.ndarray:
    """Input of one layer of the stacked workload: RMSNorm of the residual stream,
    stored in bf16 like every activation of a bf16 layer."""
    return round_to_bf16(rmsnorm(h, eps))


def full_route(x: np.ndarray, w_router: np.ndarray, bias, k: int, renormalize: bool):
    """Router logits, then top-k gating (steps 1-2 end to end)."""
    logits = router_logits(x, w_router, bias)
    ids, w = route(logits, k, renormalize)
    return logits, ids, w
