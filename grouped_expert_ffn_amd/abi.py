"""ctypes binding of libmoe.so: the C entry points under the same names.

Argument marshalling only.  Array arguments may be ``torch`` tensors (their
``data_ptr()`` is passed; they must live on the GPU), raw integer device
addresses, or ``None`` for NULL.  ``stream`` defaults to torch's current HIP
stream.  A negative status raises :class:`MoeError` with the library's message.
There is no fallback: if libmoe.so is missing or does not load, every call
raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

MOE_OK, MOE_ERR_INVALID, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_DEVICE = 0, -1, -2, -3, -4
MOE_F32, MOE_BF16, MOE_I8 = 0, 1, 2
MOE_WS_PERMUTE, MOE_WS_GROUPED_FFN, MOE_WS_FORWARD = 0, 1, 2

EXPORTS = ("moe_workspace_bytes", "moe_route", "moe_permute", "moe_grouped_ffn", "moe_combine",
           "moe_forward", "moe_forward_noalloc", "moe_time_next_launch", "moe_ffn_kernel", "moe_status_str",
           "moe_last_error", "moe_version")
(MOE_KERNEL_RMSNORM, MOE_KERNEL_ROUTER, MOE_KERNEL_TOPK, MOE_KERNEL_PERMUTE, MOE_KERNEL_GATE_UP,
 MOE_KERNEL_DOWN, MOE_KERNEL_COMBINE) = range(7)
MOE_FFN_GEMV, MOE_FFN_GEMV_MFMA, MOE_FFN_GEMM = range(3)


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        super().__init__(f"{where}: {status_str(status)}: {message}")
        self.status = status


class LayerDesc(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("n_shared", ctypes.c_int32), ("renormalize", ctypes.c_int32),
                ("act_dtype", ctypes.c_int32), ("w_dtype", ctypes.c_int32),
                ("pre_norm", ctypes.c_int32), ("norm_eps", ctypes.c_float),
                ("capacity_factor", ctypes.c_float)]


class ExpertWeights(ctypes.Structure):
    _fields_ = [("w_gate", ctypes.c_void_p), ("w_up", ctypes.c_void_p),
                ("w_down", ctypes.c_void_p), ("s_gate", ctypes.c_void_p),
                ("s_up", ctypes.c_void_p), ("s_down", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmoe.so (raises if it has not been built or does not load)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m grouped_expert_ffn_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        D = ctypes.POINTER(LayerDesc)
        W = ctypes.POINTER(ExpertWeights)
        sig = {
            "moe_workspace_bytes": (sz, [D, i32, i32]),
            "moe_route": (i32, [D, i32, vp, vp, vp, vp, vp, vp, vp, vp]),
            "moe_permute": (i32, [D, i32, vp, vp, vp, vp, vp, vp, sz, vp]),
            "moe_grouped_ffn": (i32, [D, i32, vp, W, vp, vp, vp, vp, vp, sz, vp]),
            "moe_combine": (i32, [D, i32, vp, vp, vp, vp, vp, vp]),
            "moe_forward": (i32, [D, i32, vp, vp, vp, W, vp, vp, vp, vp, vp, sz, vp]),
            "moe_forward_noalloc": (i32, [D, i32, vp, vp, vp, W, vp, vp, vp, vp, vp]),
            "moe_time_next_launch": (i32, [i32, vp, vp]),
            "moe_ffn_kernel": (i32, [D, i32]),
            "moe_status_str": (ctypes.c_char_p, [i32]),
            "moe_last_error": (ctypes.c_char_p, []),
            "moe_version": (i32, []),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().moe_status_str(status).decode()


def last_error() -> str:
    return lib().moe_last_error().decode()


def _ptr(a) -> Optional[int]:
    if a is None:
        return None
    if isinstance(a, int):
        return a or None
    if hasattr(a, "data_ptr"):
        if not a.is_cuda:
            raise ValueError("tensor arguments must be on the GPU")
        return a.data_ptr()
    raise TypeError(f"cannot pass {type(a).__name__} as a device pointer")


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream or None
    if isinstance(stream, int):
        return stream or None
    return stream.cuda_stream or None


def _check(status: int, where: str) -> None:
    if status != MOE_OK:
        raise MoeError(status, where, last_error())


def make_desc(d_model, n_experts, top_k, d_ff, n_shared=0, renormalize=False,
              act_dtype=MOE_BF16, w_dtype=None, pre_norm=False, norm_eps=1e-5,
              capacity_factor=0.0) -> LayerDesc:
    return LayerDesc(d_model, n_experts, top_k, d_ff, n_shared, int(bool(renormalize)), act_dtype,
                     act_dtype if w_dtype is None else w_dtype, int(bool(pre_norm)), norm_eps,
                     capacity_factor)


def make_weights(w_gate, w_up, w_down, s_gate=None, s_up=None, s_down=None) -> ExpertWeights:
    return ExpertWeights(_ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(s_gate), _ptr(s_up),
                         _ptr(s_down))


def moe_workspace_bytes(desc: LayerDesc, max_tokens: int, which: int) -> int:
    return int(lib().moe_workspace_bytes(ctypes.byref(desc), max_tokens, which))


def moe_route(desc, T, x, w_router, router_bias, logits_in, logits_out, topk_ids, topk_w,
              stream=None) -> None:
    _check(lib().moe_route(ctypes.byref(desc), T, _ptr(x), _ptr(w_router), _ptr(router_bias),
                           _ptr(logits_in), _ptr(logits_out), _ptr(topk_ids), _ptr(topk_w),
                           _stream(stream)), "moe_route")


def moe_permute(desc, T, topk_ids, counts, offsets, perm, inv_perm, plan, plan_bytes,
                stream=None) -> None:
    _check(lib().moe_permute(ctypes.byref(desc), T, _ptr(topk_ids), _ptr(counts), _ptr(offsets),
                             _ptr(perm), _ptr(inv_perm), _ptr(plan), plan_bytes,
                             _stream(stream)), "moe_permute")


def moe_grouped_ffn(desc, T, x, weights: ExpertWeights, offsets, perm, plan, rows, ws, ws_bytes,
                    stream=None) -> None:
    _check(lib().moe_grouped_ffn(ctypes.byref(desc), T, _ptr(x), ctypes.byref(weights),
                                 _ptr(offsets), _ptr(perm), _ptr(plan), _ptr(rows), _ptr(ws),
                                 ws_bytes, _stream(stream)), "moe_grouped_ffn")


def moe_combine(desc, T, rows, inv_perm, topk_w, residual, y, stream=None) -> None:
    _check(lib().moe_combine(ctypes.byref(desc), T, _ptr(rows), _ptr(inv_perm), _ptr(topk_w),
                             _ptr(residual), _ptr(y), _stream(stream)), "moe_combine")


def moe_forward(desc, T, x, w_router, router_bias, weights: ExpertWeights, residual, y,
                topk_ids_out, topk_w_out, ws, ws_bytes, stream=None) -> None:
    _check(lib().moe_forward(ctypes.byref(desc), T, _ptr(x), _ptr(w_router), _ptr(router_bias),
                             ctypes.byref(weights), _ptr(residual), _ptr(y), _ptr(topk_ids_out),
                             _ptr(topk_w_out), _ptr(ws), ws_bytes, _stream(stream)),
           "moe_forward")


def moe_forward_noalloc(desc, T, x, w_router, router_bias, weights: ExpertWeights, residual, y,
                        topk_ids_out, topk_w_out, stream=None) -> None:
    _check(lib().moe_forward_noalloc(ctypes.byref(desc), T, _ptr(x), _ptr(w_router),
                                     _ptr(router_bias), ctypes.byref(weights), _ptr(residual),
                                     _ptr(y), _ptr(topk_ids_out), _ptr(topk_w_out),
                                     _stream(stream)), "moe_forward_noalloc")


def moe_ffn_kernel(desc: LayerDesc, T: int) -> int:
    """The kernel family (MOE_FFN_*) the grouped FFN launches for T tokens; host-only."""
    r = int(lib().moe_ffn_kernel(ctypes.byref(desc), T))
    if r < 0:
        _check(r, "moe_ffn_kernel")
    return r


def moe_time_next_launch(kernel: int, start_event, stop_event) -> None:
    """Arm the one-shot timing hook with two ``torch.cuda.Event(enable_timing=True)``
    (or raw hipEvent_t addresses, or None to disarm)."""
    ev = lambda e: None if e is None else (e if isinstance(e, int) else e.cuda_event)  # noqa: E731
    _check(lib().moe_time_next_launch(kernel, ev(start_event), ev(stop_event)),
           "moe_time_next_launch")
