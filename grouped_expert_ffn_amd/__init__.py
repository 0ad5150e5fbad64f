"""MI355X (gfx950) MoE token-dispatch layer: HIP kernels behind a C ABI (libmoe.so).

``abi`` is the ctypes binding with the C entry points' names; ``DeviceLayer``
holds one layer's weights on the GPU and calls ``moe_forward``.  PyTorch is
used for device memory and streams only; every step of the layer runs in the
library's kernels.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from . import abi
from .abi import (MOE_BF16, MOE_F32, MOE_I8, MOE_WS_FORWARD, MOE_WS_GROUPED_FFN, MOE_WS_PERMUTE,
                  ExpertWeights, LayerDesc, MoeError, make_desc, make_weights, moe_combine,
                  moe_forward, moe_grouped_ffn, moe_permute, moe_route, moe_workspace_bytes)

DTYPES = {"f32": MOE_F32, "bf16": MOE_BF16, "i8": MOE_I8}


def to_device(a: Optional[np.ndarray], device="cuda"):
    """numpy array -> torch tensor on the GPU.  ``uint16`` arrays are bf16 bit patterns."""
    import torch
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def from_device(t) -> np.ndarray:
    """torch tensor -> numpy (bf16 comes back as ``uint16`` bit patterns)."""
    import torch
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def alloc_workspace(nbytes: int, device="cuda"):
    import torch
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


class DeviceLayer:
    """One MoE layer's weights on the GPU plus its descriptor.

    Weights are ``[out, in]`` arrays: ``w_router [E, d]``, ``w_gate``/``w_up``
    ``[E+S, I, d]``, ``w_down [E+S, d, I]`` (int8 with fp32 scales
    ``[E+S, I]``/``[E+S, d]``), as numpy arrays or GPU tensors.
    """

    def __init__(self, desc: LayerDesc, w_router, bias, w_gate, w_up, w_down,
                 s_gate=None, s_up=None, s_down=None, device="cuda"):
        conv = (lambda a: to_device(a, device) if isinstance(a, np.ndarray) else a)
        self.desc = desc
        self.w_router = conv(w_router)
        self.bias = conv(bias)
        self.w_gate, self.w_up, self.w_down = conv(w_gate), conv(w_up), conv(w_down)
        self.s_gate, self.s_up, self.s_down = conv(s_gate), conv(s_up), conv(s_down)
        self.weights = make_weights(self.w_gate, self.w_up, self.w_down,
                                    self.s_gate, self.s_up, self.s_down)
        self.device = device
        self._ws = None

    def workspace(self, T: int):
        need = moe_workspace_bytes(self.desc, T, MOE_WS_FORWARD)
        if need == 0:
            raise MoeError(abi.MOE_ERR_INVALID, "moe_workspace_bytes", abi.last_error())
        if self._ws is None or self._ws.numel() < need:
            self._ws = alloc_workspace(need, self.device)
        return self._ws

    def forward(self, x, residual=None, y=None, topk_ids=None, topk_w=None, stream=None):
        import torch
        T = x.shape[0]
        if y is None:
            y = torch.empty_like(x)
        ws = self.workspace(T)
        moe_forward(self.desc, T, x, self.w_router, self.bias, self.weights, residual, y,
                    topk_ids, topk_w, ws, ws.numel(), stream)
        return y


__all__ = ["abi", "DeviceLayer", "LayerDesc", "ExpertWeights", "MoeError", "make_desc",
           "make_weights", "moe_route", "moe_permute", "moe_grouped_ffn", "moe_combine",
           "moe_forward", "moe_workspace_bytes", "to_device", "from_device", "alloc_workspace",
           "MOE_F32", "MOE_BF16", "MOE_I8", "MOE_WS_PERMUTE", "MOE_WS_GROUPED_FFN",
           "MOE_WS_FORWARD", "DTYPES"]
