"""Device plumbing around the C ABI: upload a layer's tensors with torch, own
the packed weights and a workspace, call moe_layer_forward.

No arithmetic happens here; torch only provides device memory and streams.
"""
from __future__ import annotations

import numpy as np
import torch

from . import (MOE_BF16, MOE_F32, MOE_FP8, MOE_FP8A8, MOE_I4, MOE_I8A8, MOE_I8, MOE_MLP_RELU, MOE_MXFP4, MOE_SWIGLU, moe_layer_forward,
               moe_layer_graph_create, moe_weights_create, moe_weights_destroy, moe_weights_offload,
               moe_weights_set_tuning, moe_workspace_size)

DTYPE_CODE = {"f32": MOE_F32, "bf16": MOE_BF16, "i8": MOE_I8, "i4": MOE_I4, "fp8": MOE_FP8, "mxfp4": MOE_MXFP4,
              "fp8a8": MOE_FP8A8, "i8a8": MOE_I8A8}
KIND_CODE = {"relu": MOE_MLP_RELU, "swiglu": MOE_SWIGLU}


def to_device(a, device="cuda"):
    """numpy -> torch on the device; uint16 arrays are bf16 bit patterns."""
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


# Tuning fields (a dict of moe_tuning fields) applied to every MoELayer
# created while it is set; tests use it to force one launch form.
default_tuning: dict | None = None


class MoELayer:
    """One MoE layer resident on the GPU, built from a synthetic layer dict."""

    def __init__(self, layer: dict, device="cuda", stream=None, tuning: dict | None = None):
        sp = layer["spec"]
        self.spec = sp
        self.device = device
        self.T, self.m, self.p, self.E, self.k = sp.T, sp.m, sp.p, sp.E, sp.k
        self.x_dtype = DTYPE_CODE[sp.x_dtype]
        self.y_dtype = self.x_dtype
        self.x = to_device(layer["x"], device) if layer.get("x") is not None else None
        self.wg = to_device(layer["wg"], device)
        self.bias = to_device(layer["bias"], device)
        w1, w3, w2 = (to_device(layer[k], device) for k in ("w1", "w3", "w2"))
        s1, s3, s2 = (to_device(layer[k], device) for k in ("s1", "s3", "s2"))
        self.handle = moe_weights_create(self.m, self.p, self.E, KIND_CODE[sp.kind], DTYPE_CODE[sp.w_dtype],
                                         w1, w3, w2, s1, s3, s2, stream=stream)
        del w1, w3, w2, s1, s3, s2
        tuning = default_tuning if tuning is None else tuning
        if tuning:
            moe_weights_set_tuning(self.handle, tuning)
        self._ws = None
        self._ws_T = -1
        self.ensure_workspace(self.T)

    def offload(self, slots: int):
        """Move the experts to host memory with `slots` device cache slots (moe_weights_offload)."""
        moe_weights_offload(self.handle, slots)

    def set_tuning(self, tuning: dict | None):
        """Attach moe_tuning fields to the handle (None: automatic) and resize the workspace."""
        moe_weights_set_tuning(self.handle, tuning)
        T = max(self._ws_T, self.T)
        self._ws_T = -1
        self.ensure_workspace(T)

    def ensure_workspace(self, T):
        if T > self._ws_T:
            self.ws_bytes = moe_workspace_size(self.handle, T, self.k)
            self._ws = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=self.device)
            self._ws_T = T
        return self._ws

    def new_output(self, T=None):
        T = self.T if T is None else T
        dt = torch.float32 if self.y_dtype == MOE_F32 else torch.bfloat16
        return torch.empty((T, self.m), dtype=dt, device=self.device)

    def forward(self, x=None, y=None, T=None, dbg=None, stream=None):
        x = self.x if x is None else x
        T = x.shape[0] if T is None else T
        y = self.new_output(T) if y is None else y
        ws = self.ensure_workspace(T)
        dbg = dbg or {}
        moe_layer_forward(self.handle, self.wg, self.bias, x, self.x_dtype, T, self.m, self.p, self.E, self.k, y,
                          self.y_dtype, ws, self.ws_bytes, dbg.get("topk_idx"), dbg.get("topk_w"),
                          dbg.get("logits"), dbg.get("counts"), dbg.get("offsets"), dbg.get("perm"), stream=stream)
        return y

    def capture(self, x=None, y=None, T=None):
        """The forward into y captured as a HIP graph (moe_layer_graph_create);
        returns (graph handle, y).  Replay with moe_graph_launch, free with
        moe_graph_destroy; x, y and the workspace must stay alive meanwhile."""
        x = self.x if x is None else x
        T = x.shape[0] if T is None else T
        y = self.new_output(T) if y is None else y
        ws = self.ensure_workspace(T)
        g = moe_layer_graph_create(self.handle, self.wg, self.bias, x, self.x_dtype, T, self.m, self.p, self.E,
                                   self.k, y, self.y_dtype, ws, self.ws_bytes)
        return g, y

    def debug_buffers(self, T=None):
        T = self.T if T is None else T
        d = self.device
        return {
            "topk_idx": torch.empty((T, self.k), dtype=torch.int32, device=d),
            "topk_w": torch.empty((T, self.k), dtype=torch.float32, device=d),
            "logits": torch.empty((T, self.E), dtype=torch.float32, device=d),
            "counts": torch.empty(self.E, dtype=torch.int32, device=d),
            "offsets": torch.empty(self.E + 1, dtype=torch.int32, device=d),
            "perm": torch.empty(T * self.k, dtype=torch.int32, device=d),
        }

    def close(self):
        if self.handle is not None:
            moe_weights_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
