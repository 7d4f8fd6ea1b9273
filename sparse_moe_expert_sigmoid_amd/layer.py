"""Device buffers for one MoE layer and the three-call sequence route -> build -> forward.

Marshalling only: every step of the layer runs in the HIP library.
"""
from __future__ import annotations

import numpy as np
import torch

from . import abi

WEIGHT_KEYS = ("w13_qs", "w13_sc", "w2_qs", "w2_sc", "s13_qs", "s13_sc", "s2_qs", "s2_sc")


def to_device(a: np.ndarray, device) -> torch.Tensor:
    """numpy -> torch on `device`; uint16 bit patterns travel as int16 (same bytes)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


class DeviceWeights(dict):
    """The router and expert arrays of one layer, resident on the GPU."""

    @classmethod
    def upload(cls, inp: dict, device="cuda") -> "DeviceWeights":
        w = cls()
        w.dims = inp["dims"]
        w["w_router"] = to_device(inp["w_router"], device)
        w["bias"] = to_device(inp["bias"], device)
        # row-major Q4 arrays go up as they are; the library regroups them on the device (moe_q4_pack)
        for name in ("w13", "w2", "s13", "s2"):
            qs, sc = inp[name + "_qs"], inp[name + "_sc"]
            n_mats = qs.shape[0] if qs.ndim == 3 else 1
            rows, K = qs.shape[-2], 2 * qs.shape[-1]
            qs_in, sc_in = to_device(qs, device), to_device(sc, device)
            w[name + "_qs"] = torch.empty_like(qs_in)
            w[name + "_sc"] = torch.empty_like(sc_in)
            abi.moe_q4_pack(n_mats, rows, K, qs_in, sc_in, w[name + "_qs"], w[name + "_sc"],
                            stream=torch.cuda.current_stream(qs_in.device))
        return w


class Workspace:
    """Outputs and caller-owned workspaces for a layer call of a given shape and flags."""

    def __init__(self, dims, flags: int = 0, device="cuda"):
        self.dims = dims
        self.flags = flags
        rc = abi.moe_supports(dims, flags)
        if rc != abi.MOE_OK:
            raise abi.MoeError(rc, "moe_supports")
        T, k, d = dims.T, dims.k, dims.d
        self.routing = torch.zeros(abi.moe_routing_bytes(dims, flags), dtype=torch.uint8, device=device)
        self.scratch = torch.empty(max(abi.moe_scratch_bytes(dims, flags), 256), dtype=torch.uint8, device=device)
        self.topk_ids = torch.empty((T, k), dtype=torch.int32, device=device)
        self.topk_w = torch.empty((T, k), dtype=torch.float32, device=device)
        self.y = torch.empty((T, d), dtype=torch.float32, device=device)
        self.layout = abi.moe_routing_layout_of(dims, flags)

    def routing_view(self, name: str, count: int, dtype=torch.int32) -> torch.Tensor:
        off = self.layout[name]
        nbytes = count * torch.tensor([], dtype=dtype).element_size()
        return self.routing[off:off + nbytes].view(dtype)


def layer_call(x: torch.Tensor, w: DeviceWeights, ws: Workspace, stream=None, residual=None) -> torch.Tensor:
    """Enqueue route, build and forward for tokens x (bf16 bits as int16 [T][d]); returns ws.y.
    With `residual` (fp32 [T][d] on the device, may be ws.y) the forward adds it after routed + shared."""
    dims, f = ws.dims, ws.flags
    abi.moe_route(dims, x, w["w_router"], w["bias"], ws.topk_ids, ws.topk_w, ws.routing, flags=f, stream=stream)
    abi.moe_build_descriptors(dims, ws.topk_ids, ws.routing, flags=f, stream=stream)
    if residual is None:
        abi.moe_q4_forward(dims, x, ws.topk_ids, ws.topk_w, ws.routing, w, ws.y, ws.scratch, flags=f, stream=stream)
    else:
        abi.moe_q4_forward_residual(dims, x, ws.topk_ids, ws.topk_w, ws.routing, w, residual, ws.y, ws.scratch,
                                    flags=f, stream=stream)
    return ws.y


def layer_call_fused(x: torch.Tensor, w: DeviceWeights, ws: Workspace, stream=None, residual=None) -> torch.Tensor:
    """The same layer through the single entry point moe_layer_forward (same results); returns ws.y."""
    abi.moe_layer_forward(ws.dims, x, w["w_router"], w["bias"], w, ws.y, ws.topk_ids, ws.topk_w, ws.routing,
                          ws.scratch, residual=residual, flags=ws.flags, stream=stream)
    return ws.y


class DecodeContext:
    """A stack of MoE layers recorded once into a HIP graph by the library (moe_decode_ctx_*):
    every run() passes the residual stream h (fp32 [T][d], updated in place) through all layers,
    x = bf16(h), h = layer(x) + h.  Holds the device buffers the context's graph addresses."""

    def __init__(self, dims, layers: list, h: torch.Tensor, flags: int = 0):
        self.dims, self.flags, self.layers, self.h = dims, flags, layers, h
        self.workspace = torch.zeros(max(abi.moe_decode_ctx_workspace_bytes(dims, flags), 256), dtype=torch.uint8,
                                     device=h.device)
        self.ctx = abi.moe_decode_ctx_create(dims, layers, h, self.workspace, flags=flags)

    def run(self, stream=None) -> torch.Tensor:
        abi.moe_decode_ctx_run(self.ctx, stream)
        return self.h

    def close(self) -> None:
        if self.ctx:
            abi.moe_decode_ctx_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
