"""Device residency of one MoE layer: pack planar MXFP4 experts into blobs
(the library's layout) and move router, norm and blobs to HBM."""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import MoeShape, moe_pack_experts, moe_workspace_bytes


@dataclass
class DeviceLayer:
    router_w: "object"            # [E, H] float32
    router_b: "object"            # [E] float32
    experts: "object"             # uint8 [copies, E * stride]
    shared: "object | None"       # uint8 [copies, n_shared * stride] or None
    norm_w: "object | None"       # [H] float32 or None

    def experts_copy(self, c: int):
        return self.experts[c % self.experts.shape[0]]

    def shared_copy(self, c: int):
        return None if self.shared is None else self.shared[c % self.shared.shape[0]]


def upload_layer(shape: MoeShape, layer, device="cuda", copies: int = 1) -> DeviceLayer:
    """`layer` has router_w, router_b, experts, shared and norm_w (numpy);
    experts/shared hold planar MXFP4 arrays. `copies` independent device
    copies of the expert blobs let callers cycle weights so that a cache
    cannot hold them across calls."""
    import torch
    blobs = torch.from_numpy(moe_pack_experts(shape, layer.experts))
    experts = torch.empty((copies, blobs.numel()), dtype=torch.uint8, device=device)
    for c in range(copies):
        experts[c].copy_(blobs)
    del blobs
    shared = None
    if layer.shared is not None:
        sb = torch.from_numpy(moe_pack_experts(shape, layer.shared))
        shared = torch.empty((copies, sb.numel()), dtype=torch.uint8, device=device)
        for c in range(copies):
            shared[c].copy_(sb)
    norm_w = None if layer.norm_w is None else torch.from_numpy(
        np.ascontiguousarray(layer.norm_w, dtype=np.float32)).to(device)
    return DeviceLayer(
        torch.from_numpy(np.ascontiguousarray(layer.router_w, dtype=np.float32)).to(device),
        torch.from_numpy(np.ascontiguousarray(layer.router_b, dtype=np.float32)).to(device),
        experts, shared, norm_w)


def workspace(shape: MoeShape, device="cuda"):
    import torch
    return torch.empty(moe_workspace_bytes(shape), dtype=torch.uint8, device=device)
