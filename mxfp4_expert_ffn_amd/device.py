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
    sel_bias: "object | None" = None  # [E] float32 selection-only bias, or None
    tid2eid: "object | None" = None   # [vocab, k] int32 hash-routing table, or None

    def routing(self, token_ids=None):
        """The routing argument of the block calls for this layer: None (plain
        top-k), the selection-only bias, or the hash table with the calls'
        token ids ([T] int32 device tensor)."""
        if self.tid2eid is not None:
            if token_ids is None:
                raise ValueError("a hash-routed layer needs token ids")
            return {"tid2eid": self.tid2eid, "token_ids": token_ids}
        if self.sel_bias is not None:
            return {"sel_bias": self.sel_bias}
        return None

    def experts_copy(self, c: int):
        return self.experts[c % self.experts.shape[0]]

    def shared_copy(self, c: int):
        return None if self.shared is None else self.shared[c % self.shared.shape[0]]


def upload_layer(shape: MoeShape, layer, device="cuda", copies: int = 1) -> DeviceLayer:
    """`layer` has router_w, router_b, experts, shared and norm_w (numpy), and
    optionally sel_bias / tid2eid (routing variants);
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
    sel_bias = getattr(layer, "sel_bias", None)
    tid2eid = getattr(layer, "tid2eid", None)
    return DeviceLayer(
        torch.from_numpy(np.ascontiguousarray(layer.router_w, dtype=np.float32)).to(device),
        torch.from_numpy(np.ascontiguousarray(layer.router_b, dtype=np.float32)).to(device),
        experts, shared, norm_w,
        None if sel_bias is None else torch.from_numpy(
            np.ascontiguousarray(sel_bias, dtype=np.float32)).to(device),
        None if tid2eid is None else torch.from_numpy(
            np.ascontiguousarray(tid2eid, dtype=np.int32)).to(device))


def workspace(shape: MoeShape, device="cuda"):
    import torch
    return torch.empty(moe_workspace_bytes(shape), dtype=torch.uint8, device=device)
