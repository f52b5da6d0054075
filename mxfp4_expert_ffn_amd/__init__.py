"""Routed MXFP4 Mixture-of-Experts block for AMD Instinct MI355X (gfx950).

A thin binding over the C ABI of `libmoe_mxfp4.so` (include/moe_mxfp4.h):
each function has the C name, turns torch device tensors into pointers and
the current HIP stream, and raises `MoeError` on a negative status. Every
step of the block runs in the library's HIP kernels; PyTorch only provides
device memory and streams. There is no CPU fallback: without the built
library every call raises.
"""
from __future__ import annotations

import ctypes

import numpy as np

from . import _lib
from ._lib import (MOE_BF16, MOE_F32, MoeBlobLayout, MoeExpertPlanes, MoeLocalityOut, MoeRouteOut,
                   MoeShape)

__all__ = [
    "MoeError", "MoeShape", "make_shape", "moe_blob_layout_get", "moe_pack_experts",
    "moe_workspace_bytes", "moe_route", "moe_forward_decode", "moe_forward_prefill",
    "moe_forward_decode_noalloc", "moe_prefill_plan",
    "moe_act_quant_debug", "moe_dequant_debug", "moe_last_error", "moe_profile_next_launch", "moe_route_profile_summary",
    "moe_route_locality", "moe_route_hotlist", "LOCALITY_CACHE_SIZES", "ROUTE_FIELDS",
]

# route_counts: an int64 [E] device tensor the call adds its selections per
# expert to (the C side's uint64 route profile row)
ROUTE_FIELDS = ("topk_idx", "topk_w", "counts", "offsets", "perm", "inv", "route_counts")
_ROUTE_DTYPES = {"topk_w": "float32", "route_counts": "int64"}


class MoeError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"[{code}] {message}")
        self.code = code


def make_shape(T, H, F, E, k, act_dtype="f32", n_shared=0, alpha=1.702, limit=7.0,
               up_offset=1.0, route_scale=1.0, rms_eps=0.0, act_quant=0) -> MoeShape:
    """act_quant=1: the quantised expert-input mode (MX-FP4 expert input,
    prefill only)."""
    return MoeShape(int(T), int(H), int(F), int(E), int(k),
                    MOE_BF16 if act_dtype == "bf16" else MOE_F32, int(n_shared),
                    float(alpha), float(limit), float(up_offset), float(route_scale),
                    float(rms_eps), int(act_quant))


def moe_last_error() -> str:
    return _lib.load().moe_last_error().decode()


def _check(rc: int):
    if rc != 0:
        raise MoeError(rc, moe_last_error())


def _ptr(t, name: str, dtype=None, optional: bool = False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _route_out(route_out):
    import torch
    if route_out is None:
        return None
    ro = MoeRouteOut()
    for f in ROUTE_FIELDS:
        t = route_out.get(f)
        dt = getattr(torch, _ROUTE_DTYPES.get(f, "int32"))
        setattr(ro, f, None if t is None else _ptr(t, f, dt).value)
    return ctypes.byref(ro)


def _routing(routing):
    """routing: None, or a dict with "sel_bias" ([E] float32), or "tid2eid"
    ([vocab, k] int32) and "token_ids" ([T] int32), device tensors."""
    import torch
    if routing is None:
        return None
    r = _lib.MoeRouting()
    unknown = set(routing) - {"sel_bias", "tid2eid", "token_ids"}
    if unknown:
        raise ValueError(f"unknown routing fields {sorted(unknown)}")
    b, tab, ids = routing.get("sel_bias"), routing.get("tid2eid"), routing.get("token_ids")
    r.sel_bias = None if b is None else _ptr(b, "sel_bias", torch.float32).value
    r.tid2eid = None if tab is None else _ptr(tab, "tid2eid", torch.int32).value
    r.token_ids = None if ids is None else _ptr(ids, "token_ids", torch.int32).value
    r.vocab = 0 if tab is None else int(tab.shape[0])
    return ctypes.byref(r)


def moe_blob_layout_get(shape: MoeShape) -> dict:
    L = MoeBlobLayout()
    _check(_lib.load().moe_blob_layout_get(ctypes.byref(shape), ctypes.byref(L)))
    return {name: getattr(L, name) for name, _ in L._fields_}


def moe_pack_experts(shape: MoeShape, planes) -> np.ndarray:
    """Pack host planar MXFP4 experts (attributes or keys gate_codes, gate_scales,
    gate_bias, up_*, down_*) into n blobs; returns uint8 [n * stride] (host)."""
    get = (lambda k: planes[k]) if isinstance(planes, dict) else (lambda k: getattr(planes, k))
    names = {"gate_q": "gate_codes", "up_q": "up_codes", "down_q": "down_codes",
             "gate_s": "gate_scales", "up_s": "up_scales", "down_s": "down_scales",
             "gate_b": "gate_bias", "up_b": "up_bias", "down_b": "down_bias"}
    arrs = {}
    for cname, pname in names.items():
        a = get(pname)
        want = np.float32 if cname.endswith("_b") else np.uint8
        arrs[cname] = np.ascontiguousarray(a, dtype=want)
    n = arrs["gate_q"].shape[0]
    stride = moe_blob_layout_get(shape)["stride"]
    dst = np.empty(n * stride, dtype=np.uint8)
    p = MoeExpertPlanes(**{k: v.ctypes.data for k, v in arrs.items()})
    _check(_lib.load().moe_pack_experts(ctypes.byref(shape), n, ctypes.byref(p),
                                        dst.ctypes.data_as(ctypes.c_void_p)))
    return dst


def moe_workspace_bytes(shape: MoeShape) -> int:
    n = _lib.load().moe_workspace_bytes(ctypes.byref(shape))
    if n == 0:
        raise MoeError(_lib.MOE_ERR_INVALID_ARG, moe_last_error())
    return int(n)


def moe_route(shape, x, router_w, router_b, route_out: dict, ws, norm_w=None, stream=None,
              routing=None):
    import torch
    rc = _lib.load().moe_route(
        ctypes.byref(shape), _ptr(x, "x", (torch.float32, torch.bfloat16, torch.int16, torch.uint16)),
        _ptr(norm_w, "norm_w", torch.float32, optional=True),
        _ptr(router_w, "router_w", torch.float32), _ptr(router_b, "router_b", torch.float32),
        _routing(routing), _route_out(route_out), _ptr(ws, "ws"), ws.numel() * ws.element_size(), _stream(stream))
    _check(rc)


def _forward(fn, shape, hidden, router_w, router_b, experts, out, ws, norm_w, shared,
             route_out, stream, routing):
    import torch
    rc = fn(ctypes.byref(shape),
            _ptr(hidden, "hidden", (torch.float32, torch.bfloat16, torch.int16, torch.uint16)),
            _ptr(norm_w, "norm_w", torch.float32, optional=True),
            _ptr(router_w, "router_w", torch.float32), _ptr(router_b, "router_b", torch.float32),
            _routing(routing), _ptr(experts, "experts", torch.uint8), _ptr(shared, "shared", torch.uint8, optional=True),
            _ptr(out, "out", torch.float32), _route_out(route_out), _ptr(ws, "ws"),
            ws.numel() * ws.element_size(), _stream(stream))
    _check(rc)


def moe_forward_decode(shape, hidden, router_w, router_b, experts, out, ws, norm_w=None,
                       shared=None, route_out=None, stream=None, routing=None):
    _forward(_lib.load().moe_forward_decode, shape, hidden, router_w, router_b, experts, out, ws,
             norm_w, shared, route_out, stream, routing)


def moe_forward_prefill(shape, hidden, router_w, router_b, experts, out, ws, norm_w=None,
                        shared=None, route_out=None, stream=None, routing=None):
    _forward(_lib.load().moe_forward_prefill, shape, hidden, router_w, router_b, experts, out, ws,
             norm_w, shared, route_out, stream, routing)


def moe_forward_decode_noalloc(shape, hidden, router_w, router_b, experts, out, norm_w=None,
                               shared=None, route_out=None, stream=None, routing=None):
    """moe_forward_decode with the library's fixed per-GPU scratch as its
    workspace: no allocation; calls on one GPU must be ordered on one stream."""
    import torch
    rc = _lib.load().moe_forward_decode_noalloc(
        ctypes.byref(shape),
        _ptr(hidden, "hidden", (torch.float32, torch.bfloat16, torch.int16, torch.uint16)),
        _ptr(norm_w, "norm_w", torch.float32, optional=True),
        _ptr(router_w, "router_w", torch.float32), _ptr(router_b, "router_b", torch.float32),
        _routing(routing), _ptr(experts, "experts", torch.uint8),
        _ptr(shared, "shared", torch.uint8, optional=True),
        _ptr(out, "out", torch.float32), _route_out(route_out), _stream(stream))
    _check(rc)


def moe_prefill_plan(shape, with_norm: bool = False) -> dict:
    """The grouped GEMMs' tiling and FP8 term counts moe_forward_prefill uses
    for this shape (host only)."""
    p = _lib.MoePrefillPlan()
    _check(_lib.load().moe_prefill_plan(ctypes.byref(shape), int(bool(with_norm)), ctypes.byref(p)))
    return {name: getattr(p, name) for name, _ in p._fields_}


def moe_act_quant_debug(shape, x, codes, scales, ws, norm_w=None, stream=None):
    """The MX-FP4 expert input of the quantised mode: codes [T, H/2] and scale
    bytes [T, H/32] (uint8 device tensors) as the prefill kernels use them."""
    import torch
    T, H = shape.T, shape.H
    if codes.numel() != T * (H // 2) or scales.numel() != T * (H // 32):
        raise ValueError("codes must hold T*H/2 bytes and scales T*H/32")
    _check(_lib.load().moe_act_quant_debug(
        ctypes.byref(shape), _ptr(x, "x", (torch.float32, torch.bfloat16, torch.int16, torch.uint16)),
        _ptr(norm_w, "norm_w", torch.float32, optional=True), _ptr(codes, "codes", torch.uint8),
        _ptr(scales, "scales", torch.uint8), _ptr(ws, "ws"), ws.numel() * ws.element_size(),
        _stream(stream)))


def moe_dequant_debug(shape, blob, which: int, path: int, out, stream=None):
    import torch
    _check(_lib.load().moe_dequant_debug(ctypes.byref(shape), _ptr(blob, "blob", torch.uint8),
                                         int(which), int(path), _ptr(out, "out", torch.float32),
                                         _stream(stream)))


def moe_profile_next_launch(kernel, start_event: int, stop_event: int):
    """Arm the one-shot timing hook: raw hipEvent_t handles (ints) recorded
    around the next launch of `kernel` (a name of `_lib.KERNELS` or an id)."""
    kid = _lib.KERNELS[kernel] if isinstance(kernel, str) else int(kernel)
    _check(_lib.load().moe_profile_next_launch(kid, ctypes.c_void_p(start_event),
                                               ctypes.c_void_p(stop_event)))


def moe_route_profile_summary(counts) -> dict:
    """Summary of a host route profile table [layers][E] (uint64 or int64):
    total selections (saturating), nonzero (layer, expert) counters and the
    nonzero counters of each layer (goosedump `ExpertRouteProfile`)."""
    c = np.ascontiguousarray(counts).view(np.uint64) if np.asarray(counts).dtype == np.int64 \
        else np.ascontiguousarray(counts, dtype=np.uint64)
    if c.ndim != 2:
        raise ValueError("counts must be [layers, E]")
    sel, uniq = ctypes.c_uint64(), ctypes.c_uint64()
    per = np.zeros(c.shape[0], dtype=np.int32)
    _check(_lib.load().moe_route_profile_summary(
        c.ctypes.data_as(ctypes.c_void_p), c.shape[0], c.shape[1], ctypes.byref(sel),
        ctypes.byref(uniq), per.ctypes.data_as(ctypes.c_void_p)))
    return dict(selections=sel.value, unique_layer_experts=uniq.value, layer_unique=per.tolist())


# cache sizes the locality profile simulates by default: ds4.c's candidates
# (those not above E are used)
LOCALITY_CACHE_SIZES = (1, 2, 4, 8, 16, 32, 64, 128, 256, 384)


def _host(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def moe_route_locality(idx, weights, E: int, caps=None) -> dict:
    """Locality of a decode trace (antirez ds4.c's routed-expert locality
    profiler): idx and weights [positions, layers, k] (host arrays, or what a
    T=1 call's topk_idx / topk_w hold, copied back per position and layer).
    Returns the library's per-layer counts, route-weight sums, adjacent-token
    overlap and Jaccard sums, and the hits of each simulated cache size."""
    ix = _host(idx, np.int32)
    w = _host(weights, np.float32)
    if ix.ndim != 3 or w.shape != ix.shape:
        raise ValueError("idx and weights must both be [positions, layers, k]")
    P, L, k = ix.shape
    cs = _host([c for c in LOCALITY_CACHE_SIZES if c <= E] if caps is None else caps, np.int32)
    r = dict(caps=cs, hist=np.zeros((L, E), np.uint64), weight_hist=np.zeros((L, E), np.float64),
             cache_hits=np.zeros((cs.size, L), np.uint64),
             cache_weight_hits=np.zeros((cs.size, L), np.float64),
             adjacent_pairs=np.zeros(L, np.uint64), overlap_sum=np.zeros(L, np.float64),
             jaccard_sum=np.zeros(L, np.float64))
    vp = ctypes.c_void_p
    out = MoeLocalityOut(*(vp(r[n].ctypes.data) for n in (
        "hist", "weight_hist", "cache_hits", "cache_weight_hits", "adjacent_pairs", "overlap_sum",
        "jaccard_sum")))
    _check(_lib.load().moe_route_locality(vp(ix.ctypes.data), vp(w.ctypes.data), P, L, k, int(E),
                                          vp(cs.ctypes.data), cs.size, ctypes.byref(out)))
    return r


def moe_route_hotlist(hist, weight_hist) -> np.ndarray:
    """Every layer * E + expert of a locality histogram [layers, E], ranked by
    count and route weight (descending), then layer and expert."""
    h = _host(hist, np.uint64)
    wh = _host(weight_hist, np.float64)
    if h.ndim != 2 or wh.shape != h.shape:
        raise ValueError("hist and weight_hist must both be [layers, E]")
    order = np.zeros(h.size, np.int32)
    vp = ctypes.c_void_p
    _check(_lib.load().moe_route_hotlist(vp(h.ctypes.data), vp(wh.ctypes.data), h.shape[0],
                                         h.shape[1], vp(order.ctypes.data)))
    return order
