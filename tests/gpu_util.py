"""Helpers for the GPU parity tests: run the HIP path through the C ABI on
seeded workloads and compare with the CPU oracle."""
from __future__ import annotations

import numpy as np
import torch

import mxfp4_expert_ffn_amd as mx
from mxfp4_expert_ffn_amd.device import upload_layer, workspace
from oracle import moe as omoe

TOL = 2e-3  # max |err| relative to the RMS of the oracle output


def shape_of(cfg, T=None):
    return mx.make_shape(**cfg.shape_kwargs(T))


def device_input(cfg, x32: np.ndarray, xbf: np.ndarray | None):
    if cfg.act_dtype == "bf16":
        return torch.from_numpy(xbf.view(np.int16).copy()).cuda()
    return torch.from_numpy(np.ascontiguousarray(x32)).cuda()


def route_buffers(T, k, E, device="cuda"):
    i32 = dict(dtype=torch.int32, device=device)
    return dict(topk_idx=torch.full((T, k), -1, **i32),
                topk_w=torch.full((T, k), -1.0, dtype=torch.float32, device=device),
                counts=torch.full((E,), -1, **i32), offsets=torch.full((E + 1,), -1, **i32),
                perm=torch.full((T * k,), -1, **i32), inv=torch.full((T * k,), -1, **i32))


def to_np(d):
    return {k: v.cpu().numpy() for k, v in d.items()}


def run_forward(path, shape, dl, x_dev, out=None, route=True, copy=0, token_ids=None):
    T, H, k, E = shape.T, shape.H, shape.k, shape.E
    if out is None:
        out = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    ws = workspace(shape)
    ro = route_buffers(T, k, E) if route else None
    fn = mx.moe_forward_decode if path == "decode" else mx.moe_forward_prefill
    fn(shape, x_dev, dl.router_w, dl.router_b, dl.experts_copy(copy), out, ws, norm_w=dl.norm_w,
       shared=dl.shared_copy(copy), route_out=ro, routing=dl.routing(token_ids))
    torch.cuda.synchronize()
    return out, ro


def rel_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    ref = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(ref ** 2))
    return float(np.max(np.abs(np.asarray(gpu, dtype=np.float64) - ref)) / rms)


def gap_bound(xn: np.ndarray, router_w: np.ndarray, router_b: np.ndarray) -> np.ndarray:
    """Per-token bound on fp64 summation-order differences of the logits:
    2^-36 * max_e (sum_h |xn_h w_eh| + |b_e|). Decisions closer than this are
    ties for the purpose of comparing two fp64 evaluations."""
    mag = np.abs(xn.astype(np.float64)) @ np.abs(router_w.astype(np.float64)).T + np.abs(router_b)
    return 2.0 ** -36 * mag.max(axis=1)


def check_routing(gpu_idx, gpu_w, ref, router_w, router_b, route_scale, max_flips=0):
    """idx bit-exact except at certified near-ties of the values the selection
    ranked (logits, or logits + selection-only bias); a hash-routed block has
    no ties, its idx must equal the table rows; weights within 1e-6."""
    logits, ridx = ref.get("sel", ref["logits"]), ref["idx"]
    if ref.get("hashed"):
        assert np.array_equal(gpu_idx, ridx)
    bound = gap_bound(ref["xn"], router_w, router_b)
    bad = np.nonzero(np.any(gpu_idx != ridx, axis=1))[0]
    flips = 0
    for t in bad:
        for j in np.nonzero(gpu_idx[t] != ridx[t])[0]:
            d = abs(logits[t, gpu_idx[t, j]] - logits[t, ridx[t, j]])
            assert d <= bound[t], f"token {t} slot {j}: gpu {gpu_idx[t]} oracle {ridx[t]} gap {d}"
        flips += 1
    assert flips <= max_flips, f"{flips} certified near-tie flips"
    if flips == 0:
        assert np.max(np.abs(gpu_w - ref["w"])) <= 1e-6 * route_scale
    return flips


def check_permutation(ro: dict, idx: np.ndarray, E: int):
    counts, offsets, perm, inv = omoe.permutation(idx, E)
    assert np.array_equal(ro["counts"], counts)
    assert np.array_equal(ro["offsets"], offsets)
    assert np.array_equal(ro["perm"], perm)
    assert np.array_equal(ro["inv"], inv)


def upload(cfg, layer, copies=1):
    return upload_layer(shape_of(cfg), layer, copies=copies)
