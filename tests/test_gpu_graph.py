"""HIP-graph replay of the block (the launch mode the benchmark times): every
replay, with eager work and synchronisations in between, must give the eager
result bit for bit (both paths add a token's routes in a fixed order, with one
writer per output element), routing results included. The route profile counts the replays only
(capture runs nothing)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mxfp4_expert_ffn_amd as mx
from mxfp4_expert_ffn_amd.device import workspace
from workloads import config_by_id, make_layer, scaled
from workloads.gen import make_activations

from gpu_util import device_input, shape_of, upload

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)


def _capture(fn):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def _eager_noise(xd, dl, shape, ws):
    """Unrelated eager work between replays: another block call on other data
    (its own buffers and workspace) and a torch fill."""
    other = torch.empty((shape.T, shape.H), dtype=torch.float32, device="cuda")
    fn = mx.moe_forward_prefill if shape.T > 64 else mx.moe_forward_decode
    fn(shape, torch.flip(xd, dims=[0]).contiguous(), dl.router_w, dl.router_b, dl.experts_copy(0),
       other, ws, norm_w=dl.norm_w, shared=dl.shared_copy(0))
    other.fill_(0.5)


# (5, 2048): the DeepSeek-V4-Flash layer at full size, the kernels its bench
# line replays (bf16 operand on 64-row tiles, two workgroups per CU)
@pytest.mark.parametrize("cid,T", [(3, 128), (5, 256), (4, 96), (5, 2048)])
def test_prefill_graph_replays_equal_eager(cid, T):
    full = (cid, T) in ((3, 128), (5, 2048))
    cfg = config_by_id(cid) if full else scaled(config_by_id(cid), T=T, H=512, F=256,
                                                E=min(config_by_id(cid).E, 16))
    _announce(f"graph replay: prefill config {cid} T={T}")
    layer = make_layer(cfg)
    x, xb = make_activations(cfg, rows=cfg.T)
    dl = upload(cfg, layer)
    shape = shape_of(cfg)
    xd = device_input(cfg, x, xb)
    ws, ws_noise = workspace(shape), workspace(shape)
    i32 = dict(dtype=torch.int32, device="cuda")
    out_e = torch.empty((cfg.T, cfg.H), dtype=torch.float32, device="cuda")
    ro_e = dict(topk_idx=torch.empty((cfg.T, cfg.k), **i32), perm=torch.empty(cfg.T * cfg.k, **i32))
    mx.moe_forward_prefill(shape, xd, dl.router_w, dl.router_b, dl.experts_copy(0), out_e, ws,
                           norm_w=dl.norm_w, shared=dl.shared_copy(0), route_out=ro_e)
    torch.cuda.synchronize()
    out_g = torch.empty_like(out_e)
    ro_g = dict(topk_idx=torch.empty_like(ro_e["topk_idx"]), perm=torch.empty_like(ro_e["perm"]),
                route_counts=torch.zeros(cfg.E, dtype=torch.int64, device="cuda"))
    g = _capture(lambda: mx.moe_forward_prefill(shape, xd, dl.router_w, dl.router_b,
                                                dl.experts_copy(0), out_g, ws, norm_w=dl.norm_w,
                                                shared=dl.shared_copy(0), route_out=ro_g))
    torch.cuda.synchronize()
    assert not ro_g["route_counts"].any()  # capture executes nothing
    for rep in range(REPLAYS):
        out_g.fill_(float("nan"))
        ro_g["topk_idx"].fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), f"replay {rep}"
        assert torch.equal(ro_g["topk_idx"], ro_e["topk_idx"]) and torch.equal(ro_g["perm"], ro_e["perm"])
        _eager_noise(xd, dl, shape, ws_noise)
        torch.cuda.synchronize()
    counts = np.bincount(ro_e["topk_idx"].cpu().numpy().ravel(), minlength=cfg.E)
    assert np.array_equal(ro_g["route_counts"].cpu().numpy(), REPLAYS * counts)


def test_decode_graph_replays_equal_eager():
    cfg = config_by_id(2)
    _announce("graph replay: decode config 2, 4 tokens as T=1 calls in one graph")
    layer = make_layer(cfg)
    x, _ = make_activations(cfg, rows=4)
    dl = upload(cfg, layer)
    shape = shape_of(cfg, 1)
    ws, ws_noise = workspace(shape), workspace(shape)
    xd = torch.from_numpy(x).cuda()
    i32 = dict(dtype=torch.int32, device="cuda")

    def calls(out, idx, tab):
        for t in range(4):
            ro = dict(topk_idx=idx[t:t + 1], route_counts=tab) if tab is not None else dict(topk_idx=idx[t:t + 1])
            mx.moe_forward_decode(shape, xd[t:t + 1], dl.router_w, dl.router_b, dl.experts_copy(0),
                                  out[t:t + 1], ws, route_out=ro)

    out_e, idx_e = torch.empty((4, cfg.H), dtype=torch.float32, device="cuda"), torch.empty((4, cfg.k), **i32)
    calls(out_e, idx_e, None)
    torch.cuda.synchronize()
    out_g, idx_g = torch.empty_like(out_e), torch.empty_like(idx_e)
    tab = torch.zeros(cfg.E, dtype=torch.int64, device="cuda")
    g = _capture(lambda: calls(out_g, idx_g, tab))
    torch.cuda.synchronize()
    for rep in range(REPLAYS):
        out_g.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx_g, idx_e), f"replay {rep}"
        assert torch.equal(out_g, out_e), f"replay {rep}"
        _eager_noise(xd[:1], dl, shape, ws_noise)
        torch.cuda.synchronize()
    counts = np.bincount(idx_e.cpu().numpy().ravel(), minlength=cfg.E)
    assert np.array_equal(tab.cpu().numpy(), REPLAYS * counts)
