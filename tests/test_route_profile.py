"""Expert-route profile (goosedump `ExpertRouteProfile`): the oracle against
what the definition fixes, the library's host summary against the oracle, and
(marked gpu) the counters the HIP path accumulates against the oracle, bit for
bit, through the C ABI."""
from __future__ import annotations

import numpy as np
import pytest

from oracle import moe
from oracle.route_profile import U64_MAX, RouteProfile
from workloads import config_by_id, make_layer, scaled
from workloads.gen import make_activations


def _routing(cfg, T, layer=0):
    lay = make_layer(cfg, layer)
    x, _ = make_activations(cfg, rows=T)
    xn = x.astype(np.float64)
    if lay.norm_w is not None:
        xn = moe.rms_norm(xn, lay.norm_w, cfg.rms_eps)
    _, idx, _, _ = moe.route(xn, lay.router_w, lay.router_b, cfg.k, cfg.route_scale)
    return idx


@pytest.mark.parametrize("cid", [1, 3, 5])
def test_counts_are_k_per_token_and_equal_the_permutation_histogram(cid):
    cfg = config_by_id(cid)
    T = min(cfg.T, 64)
    idx = _routing(scaled(cfg, T=T), T)
    prof = RouteProfile(2, cfg.E)
    prof.record_block(1, idx)
    assert prof.counts[0] == [0] * cfg.E
    assert sum(prof.counts[1]) == T * cfg.k  # k distinct experts per token
    counts, _, _, _ = moe.permutation(idx, cfg.E)  # independent histogram
    assert prof.counts[1] == [int(c) for c in counts]
    assert prof.selections() == T * cfg.k
    assert prof.layer_unique_counts() == [0, int(np.count_nonzero(counts))]


def test_record_saturates_and_selections_saturate():
    prof = RouteProfile(2, 4)
    prof.counts[0][3] = U64_MAX - 1
    prof.record(0, [3])
    assert prof.counts[0][3] == U64_MAX
    prof.record(0, [3, 3])
    assert prof.counts[0][3] == U64_MAX
    prof.counts[1][0] = 5
    assert prof.selections() == U64_MAX
    prof.counts[0][3] = 7
    assert prof.selections() == 12


def test_out_of_range_layer_and_expert_are_skipped():
    prof = RouteProfile(2, 4)
    prof.record(-1, [0, 1])
    prof.record(2, [0, 1])
    prof.record(1, [4, -1, 2])
    assert prof.counts == [[0, 0, 0, 0], [0, 0, 1, 0]]


def test_constructed_unique_counts():
    prof = RouteProfile(3, 8)
    for _ in range(5):
        prof.record(0, [2, 5])        # every token the same pair
    prof.record_block(1, [[0, 1], [1, 2], [2, 0]])
    assert prof.counts[0] == [0, 0, 5, 0, 0, 5, 0, 0]
    assert prof.counts[1] == [2, 2, 2, 0, 0, 0, 0, 0]
    assert prof.layer_unique_counts() == [2, 3, 0]
    assert prof.unique_layer_experts() == 5
    assert prof.selections() == 16


def test_library_summary_equals_oracle():
    import mxfp4_expert_ffn_amd as mx
    rng = np.random.default_rng(7)
    for layers, E in [(1, 1), (3, 8), (24, 32), (2, 256)]:
        tab = rng.integers(0, 3, size=(layers, E)).astype(np.uint64)
        prof = RouteProfile(layers, E)
        prof.counts = [[int(c) for c in row] for row in tab]
        got = mx.moe_route_profile_summary(tab)
        assert got["selections"] == prof.selections()
        assert got["unique_layer_experts"] == prof.unique_layer_experts()
        assert got["layer_unique"] == prof.layer_unique_counts()
    tab = np.array([[U64_MAX - 3, 2], [0, 9]], dtype=np.uint64)  # the sum saturates
    prof = RouteProfile(2, 2)
    prof.counts = [[U64_MAX - 3, 2], [0, 9]]
    got = mx.moe_route_profile_summary(tab)
    assert got["selections"] == prof.selections() == U64_MAX
    assert got["layer_unique"] == [2, 1]


def test_library_summary_rejects_bad_arguments():
    import ctypes
    import mxfp4_expert_ffn_amd as mx
    from mxfp4_expert_ffn_amd import _lib
    lib = _lib.load()
    sel, uni = ctypes.c_uint64(), ctypes.c_uint64()
    tab = np.zeros((1, 4), dtype=np.uint64)
    p = tab.ctypes.data_as(ctypes.c_void_p)
    assert lib.moe_route_profile_summary(None, 1, 4, ctypes.byref(sel), ctypes.byref(uni), None) < 0
    assert lib.moe_route_profile_summary(p, -1, 4, ctypes.byref(sel), ctypes.byref(uni), None) < 0
    assert lib.moe_route_profile_summary(p, 1, 0, ctypes.byref(sel), ctypes.byref(uni), None) < 0
    assert lib.moe_route_profile_summary(p, 1, 4, None, ctypes.byref(uni), None) < 0
    assert "non-NULL" in mx.moe_last_error() or "need" in mx.moe_last_error()
    assert lib.moe_route_profile_summary(p, 0, 4, ctypes.byref(sel), ctypes.byref(uni), None) == 0
    assert sel.value == 0 and uni.value == 0


# ---------------------------------------------------------------- GPU (C ABI)
def _announce(msg):
    print(f"\n[case] {msg}", flush=True)


def _oracle_idx(cfg, layer, x):
    xn = x.astype(np.float64)
    if layer.norm_w is not None:
        xn = moe.rms_norm(xn, layer.norm_w, cfg.rms_eps)
    return moe.route(xn, layer.router_w, layer.router_b, cfg.k, cfg.route_scale)[1]


def _table(layers, E):
    import torch
    return torch.zeros((layers, E), dtype=torch.int64, device="cuda")


@pytest.mark.gpu
def test_gpu_decode_calls_accumulate_the_oracle_profile():
    import torch
    import mxfp4_expert_ffn_amd as mx
    from gpu_util import shape_of, upload
    from mxfp4_expert_ffn_amd.device import workspace
    cfg = config_by_id(2)
    _announce("route profile: decode config 2, 32 tokens as T=1 calls into one table")
    layer = make_layer(cfg)
    x, _ = make_activations(cfg, rows=32)
    dl = upload(cfg, layer)
    shape = shape_of(cfg, 1)
    ws = workspace(shape)
    xd = torch.from_numpy(x).cuda()
    out = torch.empty_like(xd)
    tab = _table(1, cfg.E)
    counts = torch.full((cfg.E,), -1, dtype=torch.int32, device="cuda")
    for t in range(x.shape[0]):
        # the counts export runs the permutation too: the table must not count twice
        ro = dict(route_counts=tab[0], counts=counts if t % 2 else None)
        mx.moe_forward_decode(shape, xd[t:t + 1], dl.router_w, dl.router_b, dl.experts_copy(0),
                              out[t:t + 1], ws, route_out=ro)
    torch.cuda.synchronize()
    prof = RouteProfile(1, cfg.E)
    prof.record_block(0, _oracle_idx(cfg, layer, x))
    assert np.array_equal(tab.cpu().numpy().view(np.uint64), prof.table())
    assert mx.moe_route_profile_summary(tab.cpu().numpy())["selections"] == 32 * cfg.k


@pytest.mark.gpu
def test_gpu_decode_batch_and_shared_expert_profile():
    import torch
    import mxfp4_expert_ffn_amd as mx
    from gpu_util import shape_of, upload, device_input
    from mxfp4_expert_ffn_amd.device import workspace
    base = config_by_id(5)
    cfg = scaled(base, T=8, H=256, F=256, E=16)
    _announce("route profile: decode T=8, bf16, shared expert (not a selection)")
    layer = make_layer(cfg)
    x, xb = make_activations(cfg)
    dl = upload(cfg, layer)
    shape = shape_of(cfg)
    out = torch.empty((cfg.T, cfg.H), dtype=torch.float32, device="cuda")
    tab = _table(1, cfg.E)
    mx.moe_forward_decode(shape, device_input(cfg, x, xb), dl.router_w, dl.router_b,
                          dl.experts_copy(0), out, workspace(shape), shared=dl.shared_copy(0),
                          route_out=dict(route_counts=tab[0]))
    torch.cuda.synchronize()
    prof = RouteProfile(1, cfg.E)
    prof.record_block(0, _oracle_idx(cfg, layer, x))
    assert np.array_equal(tab.cpu().numpy().view(np.uint64), prof.table())


@pytest.mark.gpu
def test_gpu_prefill_profile_accumulates_over_calls():
    import torch
    import mxfp4_expert_ffn_amd as mx
    from gpu_util import shape_of, upload
    from mxfp4_expert_ffn_amd.device import workspace
    cfg = config_by_id(3)
    _announce("route profile: prefill config 3 (T=128, Zipf loads), two calls")
    layer = make_layer(cfg)
    x, _ = make_activations(cfg)
    dl = upload(cfg, layer)
    shape = shape_of(cfg)
    ws = workspace(shape)
    xd = torch.from_numpy(x[:cfg.T]).cuda()
    out = torch.empty_like(xd)
    tab = _table(1, cfg.E)
    prof = RouteProfile(1, cfg.E)
    idx = _oracle_idx(cfg, layer, x[:cfg.T])
    for _ in range(2):
        mx.moe_forward_prefill(shape, xd, dl.router_w, dl.router_b, dl.experts_copy(0), out, ws,
                               route_out=dict(route_counts=tab[0]))
        prof.record_block(0, idx)
    torch.cuda.synchronize()
    assert np.array_equal(tab.cpu().numpy().view(np.uint64), prof.table())


@pytest.mark.gpu
def test_gpu_route_only_profile_at_full_ds4_size():
    import torch
    import mxfp4_expert_ffn_amd as mx
    from gpu_util import shape_of, upload, device_input
    from mxfp4_expert_ffn_amd.device import workspace
    cfg = config_by_id(5)
    _announce("route profile: moe_route, DS4 shape T=2048, E=256")
    layer = make_layer(cfg)
    x, xb = make_activations(cfg)
    dl = upload(cfg, layer)
    shape = shape_of(cfg)
    tab = _table(1, cfg.E)
    idx_d = torch.full((cfg.T, cfg.k), -1, dtype=torch.int32, device="cuda")
    mx.moe_route(shape, device_input(cfg, x, xb), dl.router_w, dl.router_b,
                 dict(topk_idx=idx_d, route_counts=tab[0]), workspace(shape))
    torch.cuda.synchronize()
    ridx = _oracle_idx(cfg, layer, x)
    assert np.array_equal(idx_d.cpu().numpy(), ridx)
    prof = RouteProfile(1, cfg.E)
    prof.record_block(0, ridx)
    assert np.array_equal(tab.cpu().numpy().view(np.uint64), prof.table())


@pytest.mark.gpu
def test_gpu_stack_layers_fill_their_own_rows():
    import torch
    import mxfp4_expert_ffn_amd as mx
    from gpu_util import shape_of, upload
    from mxfp4_expert_ffn_amd.device import workspace
    cfg = scaled(config_by_id(4), T=64)
    _announce("route profile: two RMSNorm + MoE layers of the stack, rows of a [24][E] table")
    x, _ = make_activations(cfg)
    shape = shape_of(cfg)
    ws = workspace(shape)
    tab = _table(24, cfg.E)
    h = torch.from_numpy(x[:cfg.T]).cuda()
    idx_d = torch.full((cfg.T, cfg.k), -1, dtype=torch.int32, device="cuda")
    prof = RouteProfile(24, cfg.E)
    for l in (0, 1):
        layer = make_layer(cfg, l)
        dl = upload(cfg, layer)
        out = torch.empty_like(h)
        h_host = h.cpu().numpy()
        mx.moe_forward_prefill(shape, h, dl.router_w, dl.router_b, dl.experts_copy(0), out, ws,
                               norm_w=dl.norm_w, route_out=dict(topk_idx=idx_d, route_counts=tab[l]))
        torch.cuda.synchronize()
        gidx = idx_d.cpu().numpy()
        # the layer's input is the GPU's previous output (teacher forcing); the
        # selections must be the oracle's on that input
        assert np.array_equal(gidx, _oracle_idx(cfg, layer, h_host))
        prof.record_block(l, gidx)
        h = out
    got = tab.cpu().numpy().view(np.uint64)
    assert np.array_equal(got, prof.table())
    s = mx.moe_route_profile_summary(got)
    assert s["selections"] == 2 * cfg.T * cfg.k
    assert s["layer_unique"][2:] == [0] * 22
