"""Routed-expert locality (antirez ds4.c's locality profiler): the oracle
against what the definitions fix, the library's host implementation against
the oracle, and (marked gpu) the locality of a decode trace that the HIP path
routed, through the C ABI."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest

from oracle import moe
from oracle.route_locality import RouteLocality, cache_sizes_for
from workloads import config_by_id, make_layer, scaled
from workloads.gen import make_activations


def _stream(idx, layer, E):
    """The in-range selections of one layer, in position then slot order."""
    return [(int(e), p, j) for p in range(len(idx)) for j, e in enumerate(idx[p][layer])
            if 0 <= int(e) < E]


def _random_trace(rng, P, L, k, E, pool=None):
    """P positions of k distinct experts per layer, drawn from a small pool so
    that experts recur; dyadic weights so that equal sums compare equal."""
    pool = E if pool is None else pool
    idx = np.stack([[rng.choice(pool, size=k, replace=False) for _ in range(L)] for _ in range(P)])
    w = rng.integers(1, 8, size=(P, L, k)).astype(np.float32) / 8
    return idx.astype(np.int32), w


# ------------------------------------------------------------- oracle pins
def test_worked_trace():
    # one layer, k = 2: selections {1, 2}, {2, 3}, {1, 3} at positions 0, 1, 2.
    # The stream 1 2 2 3 1 3 (weights .75 .25 .625 .375 .5 .5), walked by hand:
    #   size 1: only the second 2 hits (.625)
    #   size 2: the second 2 and the last 3 hit (.625 + .5)
    #   size 4: every repeat hits: 2, 1, 3 (.625 + .5 + .5)
    # Adjacent pairs share one expert each: overlap 1/2, Jaccard 1/3 per pair.
    idx = [[[1, 2]], [[2, 3]], [[1, 3]]]
    w = [[[0.75, 0.25]], [[0.625, 0.375]], [[0.5, 0.5]]]
    o = RouteLocality(1, 4, 2, caps=[1, 2, 4])
    o.record_trace(idx, w)
    assert [h[0] for h in o.cache_hits] == [1, 2, 3]
    assert [h[0] for h in o.cache_weight_hits] == [0.625, 1.125, 1.625]
    assert o.adjacent_pairs == [2] and o.overlap_sum == [1.0] and o.jaccard_sum == [2 / 3]
    assert o.hist == [[0, 2, 2, 2]] and o.weight_hist == [[0.0, 1.25, 0.875, 0.875]]
    assert o.ranked_experts(0) == [1, 2, 3]  # equal count and weight: lower index first
    assert o.hit_rate(1) == 2 / 6 and o.weighted_hit_rate(2) == 1.625 / 3.0
    assert o.mean_overlap(0) == 0.5 and o.mean_jaccard(0) == 1 / 3


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_hits_match_the_stack_distance_characterisation(seed):
    # a most-recent-first list of size n hits a selection exactly when fewer
    # than n other experts were selected since that expert's previous selection
    rng = np.random.default_rng(seed)
    P, L, k, E = 40, 3, 3, 12
    idx, w = _random_trace(rng, P, L, k, E, pool=9)
    caps = [1, 2, 3, 4, 5, 8, 12]
    o = RouteLocality(L, E, k, caps=caps)
    o.record_trace(idx, w)
    for layer in range(L):
        s = _stream(idx, layer, E)
        for ci, n in enumerate(caps):
            hits, wh = 0, 0.0
            for i, (e, p, j) in enumerate(s):
                prev = [q for q in range(i) if s[q][0] == e]
                if prev and len({s[q][0] for q in range(prev[-1] + 1, i)}) < n:
                    hits += 1
                    wh += float(w[p][layer][j])
            assert o.cache_hits[ci][layer] == hits, (layer, n)
            assert o.cache_weight_hits[ci][layer] == wh, (layer, n)


def test_closed_forms_at_size_one_and_at_full_size():
    rng = np.random.default_rng(7)
    P, L, k, E = 60, 2, 2, 6
    idx, w = _random_trace(rng, P, L, k, E)
    o = RouteLocality(L, E, k, caps=[1, E])
    o.record_trace(idx, w)
    for layer in range(L):
        s = [e for e, _, _ in _stream(idx, layer, E)]
        # size 1 holds the previous selection only
        assert o.cache_hits[0][layer] == sum(1 for i in range(1, len(s)) if s[i] == s[i - 1])
        # a list as large as the expert set never evicts: only first selections miss
        assert o.cache_hits[1][layer] == len(s) - len(set(s))


def test_hits_grow_with_the_cache_size():
    rng = np.random.default_rng(3)
    idx, w = _random_trace(rng, 80, 2, 4, 32, pool=20)
    o = RouteLocality(2, 32, 4)
    assert o.caps == [1, 2, 4, 8, 16, 32]
    o.record_trace(idx, w)
    for layer in range(2):
        hits = [o.cache_hits[ci][layer] for ci in range(len(o.caps))]
        assert hits == sorted(hits)  # inclusion: a larger list holds a smaller one
        assert hits[-1] == 80 * 4 - len(set(idx[:, layer].ravel().tolist()))


def test_cache_sizes_follow_the_expert_count():
    assert cache_sizes_for(8) == [1, 2, 4, 8]
    assert cache_sizes_for(256) == [1, 2, 4, 8, 16, 32, 64, 128, 256]
    assert cache_sizes_for(384) == [1, 2, 4, 8, 16, 32, 64, 128, 256, 384]


@pytest.mark.parametrize("prev, cur, overlap, jaccard", [
    ([0, 1, 2, 3], [3, 2, 1, 0], 1.0, 1.0),
    ([0, 1, 2, 3], [4, 5, 6, 7], 0.0, 0.0),
    ([0, 1, 2, 3], [9, 8, 3, 7], 0.25, 1 / 7),
    ([0, 1, 2, 3], [1, 2, 5, 6], 0.5, 2 / 6),
])
def test_adjacent_overlap_constructed(prev, cur, overlap, jaccard):
    o = RouteLocality(1, 10, 4, caps=[])
    o.record(0, 5, prev, [0.25] * 4)
    o.record(0, 6, cur, [0.25] * 4)
    assert o.adjacent_pairs == [1]
    assert o.mean_overlap(0) == overlap and o.mean_jaccard(0) == jaccard


def test_non_adjacent_positions_are_not_compared():
    o = RouteLocality(1, 10, 2, caps=[])
    o.record(0, 0, [1, 2], [0.5, 0.5])
    o.record(0, 2, [1, 2], [0.5, 0.5])  # position 1 is missing
    o.record(0, 3, [1, 3], [0.5, 0.5])
    assert o.adjacent_pairs == [1] and o.overlap_sum == [0.5]


def test_out_of_range_selections_count_only_in_the_adjacency():
    o = RouteLocality(1, 4, 2, caps=[4])
    o.record_trace([[[-1, 2]], [[-1, 5]]], [[[0.5, 0.5]], [[0.5, 0.5]]])
    assert o.hist == [[0, 0, 1, 0]] and o.cache_hits == [[0]]
    assert o.overlap_sum == [0.5]  # the two -1 slots match


def test_hotlist_ranks_count_then_weight_then_layer_then_expert():
    o = RouteLocality(2, 3, 1, caps=[])
    o.hist = [[2, 1, 2], [2, 0, 1]]
    o.weight_hist = [[0.5, 3.0, 0.75], [0.5, 0.0, 1.0]]
    assert o.hotlist() == [(0, 2), (0, 0), (1, 0), (0, 1), (1, 2), (1, 1)]
    assert o.ranked_experts(0) == [2, 0, 1] and o.ranked_experts(1) == [0, 2]


# ------------------------------------------------- library (host) vs oracle
def _oracle_of(idx, w, E, caps):
    P, L, k = idx.shape
    o = RouteLocality(L, E, k, caps=caps)
    o.record_trace(idx.tolist(), w.astype(np.float64).tolist())
    return o


def _assert_library_equals_oracle(idx, w, E, caps=None):
    import mxfp4_expert_ffn_amd as mx
    r = mx.moe_route_locality(idx, w, E, caps=caps)
    o = _oracle_of(idx, w, E, r["caps"].tolist())
    assert r["caps"].tolist() == o.caps
    assert r["hist"].tolist() == o.hist
    assert r["weight_hist"].tolist() == o.weight_hist  # same additions in the same order
    assert r["cache_hits"].tolist() == o.cache_hits
    assert r["cache_weight_hits"].tolist() == o.cache_weight_hits
    assert r["adjacent_pairs"].tolist() == o.adjacent_pairs
    assert r["overlap_sum"].tolist() == o.overlap_sum
    assert r["jaccard_sum"].tolist() == o.jaccard_sum
    order = mx.moe_route_hotlist(r["hist"], r["weight_hist"])
    E_ = r["hist"].shape[1]
    assert [(int(i) // E_, int(i) % E_) for i in order] == o.hotlist()
    return r, o


@pytest.mark.parametrize("seed", [0, 1])
def test_library_equals_oracle_on_random_traces(seed):
    rng = np.random.default_rng(seed)
    idx, w = _random_trace(rng, 50, 3, 4, 16, pool=11)
    _assert_library_equals_oracle(idx, w, 16)
    _assert_library_equals_oracle(idx, w, 16, caps=[3, 1, 16, 7])
    _assert_library_equals_oracle(idx, w, 16, caps=[])  # adjacency and histogram only


def _routed_trace(cfg, P, layers):
    """The oracle's own selections and route weights for P tokens, each layer
    routing the same seeded inputs (a locality trace needs only the routing)."""
    x, _ = make_activations(cfg, rows=P)
    idx = np.zeros((P, layers, cfg.k), np.int32)
    w = np.zeros((P, layers, cfg.k), np.float32)
    for l in range(layers):
        lay = make_layer(cfg, l)
        xn = x.astype(np.float64)
        if lay.norm_w is not None:
            xn = moe.rms_norm(xn, lay.norm_w, cfg.rms_eps)
        _, i, ww, _ = moe.route(xn, lay.router_w, lay.router_b, cfg.k, cfg.route_scale)
        idx[:, l], w[:, l] = i, ww
    return idx, w


@pytest.mark.parametrize("cid, P, layers", [(2, 64, 1), (4, 32, 2), (5, 24, 1)])
def test_library_equals_oracle_on_routed_traces(cid, P, layers):
    cfg = scaled(config_by_id(cid), T=P)
    idx, w = _routed_trace(cfg, P, layers)
    r, o = _assert_library_equals_oracle(idx, w, cfg.E)
    assert int(r["hist"].sum()) == P * layers * cfg.k
    assert r["caps"].tolist() == cache_sizes_for(cfg.E)
    # the route weights of a token sum to the route scale
    assert abs(float(r["weight_hist"].sum()) - P * layers * cfg.route_scale) < 1e-4 * P * layers


def test_library_locality_rejects_bad_arguments():
    import mxfp4_expert_ffn_amd as mx
    from mxfp4_expert_ffn_amd import _lib
    idx = np.zeros((2, 1, 2), np.int32)
    w = np.zeros((2, 1, 2), np.float32)
    for caps in ([0], [5], list(range(1, 18))):
        with pytest.raises(mx.MoeError):
            mx.moe_route_locality(idx, w, 4, caps=caps)
    with pytest.raises(mx.MoeError):
        mx.moe_route_locality(idx, w, 0)
    lib = _lib.load()
    out = _lib.MoeLocalityOut()  # NULL outputs
    assert lib.moe_route_locality(None, None, 0, 1, 1, 4, None, 0, ctypes.byref(out)) == \
        _lib.MOE_ERR_INVALID_ARG
    with pytest.raises(mx.MoeError):
        mx.moe_route_hotlist(np.zeros((1, 2), np.uint64), np.array([[np.nan, 0.0]]))
    # no positions: everything zero
    r = mx.moe_route_locality(np.zeros((0, 2, 3), np.int32), np.zeros((0, 2, 3), np.float32), 8)
    assert not r["hist"].any() and not r["adjacent_pairs"].any() and not r["cache_hits"].any()


# ---------------------------------------------------------------- GPU (C ABI)
@pytest.mark.gpu
def test_gpu_decode_trace_locality():
    import torch
    import mxfp4_expert_ffn_amd as mx
    from gpu_util import shape_of, upload
    from mxfp4_expert_ffn_amd.device import workspace
    cfg = config_by_id(4)
    P, L = 24, 2
    print(f"\n[case] locality: {P} T=1 decode positions through layers 0-1 of config 4", flush=True)
    x, _ = make_activations(cfg, rows=P)
    shape = shape_of(cfg, 1)
    ws = workspace(shape)
    dls = [upload(cfg, make_layer(cfg, l)) for l in range(L)]
    idx_d = torch.full((P, L, cfg.k), -1, dtype=torch.int32, device="cuda")
    w_d = torch.zeros((P, L, cfg.k), dtype=torch.float32, device="cuda")
    h = torch.from_numpy(x).cuda()
    inputs = np.zeros((L, P, cfg.H), np.float32)
    for p in range(P):
        cur = h[p:p + 1]
        for l, dl in enumerate(dls):
            inputs[l, p] = cur.cpu().numpy()[0]
            nxt = torch.empty_like(cur)
            mx.moe_forward_decode(shape, cur, dl.router_w, dl.router_b, dl.experts_copy(0), nxt, ws,
                                  norm_w=dl.norm_w,
                                  route_out=dict(topk_idx=idx_d[p, l:l + 1], topk_w=w_d[p, l:l + 1]))
            cur = nxt
    torch.cuda.synchronize()
    gidx, gw = idx_d.cpu().numpy(), w_d.cpu().numpy()
    for l in range(L):  # each layer's selections are the oracle's on the GPU's layer input
        lay = make_layer(cfg, l)
        xn = moe.rms_norm(inputs[l].astype(np.float64), lay.norm_w, cfg.rms_eps)
        _, oi, ow, _ = moe.route(xn, lay.router_w, lay.router_b, cfg.k, cfg.route_scale)
        assert np.array_equal(gidx[:, l], oi), l
        assert np.allclose(gw[:, l], ow, rtol=1e-5, atol=1e-6), l
    r, _ = _assert_library_equals_oracle(gidx, gw, cfg.E)
    assert int(r["hist"].sum()) == P * L * cfg.k
