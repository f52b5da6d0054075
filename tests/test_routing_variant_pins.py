"""Pins of the oracle's DeepSeek-V4 routing variants (oracle/moe.py
`select_experts`, `route`, `moe_block`): the selection-only expert bias and
hash routing by token id.

What fixes them: brute force over k-subsets (oracle/brute.py, pure Python,
which ranks logit + bias itself), closed forms of the softmax on constructed
routers, a hash table that names the experts a constructed router would pick,
and invariances of the readings (a constant added to every bias moves nothing;
a zero bias is plain routing; the logits of unselected experts do not move a
hash-routed token). Page: antirez `ds4.c` `ds4_layer_weights`,
`weights_validate_layout` (exp_probs_b [n_expert]; tid2eid [n_expert_used,
n_vocab] for layers below n_hash_layer), `DS4_SHAPE_FLASH`.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import pytest

from oracle import brute
from oracle import moe as omoe
from workloads import config_by_id, make_layer, make_token_ids, scaled
from workloads.gen import distinct_rows, make_activations


def _softmax_closed_form(vals, scale):
    m = max(vals)
    z = [math.exp(v - m) for v in vals]
    s = math.fsum(z)
    return [scale * v / s for v in z]


def test_zero_bias_is_plain_routing_and_constant_shift_moves_nothing():
    rng = np.random.default_rng(1)
    logits = rng.normal(size=(40, 16))
    plain = omoe.top_k(logits, 4)
    idx0, _ = omoe.select_experts(logits, 4, sel_bias=np.zeros(16))
    assert np.array_equal(idx0, plain)
    bias = rng.normal(size=16)
    a, _ = omoe.select_experts(logits, 4, sel_bias=bias)
    b, _ = omoe.select_experts(logits, 4, sel_bias=bias + 3.0)  # exact shift in float64 here
    assert np.array_equal(a, b)


@pytest.mark.parametrize("seed", range(6))
def test_biased_selection_matches_subset_enumeration(seed):
    rng = np.random.default_rng(seed)
    E, k = 7, 3
    logits = rng.normal(size=(5, E))
    bias = rng.normal(scale=0.7, size=E)
    idx, sel = omoe.select_experts(logits, k, sel_bias=bias)
    w = omoe.route_weights(logits, idx, 1.5)
    for t in range(5):
        want = brute.top_k_bruteforce([float(logits[t, e]) + float(bias[e]) for e in range(E)], k)
        assert idx[t].tolist() == want
        cf = _softmax_closed_form([float(logits[t, e]) for e in want], 1.5)
        assert np.allclose(w[t], cf, rtol=1e-14, atol=0)
        assert np.array_equal(sel[t], logits[t] + bias)


def test_forced_expert_takes_its_unbiased_weight():
    """A bias large enough forces an expert in; its weight still comes from
    its own (low) logit: exp(l_e) / sum over the selected exp(l)."""
    logits = np.array([[2.0, 1.0, 0.5, -3.0, 0.0]])
    bias = np.array([0.0, 0.0, 0.0, 10.0, 0.0])
    idx, _ = omoe.select_experts(logits, 2, sel_bias=bias)
    assert idx.tolist() == [[3, 0]]          # biased values 7.0 and 2.0, in that order
    w = omoe.route_weights(logits, idx, 1.0)
    e3, e0 = math.exp(-3.0), math.exp(2.0)
    assert w[0].tolist() == pytest.approx([e3 / (e3 + e0), e0 / (e3 + e0)], rel=1e-15)


def test_bias_ties_go_to_the_lower_index():
    logits = np.array([[0.0, 1.0, 0.5, 1.5]])
    bias = np.array([1.5, 0.5, 1.0, 0.0])   # every biased value is 1.5
    idx, _ = omoe.select_experts(logits, 3, sel_bias=bias)
    assert idx.tolist() == [[0, 1, 2]]


def _diag_layer(E, H, diag, router_b=None, sel_bias=None, tid2eid=None):
    """A layer whose router is diag(a) on the first E hidden units (logit e of
    token t = a_e * x[t, e] + b_e exactly), with tiny experts."""
    cfg = scaled(config_by_id(1), H=H, F=32, E=E, k=2, T=3)
    base = make_layer(cfg)
    rw = np.zeros((E, H), np.float32)
    rw[np.arange(E), np.arange(E)] = diag
    rb = np.zeros(E, np.float32) if router_b is None else np.asarray(router_b, np.float32)
    return dataclasses.replace(base, router_w=rw, router_b=rb, sel_bias=sel_bias, tid2eid=tid2eid)


def test_hash_rows_take_the_table_experts_with_closed_form_weights():
    E, H, k = 8, 32, 2
    table = np.array([[5, 1], [0, 7], [3, 2], [6, 4]], np.int32)
    lay = _diag_layer(E, H, np.full(E, 0.5, np.float32), tid2eid=table)
    x = np.zeros((3, H), np.float32)
    x[:, :E] = np.arange(3 * E, dtype=np.float32).reshape(3, E) / 4.0
    ids = np.array([3, 0, 1])
    r = omoe.moe_block(lay, x, k, 1.0, 10.0, 0.0, route_scale=1.5, token_ids=ids)
    assert r["idx"].tolist() == table[ids].tolist()
    for t in range(3):
        lg = [0.5 * float(x[t, e]) for e in table[ids[t]]]
        assert np.allclose(r["w"][t], _softmax_closed_form(lg, 1.5), rtol=1e-14, atol=0)
    # moving the logits of experts outside a token's row changes neither its
    # experts nor its weights
    x2 = x.copy()
    for t in range(3):
        others = [e for e in range(E) if e not in table[ids[t]]]
        x2[t, others] += 100.0
    r2 = omoe.moe_block(lay, x2, k, 1.0, 10.0, 0.0, route_scale=1.5, token_ids=ids)
    assert np.array_equal(r2["idx"], r["idx"]) and np.array_equal(r2["w"], r["w"])


def test_table_naming_a_routers_choice_equals_that_routing():
    """A router whose logits are known by construction (diag router on
    distinct inputs), and a table row per token listing its top-k by hand:
    hash routing and plain routing agree on experts, weights and output."""
    E, H, k, T = 8, 32, 3, 4
    rng = np.random.default_rng(4)
    x = np.zeros((T, H), np.float32)
    order = [rng.permutation(E) for _ in range(T)]
    for t in range(T):
        x[t, order[t]] = np.arange(E, 0, -1, dtype=np.float32)   # expert order[t][0] largest
    table = np.array([order[t][:k] for t in range(T)], np.int32)
    plain = _diag_layer(E, H, np.full(E, 0.25, np.float32))
    hashed = dataclasses.replace(plain, tid2eid=table)
    a = omoe.moe_block(plain, x, k, 1.0, 10.0, 0.0, route_scale=1.5)
    b = omoe.moe_block(hashed, x, k, 1.0, 10.0, 0.0, route_scale=1.5, token_ids=np.arange(T))
    assert a["idx"].tolist() == table.tolist()
    assert np.array_equal(a["idx"], b["idx"]) and np.array_equal(a["w"], b["w"])
    assert np.array_equal(a["out"], b["out"])


@pytest.mark.parametrize("variant", ["sel_bias", "hash"])
def test_block_matches_pure_python_brute_force(variant):
    cfg = scaled(config_by_id(1), T=3, H=64, F=32, E=6, k=2)
    lay = make_layer(cfg)
    rng = np.random.default_rng(17)
    ids = None
    if variant == "sel_bias":
        lay = dataclasses.replace(lay, sel_bias=rng.normal(scale=0.1, size=6).astype(np.float32))
    else:
        lay = dataclasses.replace(lay, tid2eid=distinct_rows(rng, 11, 6, 2))
        ids = np.array([10, 3, 3])
    x, _ = make_activations(cfg)
    r = omoe.moe_block(lay, x, cfg.k, cfg.alpha, cfg.limit, cfg.up_offset, cfg.route_scale,
                       token_ids=ids)
    outs, idxs, ws = brute.block(lay, x, cfg.k, cfg.alpha, cfg.limit, cfg.up_offset,
                                 route_scale=cfg.route_scale, token_ids=ids)
    assert r["idx"].tolist() == idxs
    assert np.allclose(r["w"], ws, rtol=1e-13, atol=0)
    assert np.allclose(r["out"], np.asarray(outs, np.float32), rtol=1e-6, atol=1e-6)


def test_hash_routing_rejects_bad_rows():
    logits = np.zeros((2, 4))
    with pytest.raises(ValueError):
        omoe.select_experts(logits, 2, hash_rows=np.array([[0, 4], [1, 2]]))
    with pytest.raises(ValueError):
        omoe.select_experts(logits, 2, hash_rows=np.array([[0, 1]]))


def test_variant_workloads_are_well_formed():
    c7, c8 = config_by_id(7), config_by_id(8)
    l7 = make_layer(scaled(c7, T=4, H=64, F=32))
    assert l7.sel_bias.shape == (256,) and l7.sel_bias.dtype == np.float32 and l7.tid2eid is None
    assert 0.4 < float(np.std(l7.sel_bias)) < 0.6
    l8 = make_layer(scaled(c8, T=4, H=64, F=32))
    t = l8.tid2eid
    assert t.shape == (129280, 6) and t.dtype == np.int32
    assert t.min() >= 0 and t.max() < 256
    assert np.all(np.sort(t, axis=1)[:, 1:] != np.sort(t, axis=1)[:, :-1])  # distinct per row
    ids = make_token_ids(c8)
    assert ids.shape == (2048,) and ids.min() >= 0 and ids.max() < 129280
    assert make_token_ids(config_by_id(5)) is None
