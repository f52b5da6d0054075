"""DeepSeek-V4 routing variants on the GPU against the oracle: the
selection-only expert bias (workload 7) and hash routing by token id
(workload 8), through moe_route, moe_forward_prefill and moe_forward_decode.

Bars: expert indices and the permutation bit-exact (a biased selection may
differ only at a certified fp64 near-tie of logit + bias; hash routing has no
ties: the indices are the table rows); route weights within 1e-6 x
route_scale; block outputs within max |err| <= 2e-3 x RMS of the oracle
output. Page: antirez ds4.c `ds4_layer_weights`, `weights_validate_layout`,
`DS4_SHAPE_FLASH` (the routing arithmetic is a reading; see oracle/moe.py).
"""
import dataclasses

import numpy as np
import pytest
import torch

import mxfp4_expert_ffn_amd as mx
from mxfp4_expert_ffn_amd.device import workspace
from oracle import moe as omoe
from workloads import config_by_id, make_layer, make_token_ids, scaled
from workloads.gen import make_activations

from gpu_util import (TOL, check_permutation, check_routing, device_input, rel_err, route_buffers,
                      run_forward, shape_of, to_np, upload)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mx._lib.load()


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)


def _ids_dev(ids):
    return None if ids is None else torch.from_numpy(np.ascontiguousarray(ids, np.int32)).cuda()


@pytest.mark.parametrize("cid,T", [(7, 1), (7, 64), (7, 2048), (8, 1), (8, 64), (8, 2048)])
def test_route_parity(cid, T):
    cfg = config_by_id(cid)
    _announce(f"route config {cid} T={T}")
    layer = make_layer(scaled(cfg, F=32, n_shared=0))  # routing needs only the router
    x, xb = make_activations(cfg, rows=T)
    ids = make_token_ids(cfg, rows=T)
    dl = upload(scaled(cfg, F=32, n_shared=0), layer)
    shape = shape_of(cfg, T)
    ro = route_buffers(T, cfg.k, cfg.E)
    mx.moe_route(shape, device_input(cfg, x, xb), dl.router_w, dl.router_b, ro, workspace(shape),
                 routing=dl.routing(_ids_dev(ids)))
    torch.cuda.synchronize()
    got = to_np(ro)
    ref = omoe.block_for_config(scaled(cfg, F=32, n_shared=0), layer, x, tokens=np.arange(0),
                                token_ids=ids)
    check_routing(got["topk_idx"], got["topk_w"], ref, layer.router_w, layer.router_b,
                  cfg.route_scale)
    check_permutation(got, got["topk_idx"], cfg.E)
    if cid == 7:
        # the bias does move selections (else the test would not see it)
        plain = omoe.top_k(ref["logits"], cfg.k)
        assert np.mean(np.any(plain != ref["idx"], axis=1)) > 0.2


@pytest.mark.parametrize("cid,T,sample", [(7, 2048, 48), (8, 2048, 48), (7, 256, None),
                                          (8, 256, None)])
def test_prefill_block(cid, T, sample):
    cfg = scaled(config_by_id(cid), T=T)
    _announce(f"prefill config {cid} T={T}")
    layer = make_layer(cfg)
    x, xb = make_activations(cfg)
    ids = make_token_ids(cfg)
    dl = upload(cfg, layer)
    out, ro = run_forward("prefill", shape_of(cfg), dl, device_input(cfg, x, xb),
                          token_ids=_ids_dev(ids))
    ro = to_np(ro)
    toks = None if sample is None else np.random.default_rng(cid).choice(T, sample, replace=False)
    ref = omoe.block_for_config(cfg, layer, x, tokens=toks, token_ids=ids)
    check_routing(ro["topk_idx"], ro["topk_w"], ref, layer.router_w, layer.router_b,
                  cfg.route_scale)
    check_permutation(ro, ro["topk_idx"], cfg.E)
    tk = ref["tokens"]
    err = rel_err(out.cpu().numpy()[tk], x[tk] + ref["delta"])
    print(f"config {cid} T={T} prefill: max|err|/rms = {err:.2e}")
    assert err <= TOL


@pytest.mark.parametrize("cid,T", [(7, 1), (7, 8), (8, 1), (8, 8)])
def test_decode_block(cid, T):
    cfg = scaled(config_by_id(cid), T=T)
    _announce(f"decode config {cid} T={T}")
    layer = make_layer(cfg)
    x, xb = make_activations(cfg)
    ids = make_token_ids(cfg)
    dl = upload(cfg, layer)
    out, ro = run_forward("decode", shape_of(cfg), dl, device_input(cfg, x, xb),
                          token_ids=_ids_dev(ids))
    ro = to_np(ro)
    ref = omoe.block_for_config(cfg, layer, x, token_ids=ids)
    check_routing(ro["topk_idx"], ro["topk_w"], ref, layer.router_w, layer.router_b,
                  cfg.route_scale)
    err = rel_err(out.cpu().numpy(), x + ref["delta"])
    print(f"config {cid} T={T} decode: max|err|/rms = {err:.2e}")
    assert err <= TOL


def test_hash_ids_and_entries_out_of_range_are_clamped():
    """Documented behaviour: ids outside [0, vocab) and table entries outside
    [0, E) are clamped into range; the oracle run on the clamped inputs gives
    the same routing."""
    cfg = scaled(config_by_id(8), T=16, hash_vocab=40, F=32, n_shared=0)
    _announce("hash routing: out-of-range ids and table entries")
    layer = make_layer(cfg)
    tab = layer.tid2eid.copy()
    tab[3, 0] = -5
    tab[7, 2] = cfg.E + 9
    layer = dataclasses.replace(layer, tid2eid=tab)
    ids = np.arange(cfg.T, dtype=np.int32) * 3 - 4      # -4 .. 41: both ends out of range
    ids[5] = 3
    ids[6] = 7
    x, xb = make_activations(cfg)
    dl = upload(cfg, layer)
    shape = shape_of(cfg)
    ro = route_buffers(cfg.T, cfg.k, cfg.E)
    mx.moe_route(shape, device_input(cfg, x, xb), dl.router_w, dl.router_b, ro, workspace(shape),
                 routing=dl.routing(_ids_dev(ids)))
    torch.cuda.synchronize()
    got = to_np(ro)
    clamped = dataclasses.replace(layer, tid2eid=np.clip(tab, 0, cfg.E - 1))
    ref = omoe.block_for_config(cfg, clamped, x, tokens=np.arange(0),
                                token_ids=np.clip(ids, 0, cfg.hash_vocab - 1))
    check_routing(got["topk_idx"], got["topk_w"], ref, layer.router_w, layer.router_b,
                  cfg.route_scale)


@pytest.mark.parametrize("cid", [7, 8])
def test_route_and_decode_select_alike(cid):
    cfg = scaled(config_by_id(cid), T=8, F=256)
    _announce(f"route vs decode selections, config {cid}")
    layer = make_layer(cfg)
    x, xb = make_activations(cfg)
    ids = _ids_dev(make_token_ids(cfg))
    dl = upload(cfg, layer)
    shape = shape_of(cfg)
    xd = device_input(cfg, x, xb)
    ro_r = route_buffers(cfg.T, cfg.k, cfg.E)
    mx.moe_route(shape, xd, dl.router_w, dl.router_b, ro_r, workspace(shape),
                 routing=dl.routing(ids))
    _, ro_d = run_forward("decode", shape, dl, xd, token_ids=ids)
    torch.cuda.synchronize()
    assert torch.equal(ro_r["topk_idx"], ro_d["topk_idx"])
    assert torch.equal(ro_r["topk_w"], ro_d["topk_w"])
