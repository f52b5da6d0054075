"""Parity of the HIP path (called through the C ABI) with the CPU oracle.

Bars: expert indices, token permutation and dequantised weights bit-exact;
route weights within 1e-6; block outputs within max |err| <= 2e-3 x RMS of
the oracle output. Indices may differ only at certified fp64 near-ties
(counted; expected none).
"""
import numpy as np
import pytest
import torch

import mxfp4_expert_ffn_amd as mx
from mxfp4_expert_ffn_amd.device import workspace
from oracle import moe as omoe
from oracle import mxfp4 as omx
from workloads import config_by_id, make_layer, scaled
from workloads.gen import ExpertPlanes, Layer, make_activations

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


# ---------------------------------------------------------------- dequant
def _dequant_gpu(shape, blob, which, path):
    rows, K = (shape.H, shape.F) if which == 2 else (shape.F, shape.H)
    out = torch.empty((rows, K), dtype=torch.float32, device="cuda")
    mx.moe_dequant_debug(shape, blob, which, path, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _same(got, ref, path):
    """Paths 0 and 1 export the decoded bits; the matrix core (path 2) adds
    each product to a +0 accumulator, so a -0 weight comes out as +0: there
    the values must be equal (every nonzero bit pattern still matches)."""
    if path == 2:
        return np.array_equal(got, ref) and np.array_equal(got[got != 0].view(np.uint32),
                                                           ref[ref != 0].view(np.uint32))
    return got.tobytes() == ref.tobytes()


def _planes(layer_planes, e, which):
    names = [("gate_codes", "gate_scales"), ("up_codes", "up_scales"), ("down_codes", "down_scales")]
    q, s = names[which]
    return getattr(layer_planes, q)[e], getattr(layer_planes, s)[e]


def test_dequant_bitexact_all_codes_and_scales():
    _announce("dequant exhaustive codes x scale bytes 2..252")
    H = F = 512
    shape = mx.make_shape(1, H, F, 1, 1)
    codes = np.arange(F * H, dtype=np.int64).reshape(F, H) % 16
    # vary the code pattern per row so nibble pairs differ
    codes = (codes + np.arange(F)[:, None]) % 16
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    sb = (2 + (np.arange(F * H // 32) % 251)).astype(np.uint8).reshape(F, H // 32)
    bias = np.zeros((1, F), np.float32)
    planes = ExpertPlanes(packed[None], sb[None], bias, packed[None], sb[None], bias,
                          packed[None], sb[None], bias)
    blob = torch.from_numpy(mx.moe_pack_experts(shape, planes)).cuda()
    ref = omx.dequant(packed, sb).astype(np.float32)
    for which in range(3):
        for path in (0, 1, 2):
            got = _dequant_gpu(shape, blob, which, path)
            assert _same(got, ref, path), (which, path)


@pytest.mark.parametrize("cid,experts", [(1, None), (2, (0, 7, 19, 31)), (5, (3, 128))])
def test_dequant_bitexact_config_weights(cid, experts):
    cfg = config_by_id(cid)
    if cid == 5:
        cfg = scaled(cfg, E=130)
    _announce(f"dequant config {cid}")
    layer = make_layer(cfg)
    shape = shape_of(cfg)
    stride = mx.moe_blob_layout_get(shape)["stride"]
    blobs = torch.from_numpy(mx.moe_pack_experts(shape, layer.experts)).cuda()
    sel = range(cfg.E) if experts is None else experts
    for e in sel:
        blob = blobs[e * stride:(e + 1) * stride]
        for which in range(3):
            ref = omx.dequant(*_planes(layer.experts, e, which)).astype(np.float32)
            for path in (0, 1, 2):
                assert _same(_dequant_gpu(shape, blob, which, path), ref, path), (e, which, path)


# ---------------------------------------------------------------- routing
@pytest.mark.parametrize("cid,T", [(1, 8), (2, 16), (2, 1000), (3, 128), (4, 512), (5, 2048),
                                   (6, 2048)])
def test_route_parity(cid, T):
    cfg = config_by_id(cid)
    _announce(f"route config {cid} T={T}")
    # routing only needs the router; keep the experts tiny
    layer = make_layer(scaled(cfg, F=32, n_shared=0))
    x, xb = make_activations(cfg, rows=T)
    shape = shape_of(cfg, T)
    ro = route_buffers(T, cfg.k, cfg.E)
    nw = None if layer.norm_w is None else torch.from_numpy(layer.norm_w).cuda()
    mx.moe_route(shape, device_input(cfg, x, xb), torch.from_numpy(layer.router_w).cuda(),
                 torch.from_numpy(layer.router_b).cuda(), ro, workspace(shape), norm_w=nw)
    torch.cuda.synchronize()
    got = to_np(ro)
    xn = x.astype(np.float64) if layer.norm_w is None else omoe.rms_norm(x, layer.norm_w, cfg.rms_eps)
    logits, idx, w, _ = omoe.route(xn, layer.router_w, layer.router_b, cfg.k, cfg.route_scale)
    ref = dict(logits=logits, idx=idx, w=w, xn=xn)
    check_routing(got["topk_idx"], got["topk_w"], ref, layer.router_w, layer.router_b,
                  cfg.route_scale)
    check_permutation(got, got["topk_idx"], cfg.E)


# routes (T * k) at and around the 1024-route chunks the permutation works in,
# with the largest expert count and with every token's first choice forced onto
# one expert (its count spans chunks)
@pytest.mark.parametrize("T,k,E,skew", [(1023, 1, 8, False), (1024, 1, 16, False), (1025, 1, 16, False),
                                        (512, 2, 512, False), (683, 3, 300, False), (700, 3, 24, True),
                                        (2048, 6, 257, True)])
def test_permutation_at_chunk_edges(T, k, E, skew):
    _announce(f"permutation T={T} k={k} E={E} skew={skew}")
    H = 64
    rng = np.random.default_rng(T * 31 + E)
    rw = rng.normal(0.0, 0.05, size=(E, H)).astype(np.float32)
    rb = rng.normal(0.0, 0.05, size=E).astype(np.float32)
    if skew:
        rb[E // 3] = 50.0  # every token's first choice
    x = rng.normal(0.0, 1.0, size=(T, H)).astype(np.float32)
    shape = mx.make_shape(T, H, 32, E, k)
    ro = route_buffers(T, k, E)
    mx.moe_route(shape, torch.from_numpy(x).cuda(), torch.from_numpy(rw).cuda(),
                 torch.from_numpy(rb).cuda(), ro, workspace(shape))
    torch.cuda.synchronize()
    got = to_np(ro)
    if skew:
        assert np.all(got["topk_idx"][:, 0] == E // 3)
    logits, idx, w, _ = omoe.route(x.astype(np.float64), rw, rb, k, 1.0)
    check_routing(got["topk_idx"], got["topk_w"], dict(logits=logits, idx=idx, w=w, xn=x.astype(np.float64)),
                  rw, rb, 1.0)
    check_permutation(got, got["topk_idx"], E)


def test_route_ties_go_to_lowest_index():
    _announce("route ties")
    T, H, E, k = 5, 64, 16, 4
    shape = mx.make_shape(T, H, 32, E, k)
    rw = np.zeros((E, H), np.float32)
    rw[9] = rw[3] = 0.01          # experts 3 and 9 tie above the rest
    rb = np.zeros(E, np.float32)
    rb[12] = 1.0
    x = np.ones((T, H), np.float32)
    x[1] = 0.0                    # token 1: all logits equal to the bias
    x[2] *= -0.0
    ro = route_buffers(T, k, E)
    mx.moe_route(shape, torch.from_numpy(x).cuda(), torch.from_numpy(rw).cuda(),
                 torch.from_numpy(rb).cuda(), ro, workspace(shape))
    torch.cuda.synchronize()
    got = to_np(ro)
    ref = omoe.top_k(omoe.router_logits(x, rw, rb), k)
    assert np.array_equal(got["topk_idx"], ref)
    assert got["topk_idx"][1].tolist() == [12, 0, 1, 2]
    check_permutation(got, got["topk_idx"], E)


# ---------------------------------------------------------------- whole block
def _oracle(cfg, layer, x, tokens=None, stats=None):
    return omoe.block_for_config(cfg, layer, x, tokens=tokens, stats=stats)


def _check_block(cfg, layer, x, out, ro, tokens=None):
    ref = _oracle(cfg, layer, x, tokens)
    toks = ref["tokens"]
    err = rel_err(out[toks], x[toks] + ref["delta"])
    check_routing(ro["topk_idx"], ro["topk_w"], ref, layer.router_w, layer.router_b,
                  cfg.route_scale)
    assert err <= TOL, f"max|err|/rms = {err:.3e}"
    return err


@pytest.mark.parametrize("path", ["decode", "prefill"])
def test_block_tiny_config(path):
    cfg = config_by_id(1)
    _announce(f"block config 1 {path}")
    layer = make_layer(cfg)
    x, xb = make_activations(cfg)
    dl = upload(cfg, layer)
    out, ro = run_forward(path, shape_of(cfg), dl, device_input(cfg, x, xb))
    ro = to_np(ro)
    err = _check_block(cfg, layer, x, out.cpu().numpy(), ro)
    check_permutation(ro, ro["topk_idx"], cfg.E)
    print(f"config 1 {path}: max|err|/rms = {err:.2e}")


def test_decode_gptoss_tokens():
    cfg = config_by_id(2)
    _announce("decode config 2, 64 sampled tokens as T=1 calls")
    layer = make_layer(cfg)
    x, _ = make_activations(cfg)
    dl = upload(cfg, layer)
    shape = shape_of(cfg, 1)
    toks = np.random.default_rng(0).choice(x.shape[0], 64, replace=False)
    xd = torch.from_numpy(x).cuda()
    out = torch.empty_like(xd)
    ws = workspace(shape)
    ro = route_buffers(x.shape[0], cfg.k, cfg.E)
    for t in toks:
        r1 = {k: v[t:t + 1] if k in ("topk_idx", "topk_w") else None for k, v in ro.items()}
        mx.moe_forward_decode(shape, xd[t:t + 1], dl.router_w, dl.router_b, dl.experts_copy(0),
                              out[t:t + 1], ws, route_out=r1)
    torch.cuda.synchronize()
    ref = _oracle(cfg, layer, x, tokens=toks)
    got_idx = ro["topk_idx"].cpu().numpy()[toks]
    ridx = ref["idx"][toks]
    sub = dict(logits=ref["logits"][toks], idx=ridx, w=ref["w"][toks], xn=ref["xn"][toks])
    check_routing(got_idx, ro["topk_w"].cpu().numpy()[toks], sub, layer.router_w, layer.router_b, 1.0)
    err = rel_err(out.cpu().numpy()[toks], x[toks] + ref["delta"])
    print(f"config 2 decode: max|err|/rms = {err:.2e}")
    assert err <= TOL


def test_prefill_gptoss_zipf_full():
    cfg = config_by_id(3)
    _announce("prefill config 3 T=128 (all tokens checked)")
    layer = make_layer(cfg)
    x, _ = make_activations(cfg)
    dl = upload(cfg, layer)
    out, ro = run_forward("prefill", shape_of(cfg), dl, device_input(cfg, x, None))
    ro = to_np(ro)
    stats = {}
    ref = _oracle(cfg, layer, x, stats=stats)
    check_routing(ro["topk_idx"], ro["topk_w"], ref, layer.router_w, layer.router_b, 1.0)
    check_permutation(ro, ro["topk_idx"], cfg.E)
    err = rel_err(out.cpu().numpy(), x + ref["delta"])
    print(f"config 3 prefill: max|err|/rms = {err:.2e}; loads {np.bincount(ro['topk_idx'].ravel(), minlength=32).tolist()}")
    assert stats["gate_clamped"] > 0 and stats["up_clamped"] > 0
    assert err <= TOL


def test_prefill_ds4_flash_full_size_sampled():
    cfg = config_by_id(5)
    _announce("prefill config 5 T=2048 (64 sampled tokens checked)")
    layer = make_layer(cfg)
    x, xb = make_activations(cfg)
    dl = upload(cfg, layer)
    out, ro = run_forward("prefill", shape_of(cfg), dl, device_input(cfg, x, xb))
    ro = to_np(ro)
    toks = np.random.default_rng(5).choice(cfg.T, 64, replace=False)
    ref = _oracle(cfg, layer, x, tokens=toks)
    check_routing(ro["topk_idx"], ro["topk_w"], ref, layer.router_w, layer.router_b, 1.5)
    check_permutation(ro, ro["topk_idx"], cfg.E)
    err = rel_err(out.cpu().numpy()[toks], x[toks] + ref["delta"])
    print(f"config 5 prefill: max|err|/rms = {err:.2e}")
    assert err <= TOL


def test_ds4_pro_full_size_sampled():
    """The DeepSeek-V4-Pro shape (H=7168, F=3072, 384 experts top-6 + shared,
    route scale 2.5) at T=2048: prefill on 16 sampled tokens, and 4 tokens as
    T=1 decode calls."""
    cfg = config_by_id(6)
    _announce("prefill config 6 (DS4-Pro shape) T=2048 (16 sampled tokens) + 4 decode calls")
    layer = make_layer(cfg)
    x, xb = make_activations(cfg)
    dl = upload(cfg, layer)
    xd = device_input(cfg, x, xb)
    out, ro = run_forward("prefill", shape_of(cfg), dl, xd)
    ro = to_np(ro)
    toks = np.random.default_rng(6).choice(cfg.T, 16, replace=False)
    ref = _oracle(cfg, layer, x, tokens=toks)
    check_routing(ro["topk_idx"], ro["topk_w"], ref, layer.router_w, layer.router_b, 2.5)
    check_permutation(ro, ro["topk_idx"], cfg.E)
    err = rel_err(out.cpu().numpy()[toks], x[toks] + ref["delta"])
    print(f"config 6 prefill: max|err|/rms = {err:.2e}")
    assert err <= TOL
    shape1 = shape_of(cfg, 1)
    ws1 = workspace(shape1)
    dec = torch.full((4, cfg.H), float("nan"), dtype=torch.float32, device="cuda")
    for i, t in enumerate(toks[:4]):
        mx.moe_forward_decode(shape1, xd[t:t + 1], dl.router_w, dl.router_b, dl.experts_copy(0),
                              dec[i:i + 1], ws1, shared=dl.shared_copy(0))
    torch.cuda.synchronize()
    err = rel_err(dec.cpu().numpy(), x[toks[:4]] + ref["delta"][:4])
    print(f"config 6 decode: max|err|/rms = {err:.2e}")
    assert err <= TOL


def test_prefill_stack24_teacher_forced():
    cfg = config_by_id(4)
    _announce("prefill config 4: 24 layers T=512, per-layer teacher forcing")
    x, _ = make_activations(cfg)
    shape = shape_of(cfg)
    h = torch.from_numpy(x).cuda()
    ws = workspace(shape)
    check_layers = {0, 4, 9, 14, 19, 23}
    rng = np.random.default_rng(4)
    worst = 0.0
    for l in range(cfg.layers):
        layer = make_layer(cfg, l)
        dl = upload(cfg, layer)
        ro = route_buffers(cfg.T, cfg.k, cfg.E)
        out = torch.empty_like(h)
        mx.moe_forward_prefill(shape, h, dl.router_w, dl.router_b, dl.experts_copy(0), out, ws,
                               norm_w=dl.norm_w, route_out=ro)
        torch.cuda.synchronize()
        hin = h.cpu().numpy()
        got = to_np(ro)
        toks = rng.choice(cfg.T, 32, replace=False) if l in check_layers else np.array([0])
        ref = _oracle(cfg, layer, hin, tokens=toks)
        check_routing(got["topk_idx"], got["topk_w"], ref, layer.router_w, layer.router_b, 1.0)
        check_permutation(got, got["topk_idx"], cfg.E)
        if l in check_layers:
            err = rel_err(out.cpu().numpy()[toks], hin[toks] + ref["delta"])
            worst = max(worst, err)
            assert err <= TOL, (l, err)
        h = out
        del dl
    print(f"config 4 stack: worst per-layer max|err|/rms = {worst:.2e}")


def test_config4_decode_stack():
    """T=1 decode through the 24 layers of config 4 (RMSNorm + MoE each), the
    output of each layer the input of the next; every layer's routing and
    layers 0, 11 and 23's outputs against the oracle on the GPU's own layer
    input (teacher forcing)."""
    cfg = config_by_id(4)
    _announce("decode config 4 layers: one token at T=1 through 24 layers, teacher forcing")
    x, _ = make_activations(cfg, rows=1)
    shape = shape_of(cfg, 1)
    h = torch.from_numpy(x).cuda()
    ws = workspace(shape)
    check_layers = {0, 11, 23}
    worst = 0.0
    for l in range(cfg.layers):
        layer = make_layer(cfg, l)
        dl = upload(cfg, layer)
        ro = route_buffers(1, cfg.k, cfg.E)
        out = torch.full_like(h, float("nan"))
        mx.moe_forward_decode(shape, h, dl.router_w, dl.router_b, dl.experts_copy(0), out, ws,
                              norm_w=dl.norm_w, route_out=ro)
        torch.cuda.synchronize()
        hin = h.cpu().numpy()
        got = to_np(ro)
        ref = _oracle(cfg, layer, hin)
        check_routing(got["topk_idx"], got["topk_w"], ref, layer.router_w, layer.router_b, 1.0)
        check_permutation(got, got["topk_idx"], cfg.E)
        if l in check_layers:
            err = rel_err(out.cpu().numpy(), hin + ref["delta"])
            worst = max(worst, err)
            assert err <= TOL, (l, err)
        h = out
        del dl
    print(f"config 4 decode stack: worst per-layer max|err|/rms = {worst:.2e}")


# ---------------------------------------------------------------- edge cases
def _small(cid, **kw):
    return scaled(config_by_id(cid), **kw)


EDGE = {
    "ragged": _small(3, T=37, H=320, F=320, E=5, k=3),
    "single_expert": _small(1, T=9, E=1, k=1),
    "k_equals_E": _small(1, T=6, E=4, k=4),
    "crowded": _small(1, T=50, E=2, k=2, H=192, F=96),
    # past 96 rows per expert: the grouped GEMMs take 32-row tiles
    "deep_tiles": _small(1, T=120, E=2, k=2, H=192, F=160),
    "bf16_shared_scale": _small(5, T=19, H=256, F=128, E=12, k=6),
    "norm": _small(4, T=21, H=256, F=192, E=8, k=4, layers=1),
    "max_H": _small(1, T=3, H=16384, F=64, E=2, k=1),
    "max_F_decode": _small(1, T=2, H=64, F=8192, E=2, k=2),
    # no clamp in effect: activations are unbounded, the FP8-term scales follow
    "unclamped": _small(1, T=7, E=4, k=2, limit=1e30),
    # widths that end in a partial 128-wide step (3 and 5 MX blocks)
    "narrow": _small(2, T=11, H=96, F=160, E=6, k=3),
    # a decode batch past the GEMV router (tiled router + its own quantise)
    "decode_T40": _small(2, T=40, H=512, F=384, E=16, k=4),
    # more than 256 experts: eight per lane in the top-k, a ninth bit plane in
    # the permutation (the DS4-Pro expert count, and the maximum with k = 8)
    "pro_experts": _small(6, T=64, H=256, F=128, E=384, k=6),
    "max_E": _small(1, T=40, H=128, F=64, E=512, k=8),
    # a group with 16 tiles and 20 gate/up row blocks (the shared expert here)
    # runs tile by tile in the grouped GEMMs
    "tile_major": _small(5, T=256, H=256, F=2560, E=4, k=2),
    # the largest expert hidden size the library takes (prefill only; decode
    # stops at 8192)
    "max_F": _small(1, T=3, H=64, F=16384, E=2, k=1),
    # the largest decode batch, bf16 input with a shared expert
    "decode_T64": _small(5, T=64, H=256, F=128, E=12, k=6),
    # the prefill gate/up's bfloat16 operand on widths that end in a partial
    # 128-wide step: 32-row tiles over H = 2880 (22.5 steps), and 16-row
    # tiles over H = 96 (one partial step)
    "bf16_ragged_K": _small(5, T=45, H=2880, F=352, E=8, k=4),
    "bf16_narrow": _small(5, T=11, H=96, F=160, E=6, k=3),
}


@pytest.mark.parametrize("name", sorted(EDGE))
@pytest.mark.parametrize("path", ["decode", "prefill"])
def test_edge_cases(name, path):
    cfg = EDGE[name]
    if path == "decode" and (cfg.T > 64 or cfg.H > 8192 or cfg.F > 8192):
        pytest.skip("outside decode limits")
    _announce(f"edge {name} {path}")
    layer = make_layer(cfg)
    x, xb = make_activations(cfg, rows=cfg.T)
    dl = upload(cfg, layer)
    out, ro = run_forward(path, shape_of(cfg), dl, device_input(cfg, x, xb))
    ro = to_np(ro)
    err = _check_block(cfg, layer, x, out.cpu().numpy(), ro)
    check_permutation(ro, ro["topk_idx"], cfg.E)
    print(f"edge {name} {path}: max|err|/rms = {err:.2e}")


def _degenerate_rows(H, rng):
    """Token rows whose values stress the FP8-term encoding of the expert input:
    zeros, negative zeros, one nonzero 32-value block, a constant row, rows
    scaled by 2^-60 and 2^20, and exact +-1."""
    x = np.zeros((8, H), np.float32)
    x[1] = -0.0
    x[2, 32:64] = rng.normal(0.0, 1.0, 32)
    x[3] = 0.5
    x[4] = rng.normal(0.0, 1.0, H) * 2.0 ** -60
    x[5] = rng.normal(0.0, 1.0, H) * 2.0 ** 20
    x[6] = rng.normal(0.0, 1.0, H)
    x[7] = np.where(np.arange(H) % 2 == 0, 1.0, -1.0)
    return x


@pytest.mark.parametrize("cid", [1, 4, 5])
@pytest.mark.parametrize("path", ["decode", "prefill"])
def test_degenerate_token_values(cid, path):
    from workloads.gen import _round_to_bf16_bits, bf16_bits_to_f32
    base = {1: dict(H=256, F=256), 4: dict(H=256, F=192, E=8, k=4, layers=1),
            5: dict(H=256, F=128, E=12, k=6)}[cid]
    cfg = _small(cid, T=8, **base)
    _announce(f"degenerate token values, config {cid} {path}")
    layer = make_layer(cfg)
    x = _degenerate_rows(cfg.H, np.random.default_rng(11))
    xb = None
    if cfg.act_dtype == "bf16":
        xb = _round_to_bf16_bits(x)
        x = bf16_bits_to_f32(xb)
    dl = upload(cfg, layer)
    out, ro = run_forward(path, shape_of(cfg), dl, device_input(cfg, x, xb))
    out = out.cpu().numpy()
    ro = to_np(ro)
    ref = _oracle(cfg, layer, x)
    check_routing(ro["topk_idx"], ro["topk_w"], ref, layer.router_w, layer.router_b,
                  cfg.route_scale)
    want = x + ref["delta"]
    assert np.isfinite(out).all()
    # each token against its own output's RMS (stricter than the block-wide bar)
    for t in range(cfg.T):
        err = rel_err(out[t:t + 1], want[t:t + 1])
        assert err <= TOL, f"token {t}: max|err|/rms = {err:.3e}"


@pytest.mark.parametrize("path", ["decode", "prefill"])
def test_single_token_norm_rows(path):
    # T = 1 with an RMSNorm: rms_inv_kernel computes the token's norm scale,
    # then the router launch reads it; every degenerate row on its own
    cfg = _small(4, T=1, H=256, F=192, E=8, k=4, layers=1)
    _announce(f"single-token RMSNorm rows {path}")
    layer = make_layer(cfg)
    dl = upload(cfg, layer)
    rows = _degenerate_rows(cfg.H, np.random.default_rng(12))
    for t in range(rows.shape[0]):
        x = rows[t:t + 1]
        out, ro = run_forward(path, shape_of(cfg), dl, torch.from_numpy(x).cuda())
        err = _check_block(cfg, layer, x, out.cpu().numpy(), to_np(ro))
        assert np.isfinite(out.cpu().numpy()).all(), t
        print(f"row {t}: max|err|/rms = {err:.2e}")


def test_decode_limit_is_an_error():
    cfg = _small(1, T=65)
    shape = shape_of(cfg)
    layer = make_layer(cfg)
    x, _ = make_activations(cfg, rows=cfg.T)
    dl = upload(cfg, layer)
    with pytest.raises(mx.MoeError):
        run_forward("decode", shape, dl, torch.from_numpy(x).cuda())


def test_empty_batch_is_a_noop():
    cfg = config_by_id(1)
    layer = make_layer(cfg)
    dl = upload(cfg, layer)
    shape = shape_of(cfg, 0)
    x = torch.zeros(4, dtype=torch.float32, device="cuda")
    out = torch.full((4,), 7.0, dtype=torch.float32, device="cuda")
    ws = workspace(shape)
    for fn in (mx.moe_forward_decode, mx.moe_forward_prefill):
        fn(shape, x, dl.router_w, dl.router_b, dl.experts_copy(0), out, ws)
    torch.cuda.synchronize()
    assert out.cpu().tolist() == [7.0] * 4


@pytest.mark.parametrize("path", ["decode", "prefill"])
def test_in_place_output(path):
    cfg = _small(1, T=7)
    _announce(f"in-place {path}")
    layer = make_layer(cfg)
    x, _ = make_activations(cfg, rows=cfg.T)
    dl = upload(cfg, layer)
    h = torch.from_numpy(x).cuda()
    out, ro = run_forward(path, shape_of(cfg), dl, h, out=h)
    err = _check_block(cfg, layer, x, out.cpu().numpy(), to_np(ro))
    assert err <= TOL


def test_prefill_routing_is_deterministic():
    cfg = config_by_id(3)
    layer = make_layer(scaled(cfg, F=64))
    x, _ = make_activations(cfg)
    c2 = scaled(cfg, F=64)
    dl = upload(c2, layer)
    a = to_np(run_forward("prefill", shape_of(c2), dl, torch.from_numpy(x).cuda())[1])
    b = to_np(run_forward("prefill", shape_of(c2), dl, torch.from_numpy(x).cuda())[1])
    for k in a:
        assert a[k].tobytes() == b[k].tobytes(), k


@pytest.mark.parametrize("T", [1, 8, 40])
def test_route_and_decode_select_alike(T):
    """moe_route and moe_forward_decode add the router's split-K partials in
    one order, so they select the same experts with the same weights, also at
    fp64 near-ties: each expert has a twin whose router row is a permutation
    of its own, and the tokens are constant rows, so twins' logits are equal
    in exact arithmetic and differ only by the rounding of their partial sums.
    T = 40 takes the tiled router in both."""
    _announce(f"route vs decode selections, T={T}")
    H, F, E, k = 2880, 64, 32, 4
    rng = np.random.default_rng(31 + T)
    rw = rng.normal(0.0, 0.05, size=(E, H)).astype(np.float32)
    for e in range(E // 2):
        rw[e + E // 2] = rw[e][rng.permutation(H)]
    half = rng.normal(0.0, 0.5, size=E // 2)
    rb = np.concatenate([half, half]).astype(np.float32)   # twins share their bias
    x = (rng.normal(0.0, 1.0, size=(T, 1)) * np.ones((1, H))).astype(np.float32)
    cfg = scaled(config_by_id(2), T=T, H=H, F=F, E=E, k=k)
    layer = make_layer(cfg)
    layer.router_w, layer.router_b = rw, rb
    dl = upload(cfg, layer)
    shape = shape_of(cfg)
    xd = torch.from_numpy(x).cuda()
    ro_r, ro_d = route_buffers(T, k, E), route_buffers(T, k, E)
    mx.moe_route(shape, xd, dl.router_w, dl.router_b, ro_r, workspace(shape))
    out = torch.empty_like(xd)
    mx.moe_forward_decode(shape, xd, dl.router_w, dl.router_b, dl.experts_copy(0), out,
                          workspace(shape), route_out=ro_d)
    torch.cuda.synchronize()
    assert torch.equal(ro_r["topk_idx"], ro_d["topk_idx"])
    assert torch.equal(ro_r["topk_w"], ro_d["topk_w"])
    for f in ("counts", "offsets", "perm", "inv"):
        assert torch.equal(ro_r[f], ro_d[f]), f
    ref = omoe.top_k(omoe.router_logits(x, rw, rb), k)
    # the oracle sums in another order: away from certified near-ties it agrees
    check_routing(ro_d["topk_idx"].cpu().numpy(), ro_d["topk_w"].cpu().numpy(),
                  dict(logits=omoe.router_logits(x, rw, rb), idx=ref,
                       w=omoe.route_weights(omoe.router_logits(x, rw, rb), ref, 1.0), xn=x),
                  rw, rb, 1.0, max_flips=T)


@pytest.mark.parametrize("cid,T", [(2, 1), (5, 8)])
def test_decode_is_deterministic(cid, T):
    """Every route of a token is added by one workgroup in a fixed order: two
    runs give the same bits."""
    cfg = config_by_id(cid)
    if cid == 5:
        cfg = scaled(cfg, E=32)
    _announce(f"decode determinism config {cid} T={T}")
    layer = make_layer(cfg)
    x, xb = make_activations(cfg, rows=T)
    dl = upload(cfg, layer)
    shape = shape_of(cfg, T)
    xd = device_input(cfg, x, xb)
    a, _ = run_forward("decode", shape, dl, xd)
    b, _ = run_forward("decode", shape, dl, xd)
    assert torch.equal(a, b)
