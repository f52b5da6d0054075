"""The quantised modes (act_quant = 1: MX-FP4 expert input; 2: and MX-FP4
SwiGLU output) on the GPU against the oracle.

Bars:
- the MX-FP4 expert input (codes and scale bytes, moe_act_quant_debug) is
  bit-exact against `oracle.act_quant.quantize_rows` of the oracle's float32
  expert input. Without a norm both sides round the same float32 values. With
  a norm the float32 value comes from two fp64 evaluations whose summation
  orders differ; a code may then differ only in a block holding an element
  whose fp64 value sits within fp64 noise of a float32 rounding midpoint
  (counted; expected none);
- block outputs within the exact mode's bound, max |err| <= 2e-3 x RMS of the
  oracle output (`oracle.moe.block_for_config(..., act_quant=1)`): with the
  codes bit-exact, each gate/up product of two E2M1 values times two
  power-of-two scales is exact in the float32 accumulator, so the mode adds
  only float32 accumulation error to the exact mode's FP8-term error of the
  SwiGLU output;
- the mode changes the output by more than that bound against the exact
  block, so the test would see a path that ignored the mode;
- mode 2: the same bound plus an allowance, computed from the oracle alone,
  for SwiGLU values at an MX-FP4 rounding edge (see kEdge below).
Page: antirez ds4.c `dsv4_fp4_act_quantize_row_inplace_cpu`,
`dsv4_e2m1fn_dequant_cpu`; goosedump `mixture_of_experts` (`Q8Activation`:
the expert input quantised once for every expert row).
"""
import numpy as np
import pytest
import torch

import mxfp4_expert_ffn_amd as mx
from mxfp4_expert_ffn_amd.device import workspace
from oracle import act_quant as aq
from oracle import moe as omoe
from oracle import mxfp4 as omx
from workloads import config_by_id, make_layer, scaled
from workloads.gen import make_activations

from gpu_util import (TOL, check_permutation, check_routing, device_input, rel_err, run_forward,
                      shape_of, to_np, upload)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mx._lib.load()


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)


def _unpack(packed: np.ndarray) -> np.ndarray:
    p = packed.astype(np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def _gpu_codes(shape, x_dev, norm_w=None):
    T, H = shape.T, shape.H
    codes = torch.full((T, H // 2), 0xEE, dtype=torch.uint8, device="cuda")
    scales = torch.full((T, H // 32), 0xEE, dtype=torch.uint8, device="cuda")
    ws = workspace(shape)
    mx.moe_act_quant_debug(shape, x_dev, codes, scales, ws, norm_w=norm_w)
    torch.cuda.synchronize()
    return _unpack(codes.cpu().numpy()), scales.cpu().numpy()


def _midpoint_blocks(v64: np.ndarray) -> np.ndarray:
    """Blocks [T, H/32] holding an element whose fp64 value is within 2^-40
    (relative) of a float32 rounding midpoint: there two fp64 evaluations of
    the same expression may round to different float32 values."""
    f32 = v64.astype(np.float32)
    ulp = np.spacing(np.abs(f32)).astype(np.float64)
    gap = np.abs(0.5 * ulp - np.abs(v64 - f32.astype(np.float64)))
    near = gap <= np.abs(v64) * 2.0 ** -40
    return near.reshape(v64.shape[0], -1, 32).any(axis=-1)


def _check_codes(got_c, got_s, x32, v64=None):
    want_c, want_s, _ = aq.quantize_rows(x32)
    bad = (got_s != want_s) | (got_c != want_c).reshape(got_s.shape + (32,)).any(axis=-1)
    if v64 is None:
        assert not bad.any(), f"{int(bad.sum())} blocks differ, first at {np.argwhere(bad)[:4].tolist()}"
    else:
        edge = _midpoint_blocks(v64)
        assert not (bad & ~edge).any(), f"blocks off a rounding edge differ: {np.argwhere(bad & ~edge)[:4].tolist()}"
        print(f"{int(bad.sum())} blocks differ at float32 rounding edges ({int(edge.sum())} such blocks)")
    return want_c, want_s


def _edge_rows(H: int, rng) -> np.ndarray:
    """Rows that reach every branch of the round trip: planted ties at each
    E2M1 midpoint, exact grid values, wide exponent spread, all-zero and
    signed-zero blocks, blocks below the amax floor (subnormal and tiny
    normal values), the largest float32 magnitudes, amax exactly 1.5 * 2^E
    and one ulp above."""
    nb = H // 32
    rows = []
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], np.float32)
    r = (rng.normal(size=H) * 2.0 ** rng.integers(-30, 30, size=H)).astype(np.float32)
    for b in range(0, nb, 3):
        e = int(rng.integers(-20, 20))
        r[32 * b:32 * b + 8] = mids * np.float32(2.0 ** e)
        r[32 * b + 8:32 * b + 16] = -mids * np.float32(2.0 ** e)
        r[32 * b + 16:32 * b + 32] = 0.0
    rows.append(r)
    z = np.zeros(H, np.float32)
    z[32:64] = -0.0
    z[64:96] = np.float32(1e-39) * rng.choice([-1, 1], size=32)       # subnormal
    z[96:128] = np.float32(3e-38) * rng.normal(size=32)               # below 6 * 2^-126
    if nb > 4:
        z[128:160] = np.float32(3.0e38) * rng.choice([-1, 1], size=32)  # near the float32 top
    rows.append(z)
    a = rng.normal(size=H).astype(np.float32)
    for b in range(nb):
        a[32 * b] = np.float32(1.5 * 2.0 ** (b % 9 - 4))              # amax = 1.5 * 2^E
        if b % 2:
            a[32 * b] = np.nextafter(a[32 * b], np.float32(np.inf))   # one ulp above
        a[32 * b + 1:32 * b + 32] = np.clip(a[32 * b + 1:32 * b + 32], -1.4, 1.4) * 2.0 ** (b % 9 - 4)
    rows.append(a)
    return np.stack(rows).astype(np.float32)


@pytest.mark.parametrize("H", [256, 2880])
def test_codes_bitexact_edge_rows(H):
    _announce(f"act_quant codes: edge rows H={H}")
    x = _edge_rows(H, np.random.default_rng(H))
    shape = mx.make_shape(T=x.shape[0], H=H, F=256, E=8, k=2)
    got_c, got_s = _gpu_codes(shape, torch.from_numpy(x).cuda())
    _check_codes(got_c, got_s, x)


@pytest.mark.parametrize("cid,T", [(3, 128), (5, 256), (6, 64)])
def test_codes_bitexact_workload_inputs(cid, T):
    cfg = scaled(config_by_id(cid), T=T)
    _announce(f"act_quant codes: config {cid} T={T} ({cfg.act_dtype})")
    x, xb = make_activations(cfg)
    got_c, got_s = _gpu_codes(shape_of(cfg), device_input(cfg, x, xb))
    _check_codes(got_c, got_s, x)


def test_codes_with_norm():
    cfg = scaled(config_by_id(4), T=96)
    _announce("act_quant codes: config 4 with RMSNorm, T=96")
    layer = make_layer(cfg)
    x, _ = make_activations(cfg)
    xn = omoe.rms_norm(x, layer.norm_w, cfg.rms_eps)
    dl = upload(cfg, layer)
    got_c, got_s = _gpu_codes(shape_of(cfg), torch.from_numpy(x).cuda(), norm_w=dl.norm_w)
    _check_codes(got_c, got_s, xn.astype(np.float32), v64=xn)


def _aq_shape(cfg, T=None):
    kw = cfg.shape_kwargs(T)
    kw["act_quant"] = 1
    return mx.make_shape(**kw)


@pytest.mark.parametrize("cid,T,tile", [(1, 8, 16), (3, 128, 16), (4, 512, 32), (5, 1024, 32),
                                        (5, 2048, 64)])
def test_prefill_block(cid, T, tile):
    """Whole block in the mode, against the oracle in the same mode; sampled
    tokens at the DeepSeek-V4-Flash shape. Covers 16-, 32- and 64-row tiles."""
    cfg = scaled(config_by_id(cid), T=T)
    _announce(f"act_quant prefill: config {cid} T={T}")
    layer = make_layer(cfg)
    x, xb = make_activations(cfg)
    shape = _aq_shape(cfg)
    plan = mx.moe_prefill_plan(shape, with_norm=layer.norm_w is not None)
    assert plan["tile_rows"] == tile and plan["x_terms"] == 0
    dl = upload(cfg, layer)
    out, ro = run_forward("prefill", shape, dl, device_input(cfg, x, xb))
    ro = to_np(ro)
    out = out.cpu().numpy()
    toks = None if T <= 512 else np.random.default_rng(T).choice(T, 48, replace=False)
    ref = omoe.block_for_config(cfg, layer, x, tokens=toks, act_quant=1)
    check_routing(ro["topk_idx"], ro["topk_w"], ref, layer.router_w, layer.router_b,
                  cfg.route_scale)
    check_permutation(ro, ro["topk_idx"], cfg.E)
    tk = ref["tokens"]
    err = rel_err(out[tk], x[tk] + ref["delta"])
    exact = omoe.block_for_config(cfg, layer, x, tokens=toks)
    moved = rel_err(x[tk] + exact["delta"], x[tk] + ref["delta"])
    print(f"config {cid} T={T} act_quant: max|err|/rms = {err:.2e}; mode moves the output {moved:.2e}")
    assert err <= TOL, f"max|err|/rms = {err:.3e}"
    assert moved > 5 * TOL


def test_prefill_block_matches_exact_mode_on_grid_inputs():
    """Inputs already on the MX-FP4 grid: the round trip leaves them as they
    are, so both modes compute the same block (to the exact mode's bound)."""
    cfg = scaled(config_by_id(3), T=64)
    _announce("act_quant prefill: grid inputs, both modes")
    layer = make_layer(cfg)
    rng = np.random.default_rng(9)
    codes = rng.integers(0, 16, size=(cfg.T, cfg.H)).astype(np.uint8)
    codes[:, ::32] = 7
    e = rng.integers(-3, 1, size=(cfg.T, cfg.H // 32))
    x = (omx.E2M1[codes].reshape(cfg.T, -1, 32) * np.ldexp(1.0, e)[..., None]).reshape(cfg.T, cfg.H)
    x = x.astype(np.float32)
    dl = upload(cfg, layer)
    xd = torch.from_numpy(x).cuda()
    out_q, _ = run_forward("prefill", _aq_shape(cfg), dl, xd)
    out_e, _ = run_forward("prefill", shape_of(cfg), dl, xd)
    ref = omoe.block_for_config(cfg, layer, x)
    assert rel_err(out_q.cpu().numpy(), x + ref["delta"]) <= TOL
    assert rel_err(out_e.cpu().numpy(), x + ref["delta"]) <= TOL


def test_decode_rejects_the_mode():
    cfg = config_by_id(1)
    layer = make_layer(cfg)
    x, _ = make_activations(cfg)
    dl = upload(cfg, layer)
    shape = _aq_shape(cfg)
    out = torch.zeros((cfg.T, cfg.H), dtype=torch.float32, device="cuda")
    with pytest.raises(mx.MoeError) as ei:
        mx.moe_forward_decode(shape, torch.from_numpy(x).cuda(), dl.router_w, dl.router_b,
                              dl.experts_copy(0), out, workspace(shape))
    assert ei.value.code == mx._lib.MOE_ERR_UNSUPPORTED


# ---------------------------------------------------------------- mode 2
# The SwiGLU output is rounded to MX-FP4 on each side from its own float32
# value: the oracle's from fp64 arithmetic, the GPU's from float32 matrix-core
# accumulation of exact FP4 x FP4 products. Where a value lies within
# kEdge x 2^e of an E2M1 decision boundary of its block (scale 2^e), or its
# block maximum within kEdge x 2^e of the point where the scale changes, the
# two sides may take neighbouring codes. The bar for a token is then the exact
# mode's 2e-3 x RMS plus, per such value f of slot j, the route weight times
# the code step at that boundary times |W_down[:, f]| (every code of the block
# when its scale is in doubt). kEdge = 2^-13 of the scale, 2e-5 of the block
# maximum, against float32 accumulation errors near 1e-6 of it. A value whose
# gate and up were both clamped holds no accumulated product: both sides
# evaluate limit * sigmoid(alpha * limit) * (+-limit + offset) from the same
# constants, within a few float32 ulps, so its edge is kEdgeClamped = 2^-18 of
# the scale (gpt-oss's clamped outputs, 55.99963 on a scale of 16, sit 2.3e-5
# of the scale below the 3.5 boundary).
kEdge = 2.0 ** -13
kEdgeClamped = 2.0 ** -18
_BOUNDS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
_STEPS = np.array([0.5, 0.5, 0.5, 0.5, 1.0, 1.0, 2.0])


def _edge_steps(a64: np.ndarray, clamped: np.ndarray) -> np.ndarray:
    """Per value of `a` [rows, F]: the code step it may take at a rounding edge
    (in units of its value), 0 where it is clear of every edge."""
    rows, F = a64.shape
    width = np.where(clamped, kEdgeClamped, kEdge).reshape(rows, F // 32, 32)
    blk = a64.reshape(rows, F // 32, 32)
    amax = np.maximum(np.abs(blk).max(axis=-1).astype(np.float32), np.float32(aq.AMAX_FLOOR))
    sc = np.ldexp(1.0, aq.block_exponent(amax))              # [rows, nb]
    r = np.abs(blk) / sc[..., None]
    near = np.abs(r[..., None] - _BOUNDS) <= width[..., None]  # [rows, nb, 32, 7]
    step = np.where(near, _STEPS, 0.0).max(axis=-1) * sc[..., None]
    # a block maximum at the scale's edge (1.5 x 2^E) may move every code
    m = amax.astype(np.float64)
    E = np.floor(np.log2(m)).astype(np.int64)
    doubt = np.abs(m - 1.5 * np.ldexp(1.0, E)) <= kEdge * sc
    step = np.where(doubt[..., None], 4.0 * sc[..., None], step)
    return step.reshape(rows, F)


def _edge_allowance(cfg, layer, ref, stats, toks) -> np.ndarray:
    """[len(toks), H]: the output movement rounding-edge codes may cause."""
    pos = {int(t): i for i, t in enumerate(toks)}
    allow = np.zeros((len(toks), cfg.H))
    for rec in stats["act"]:
        planes = layer.shared if rec["shared"] else layer.experts
        wd = np.abs(omx.dequant(planes.down_codes[rec["e"]], planes.down_scales[rec["e"]]))
        st = _edge_steps(rec["a"], rec["clamped"])
        for i, t in enumerate(rec["tokens"]):
            if int(t) not in pos or not st[i].any():
                continue
            w = 1.0 if rec["shared"] else float(ref["w"][int(t), rec["slots"][i]])
            allow[pos[int(t)]] += w * (wd @ st[i])
    return allow


@pytest.mark.parametrize("cid,T,tile", [(1, 8, 16), (3, 128, 16), (5, 1024, 32), (5, 2048, 64)])
def test_prefill_block_mode2(cid, T, tile):
    """SwiGLU output quantised too: FP4 x FP4 down products."""
    cfg = scaled(config_by_id(cid), T=T)
    _announce(f"act_quant 2 prefill: config {cid} T={T}")
    layer = make_layer(cfg)
    x, xb = make_activations(cfg)
    kw = cfg.shape_kwargs()
    kw["act_quant"] = 2
    shape = mx.make_shape(**kw)
    plan = mx.moe_prefill_plan(shape, with_norm=layer.norm_w is not None)
    assert plan["tile_rows"] == tile and plan["x_terms"] == 0 and plan["act_terms"] == 0
    dl = upload(cfg, layer)
    out, ro = run_forward("prefill", shape, dl, device_input(cfg, x, xb))
    ro = to_np(ro)
    out = out.cpu().numpy()
    toks = np.arange(T) if T <= 128 else np.random.default_rng(T + 2).choice(T, 12, replace=False)
    stats = {}
    ref = omoe.block_for_config(cfg, layer, x, tokens=toks, stats=stats, act_quant=2)
    check_routing(ro["topk_idx"], ro["topk_w"], ref, layer.router_w, layer.router_b,
                  cfg.route_scale)
    want = x[toks] + ref["delta"]
    rms = np.sqrt(np.mean(want.astype(np.float64) ** 2))
    allow = _edge_allowance(cfg, layer, ref, stats, toks)
    err = np.abs(out[toks].astype(np.float64) - want)
    bar = TOL * rms + allow
    clear = ~allow.any(axis=1)
    print(f"config {cid} T={T} mode 2: max|err|/rms = {err.max() / rms:.2e}; tokens clear of "
          f"rounding edges {int(clear.sum())}/{len(toks)}, their max|err|/rms = "
          f"{(err[clear].max() / rms) if clear.any() else float('nan'):.2e}")
    assert np.all(err <= bar), f"worst excess {float((err - bar).max()) / rms:.3e} x RMS"
    # against the mode that keeps the SwiGLU output exact, the difference is real
    one = omoe.block_for_config(cfg, layer, x, tokens=toks, act_quant=1)
    assert rel_err(x[toks] + one["delta"], want) > 5 * TOL
