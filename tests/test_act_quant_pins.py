"""Pins of the oracle's MX-FP4 activation round trip (oracle/act_quant.py) and
of the quantised expert-input mode of the block, against what the page's rule
and the mathematics fix: nearest E2M1 value with ties to the even code found
by enumerating all sixteen codes, the page's own float32 scale formula where it
has no rounding edge, the minimal scale, idempotence on grid values, the error
bound, and the block's behaviour on inputs the round trip leaves unchanged.
Page: antirez `ds4.c`, `dsv4_fp4_act_quantize_row_inplace_cpu`,
`dsv4_e2m1fn_dequant_cpu`."""
from __future__ import annotations

import math

import numpy as np
import pytest

from oracle import act_quant as aq
from oracle import moe as omoe
from oracle import mxfp4
from workloads import config_by_id, make_layer, scaled
from workloads.gen import make_activations


def _brute_code(v: float, e: int) -> int:
    """The code whose value (E2M1 closed form times 2^e) is nearest to v, over
    all sixteen codes with v's sign; equal distances go to the code with a zero
    mantissa bit (the even index)."""
    neg = v < 0
    best, best_d = None, None
    for c in range(16):
        if bool(c & 8) != neg:
            continue
        val = mxfp4.e2m1_value(c) * 2.0 ** e
        d = abs(v - val)
        if best is None or d < best_d or (d == best_d and (c & 1) == 0 and (best & 1) == 1):
            best, best_d = c, d
    return best


def test_ties_go_to_the_even_code():
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    want = [0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]   # the lower or upper neighbour with the even index
    row = np.zeros(32, np.float32)
    row[:7] = mids
    row[7] = 6.0                                # block maximum: scale 1
    row[8:15] = [-m for m in mids]
    c, s, v = aq.quantize_rows(row[None])
    assert s[0, 0] == 127
    assert np.array_equal(v[0, :7], want) and np.array_equal(v[0, 8:15], [-w for w in want])
    assert all(int(x) & 1 == 0 for x in c[0, :7])


@pytest.mark.parametrize("seed", range(4))
def test_nearest_code_matches_enumeration(seed):
    rng = np.random.default_rng(seed)
    x = (rng.normal(size=(6, 64)) * 2.0 ** rng.integers(-20, 20, size=(6, 1))).astype(np.float32)
    # plant exact midpoints of the grid in a few blocks
    x[0, :8] = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], np.float32)
    codes, scales, vals = aq.quantize_rows(x)
    for r in range(x.shape[0]):
        for b in range(x.shape[1] // 32):
            e = int(scales[r, b]) - 127
            for i in range(32):
                xv = float(x[r, 32 * b + i])
                c = _brute_code(xv, e)
                # the page clamps to +-6 first: beyond that the largest code is nearest anyway
                assert codes[r, 32 * b + i] == c, (r, b, i, xv, e)
                assert vals[r, 32 * b + i] == mxfp4.e2m1_value(c) * 2.0 ** e


def test_scale_is_the_smallest_that_fits():
    rng = np.random.default_rng(7)
    mags = 2.0 ** rng.uniform(-140, 100, size=4000)
    x = (mags * rng.choice([-1, 1], size=mags.size)).astype(np.float32).reshape(-1, 32)
    _, scales, _ = aq.quantize_rows(x)
    amax = np.maximum(np.abs(x).max(axis=1).astype(np.float64), aq.AMAX_FLOOR)
    e = scales[:, 0].astype(np.int64) - 127
    assert np.all(amax <= 6.0 * np.ldexp(1.0, e))
    assert np.all((e == -126) | (amax > 3.0 * np.ldexp(1.0, e)))


def test_exponent_equals_the_pages_float32_formula_off_its_rounding_edge():
    """2^ceil(log2f(amax/6)) computed in float32 as the page does, against the
    exact exponent: equal wherever log2(amax/6) is not within float32 rounding
    of an integer from above."""
    rng = np.random.default_rng(3)
    amax = (2.0 ** rng.uniform(-100, 100, size=20000)).astype(np.float32)
    q = (amax / np.float32(6.0)).astype(np.float32)
    lg = np.log2(q.astype(np.float32))
    page = np.ceil(lg).astype(np.int64)
    exact = aq.block_exponent(amax)
    lg64 = np.log2(amax.astype(np.float64) / 6.0)
    edge = np.abs(lg64 - np.round(lg64)) < 1e-5
    assert np.array_equal(page[~edge], exact[~edge])
    assert (~edge).sum() > 19000


def test_grid_values_are_fixed_points_and_error_is_bounded():
    rng = np.random.default_rng(11)
    codes = rng.integers(0, 16, size=(8, 128)).astype(np.uint8)
    e = rng.integers(-20, 20, size=(8, 4))
    grid = (mxfp4.E2M1[codes].reshape(8, 4, 32) * np.ldexp(1.0, e)[..., None]).reshape(8, 128)
    _, _, v = aq.quantize_rows(grid.astype(np.float32))
    assert np.array_equal(v, grid)
    x = rng.normal(size=(16, 256)).astype(np.float32)
    _, s, v = aq.quantize_rows(x)
    scale = np.repeat(np.ldexp(1.0, s.astype(np.int64) - 127), 32, axis=1)
    r = np.abs(x.astype(np.float64)) / scale
    bound = scale * np.maximum(0.25, r / 4.0)
    assert np.all(np.abs(v - x) <= bound)


def test_zero_blocks_and_signed_zero():
    x = np.zeros((1, 64), np.float32)
    x[0, 32:] = -0.0
    c, s, v = aq.quantize_rows(x)
    assert np.all(c == 0) and np.all(s == 1) and np.all(v == 0.0)  # scale 2^-126
    tiny = np.zeros((1, 32), np.float32)
    tiny[0, 0], tiny[0, 1] = 8.0, -1e-3     # small next to the block maximum: rounds to -0
    c, _, v = aq.quantize_rows(tiny)
    assert c[0, 1] == 8 and v[0, 1] == 0.0 and math.copysign(1, v[0, 1]) < 0


def test_pack_codes_low_nibble_first():
    c = np.array([[1, 2, 15, 8]], np.uint8)
    assert aq.pack_codes(c).tolist() == [[0x21, 0x8F]]


def _grid_input(cfg, rng):
    T, H = cfg.T, cfg.H
    codes = rng.integers(0, 16, size=(T, H)).astype(np.uint8)
    codes[:, ::32] = 7                        # every block holds +6 x 2^e: its maximum
    e = rng.integers(-3, 1, size=(T, H // 32))
    x = (mxfp4.E2M1[codes].reshape(T, H // 32, 32) * np.ldexp(1.0, e)[..., None]).reshape(T, H)
    return x.astype(np.float32)


def test_block_mode_is_identity_on_grid_inputs_and_keeps_routing():
    cfg = scaled(config_by_id(1), T=6)
    layer = make_layer(cfg)
    x = _grid_input(cfg, np.random.default_rng(5))
    a = omoe.block_for_config(cfg, layer, x)
    b = omoe.block_for_config(cfg, layer, x, act_quant=1)
    assert np.array_equal(a["idx"], b["idx"])
    assert np.array_equal(a["out"], b["out"]) and np.array_equal(a["delta"], b["delta"])


def test_block_mode_changes_general_inputs_but_not_routing():
    cfg = config_by_id(1)
    layer = make_layer(cfg)
    x, _ = make_activations(cfg)
    a = omoe.block_for_config(cfg, layer, x)
    b = omoe.block_for_config(cfg, layer, x, act_quant=1)
    assert np.array_equal(a["idx"], b["idx"]) and np.array_equal(a["w"], b["w"])
    rms = np.sqrt(np.mean(a["delta"] ** 2))
    diff = np.abs(a["delta"] - b["delta"]).max() / rms
    assert 1e-3 < diff < 1.0
    # the experts' input is exactly the round trip of the float32 input
    assert np.array_equal(b["xe"], aq.quantize_rows(x.astype(np.float32))[2])


def test_mode2_single_expert_composition():
    """act_quant 2 on one expert (E = k = 1, so the route weight is the route
    scale): the block equals the composition written out with the page-table
    decoding of the weights (`oracle.brute`), the pure-Python clamped SwiGLU,
    and the round trip applied to the expert input and to the SwiGLU output."""
    from oracle import brute
    cfg = scaled(config_by_id(1), T=5, H=64, F=96, E=1, k=1, route_scale=1.5)
    layer = make_layer(cfg)
    x, _ = make_activations(cfg)
    ex = layer.experts
    wg = np.array(brute.decode_matrix(ex.gate_codes[0], ex.gate_scales[0], cfg.F, cfg.H))
    wu = np.array(brute.decode_matrix(ex.up_codes[0], ex.up_scales[0], cfg.F, cfg.H))
    wd = np.array(brute.decode_matrix(ex.down_codes[0], ex.down_scales[0], cfg.H, cfg.F))
    xe = aq.quantize_rows(x)[2]
    g = xe @ wg.T + ex.gate_bias[0]
    u = xe @ wu.T + ex.up_bias[0]
    h = np.vectorize(lambda a, b: brute.swiglu_scalar(a, b, cfg.alpha, cfg.limit, cfg.up_offset))(g, u)
    hq = aq.quantize_rows(h.astype(np.float32))[2]
    want = cfg.route_scale * (hq @ wd.T + ex.down_bias[0])
    got = omoe.block_for_config(cfg, layer, x, act_quant=2)
    assert np.allclose(got["delta"], want, rtol=1e-12, atol=1e-12 * np.abs(want).max())
    # and it differs from mode 1, whose down input is the unrounded SwiGLU output
    one = omoe.block_for_config(cfg, layer, x, act_quant=1)
    assert not np.allclose(one["delta"], got["delta"], rtol=1e-6, atol=0)


def test_mode2_collects_the_unrounded_swiglu_output():
    cfg = scaled(config_by_id(1), T=4)
    layer = make_layer(cfg)
    x, _ = make_activations(cfg)
    stats = {}
    omoe.block_for_config(cfg, layer, x, stats=stats, act_quant=2)
    acts = stats["act"]
    assert len(acts) == len(np.unique(omoe.block_for_config(cfg, layer, x)["idx"]))
    assert all(r["a"].shape == (len(r["tokens"]), cfg.F) for r in acts)
