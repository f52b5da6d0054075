"""Pins of the CPU oracle against what the pages and mathematics fix.

Each test is chosen so that a plausible slip in the oracle (a wrong sign or
nibble, a dropped bias, softmax before top-k, a transposed operand, a wrong
tie rule) fails at least one of them. None of these tests needs a GPU.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import brute, moe, mxfp4
from workloads import config_by_id, make_layer, scaled
from workloads.gen import ExpertPlanes, Layer, make_activations

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def page_e2m1_table():
    with open(os.path.join(GOLDEN, "e2m1_magnitudes.txt")) as f:
        rows = [ln for ln in f if ln.strip() and not ln.startswith("#")]
    return [float(v) for v in rows[0].split()]


# ---------------------------------------------------------------- MXFP4 decode
def test_e2m1_closed_form_equals_page_table_bitwise():
    table = page_e2m1_table()
    assert len(table) == 8
    for code in range(16):
        page = table[code & 7]
        expect = np.float64(-page if code & 8 else page)
        got = mxfp4.E2M1[code]
        assert got.tobytes() == expect.tobytes(), code
    assert np.signbit(mxfp4.E2M1[8]) and mxfp4.E2M1[8] == 0.0
    assert not np.signbit(mxfp4.E2M1[0])


def test_nibble_order_fixture():
    # documented layout: element 2i in the low nibble of byte i
    packed = np.array([[0x21, 0xF8]], dtype=np.uint8)
    assert mxfp4.unpack_codes(packed).tolist() == [[1, 2, 8, 15]]


def _page_fp4_quantize_block(x32):
    """The page's MX-style FP4 round trip of one 32-element block, restated.

    antirez ds4.c, dsv4_fp4_act_quantize_row_inplace_cpu and
    dsv4_e2m1fn_dequant_cpu: amax of the block (floored at 7.05e-38),
    scale = 2^ceil(log2(amax/6)), v = x/scale clamped to +-6, nearest E2M1
    magnitude with ties to the even code, value = sign * magnitude * scale.
    Returns the fake-quantised float32 values, 4-bit codes and the exponent.
    """
    table = np.array(page_e2m1_table(), dtype=np.float32)
    amax = np.float32(max(np.max(np.abs(x32)), np.float32(7.052966104933725e-38)))
    exp = int(math.ceil(math.log2(float(amax) / 6.0)))
    scale = np.float32(math.ldexp(1.0, exp))
    vals, codes = [], []
    for xi in x32:
        v = np.float32(xi / scale)
        v = min(max(v, np.float32(-6.0)), np.float32(6.0))
        sign = np.float32(-1.0) if v < 0 else np.float32(1.0)
        ax = abs(v)
        best, best_diff = 0, abs(ax - table[0])
        for i in range(1, 8):
            d = abs(ax - table[i])
            if d < best_diff or (d == best_diff and i % 2 == 0 and best % 2 == 1):
                best, best_diff = i, d
        vals.append(np.float32(sign * table[best]) * scale)
        codes.append(best | (8 if v < 0 else 0))
    return np.array(vals, dtype=np.float32), codes, exp


def test_dequant_reproduces_page_mx_round_trip():
    rng = np.random.default_rng(7)
    rows, K = 6, 96
    x = (rng.normal(size=(rows, K)) * np.exp(rng.normal(size=(rows, 1)) * 3)).astype(np.float32)
    x[0, :32] = 0.0                              # all-zero block: smallest scale
    x[1, 5] = -0.0
    fake = np.empty_like(x)
    packed = np.zeros((rows, K // 2), dtype=np.uint8)
    scales = np.zeros((rows, K // 32), dtype=np.uint8)
    for r in range(rows):
        for b in range(K // 32):
            vals, codes, exp = _page_fp4_quantize_block(x[r, 32 * b:32 * b + 32])
            fake[r, 32 * b:32 * b + 32] = vals
            scales[r, b] = exp + 127
            for i, c in enumerate(codes):
                j = 32 * b + i
                packed[r, j // 2] |= (c << 4) if j % 2 else c
    got = mxfp4.dequant(packed, scales).astype(np.float32)
    assert got.tobytes() == fake.tobytes()


def test_e8m0_is_power_of_two_and_nan_at_255():
    for b in range(255):
        v = mxfp4.E8M0[b]
        m, e = math.frexp(v)
        assert m == 0.5 and e - 1 == b - 127
    assert math.isnan(mxfp4.E8M0[255])


# ---------------------------------------------------------------- top-k
def _page_insertion_top_k(logits, k):
    """goosedump top_experts restated: a value enters at the first slot it
    strictly exceeds, shifting the rest right."""
    vals = [-math.inf] * k
    idx = [0] * k
    for i, v in enumerate(logits):
        pos = next((p for p in range(k) if v > vals[p]), k)
        if pos < k:
            vals[pos + 1:] = vals[pos:-1]
            idx[pos + 1:] = idx[pos:-1]
            vals[pos], idx[pos] = v, i
    return idx


def test_top_k_matches_brute_force_and_page_rule_with_ties():
    rng = np.random.default_rng(11)
    choices = np.array([-2.0, -1.0, -0.0, 0.0, 0.5, 1.0, 2.0])
    n = 0
    for E in range(1, 9):
        for k in range(1, min(E, 4) + 1):
            logits = choices[rng.integers(0, len(choices), size=(60, E))]
            got = moe.top_k(logits, k)
            for t in range(logits.shape[0]):
                row = logits[t].tolist()
                assert got[t].tolist() == brute.top_k_bruteforce(row, k)
                assert got[t].tolist() == _page_insertion_top_k(row, k)
                n += 1
    # continuous values as well
    logits = rng.normal(size=(300, 8))
    got = moe.top_k(logits, 3)
    for t in range(300):
        assert got[t].tolist() == brute.top_k_bruteforce(logits[t].tolist(), 3)
    assert n > 1000


def test_top_k_equal_logits_pick_lowest_indices():
    assert moe.top_k(np.zeros((1, 8)), 3).tolist() == [[0, 1, 2]]
    # -0.0 and +0.0 tie: the lower index wins
    assert moe.top_k(np.array([[0.0, -0.0, -1.0]]), 1).tolist() == [[0]]
    assert moe.top_k(np.array([[-0.0, 0.0, -1.0]]), 1).tolist() == [[0]]


# ---------------------------------------------------------------- route weights
def test_route_weights_sum_to_scale_and_descend():
    rng = np.random.default_rng(3)
    for scale in (1.0, 1.5):
        logits = rng.normal(size=(200, 32)) * 3
        idx = moe.top_k(logits, 4)
        w = moe.route_weights(logits, idx, scale)
        assert np.all(np.abs(w.sum(axis=1) - scale) <= 4 * 2.0 ** -50 * scale)
        assert np.all(np.diff(w, axis=1) <= 0)


def test_route_weights_special_cases():
    logits = np.array([[0.3, -1.0, 2.0]])
    idx = moe.top_k(logits, 1)
    assert moe.route_weights(logits, idx, 1.5).tolist() == [[1.5]]
    eq = np.full((1, 5), 0.7)
    w = moe.route_weights(eq, moe.top_k(eq, 4), 1.0)
    assert np.allclose(w, 0.25, rtol=0, atol=1e-16)
    # two selected logits a, b: weights are the logistic of the difference
    two = np.array([[1.25, -0.5, 0.0]])
    w = moe.route_weights(two, moe.top_k(two, 2), 1.0)
    assert abs(w[0, 0] - 1.0 / (1.0 + math.exp(-(1.25 - 0.0)))) < 1e-15


# ---------------------------------------------------------------- SwiGLU
def test_swiglu_reduces_to_textbook_silu_glu_when_unclamped():
    g = np.array([-3.0, -0.5, 0.0, 1.0, 2.0])
    u = np.array([0.5, 2.0, 7.0, 1.0, -1.0])
    a = moe.swiglu(g, u, alpha=1.0, limit=1e30, up_offset=0.0)
    silu = np.array([-3.0 / (1 + math.e ** 3), -0.5 / (1 + math.e ** 0.5), 0.0,
                     0.7310585786300049, 1.7615941559557649])
    assert np.allclose(a, silu * u, rtol=1e-15, atol=0)


def test_swiglu_clamp_points():
    L, al = 7.0, 1.702
    # gate above the limit behaves exactly as the limit
    assert moe.swiglu(np.array([50.0]), np.array([0.5]), al, L, 1.0)[0] == \
        moe.swiglu(np.array([L]), np.array([0.5]), al, L, 1.0)[0]
    # up is clamped on both sides
    hi = moe.swiglu(np.array([1.0]), np.array([100.0]), al, L, 1.0)[0]
    lo = moe.swiglu(np.array([1.0]), np.array([-100.0]), al, L, 1.0)[0]
    s1 = 1.0 / (1.0 + math.exp(-al))
    assert abs(hi - s1 * 8.0) < 1e-15 and abs(lo - s1 * -6.0) < 1e-15
    # gate is not clamped below: large negative gate gives ~0
    assert abs(moe.swiglu(np.array([-50.0]), np.array([3.0]), al, L, 1.0)[0]) < 1e-30


# ---------------------------------------------------------------- helpers
def _tiny_layer(rng, H, F, E, n_shared=0, norm=False, zero_down=False):
    def planes(n):
        def codes(rows, K):
            return rng.integers(0, 256, size=(n, rows, K // 2), dtype=np.uint8)

        def sc(rows, K):
            return rng.integers(123, 128, size=(n, rows, K // 32), dtype=np.uint8)

        def b(rows):
            return rng.normal(0, 0.02, size=(n, rows)).astype(np.float32)
        dc = codes(H, F) * 0 if zero_down else codes(H, F)
        return ExpertPlanes(codes(F, H), sc(F, H), b(F), codes(F, H), sc(F, H), b(F),
                            dc, sc(H, F), b(H))
    rw = rng.normal(0, 0.3, size=(E, H)).astype(np.float32)
    rb = rng.normal(0, 0.3, size=E).astype(np.float32)
    nw = (1 + rng.normal(0, 0.1, size=H)).astype(np.float32) if norm else None
    return Layer(rw, rb, planes(E), planes(n_shared) if n_shared else None, nw)


# ---------------------------------------------------------------- whole block
@pytest.mark.parametrize("variant", ["gptoss", "ds4", "norm"])
def test_numpy_oracle_equals_pure_python_brute_force(variant):
    rng = np.random.default_rng({"gptoss": 1, "ds4": 2, "norm": 3}[variant])
    H, F, E, T = 64, 64, 6, 4
    if variant == "gptoss":
        layer, k, c = _tiny_layer(rng, H, F, E), 2, (1.702, 7.0, 1.0, 1.0, None)
    elif variant == "ds4":
        layer, k, c = _tiny_layer(rng, H, F, E, n_shared=1), 3, (1.0, 10.0, 0.0, 1.5, None)
    else:
        layer, k, c = _tiny_layer(rng, H, F, E, norm=True), 2, (1.702, 7.0, 1.0, 1.0, 1e-5)
    x = rng.normal(size=(T, H)).astype(np.float32)
    r = moe.moe_block(layer, x, k, *c[:3], route_scale=c[3], rms_eps=c[4])
    outs, idxs, ws = brute.block(layer, x, k, *c[:3], route_scale=c[3], rms_eps=c[4])
    assert r["idx"].tolist() == idxs
    assert np.max(np.abs(r["w"] - np.array(ws))) < 1e-14
    ref = np.array(outs)
    full = x.astype(np.float64) + r["delta"]
    rms = np.sqrt(np.mean(ref ** 2))
    assert np.max(np.abs(full - ref)) <= 1e-12 * rms


def _dense_from_values(rng, rows, K):
    """Random MXFP4 matrix built from the page table: dense values + packed planes."""
    table = page_e2m1_table()
    mag = rng.integers(0, 8, size=(rows, K))
    sign = rng.integers(0, 2, size=(rows, K))
    sb = rng.integers(120, 130, size=(rows, K // 32)).astype(np.uint8)
    dense = np.array(table)[mag] * np.where(sign == 1, -1.0, 1.0) \
        * np.repeat(2.0 ** (sb.astype(np.int64) - 127), 32, axis=1)
    codes = (mag | (sign << 3)).astype(np.uint8)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return dense, packed, sb


@pytest.mark.parametrize("scale", [1.0, 1.5])
def test_single_expert_top1_equals_dense_swiglu_ffn(scale):
    rng = np.random.default_rng(5)
    H, F, T = 96, 64, 7
    wg, gq, gs = _dense_from_values(rng, F, H)
    wu, uq, us = _dense_from_values(rng, F, H)
    wd, dq, ds = _dense_from_values(rng, H, F)
    bg, bu, bd = (rng.normal(0, 0.1, size=n).astype(np.float32) for n in (F, F, H))
    planes = ExpertPlanes(gq[None], gs[None], bg[None], uq[None], us[None], bu[None],
                          dq[None], ds[None], bd[None])
    layer = Layer(rng.normal(size=(1, H)).astype(np.float32), np.zeros(1, np.float32), planes)
    x = rng.normal(size=(T, H)).astype(np.float32)
    r = moe.moe_block(layer, x, 1, alpha=1.0, limit=1e30, up_offset=0.0, route_scale=scale)
    # dense FFN with the textbook SiLU-gated unit
    g = x.astype(np.float64) @ wg.T + bg
    u = x.astype(np.float64) @ wu.T + bu
    h = (g / (1.0 + np.exp(-g))) * u
    y = h @ wd.T + bd
    assert np.max(np.abs(r["delta"] - scale * y)) <= 1e-12 * np.max(np.abs(y))


def test_route_weight_multiplies_after_down_bias():
    rng = np.random.default_rng(9)
    H, F, E, T, k = 64, 32, 5, 6, 2
    layer = _tiny_layer(rng, H, F, E, zero_down=True)
    x = rng.normal(size=(T, H)).astype(np.float32)
    r = moe.moe_block(layer, x, k, 1.702, 7.0, 1.0)
    expect = np.zeros((T, H))
    for t in range(T):
        for j in range(k):
            expect[t] += r["w"][t, j] * layer.experts.down_bias[r["idx"][t, j]]
    assert np.max(np.abs(r["delta"] - expect)) < 1e-15


def test_clamps_are_hit_and_matter_on_tiny_config():
    cfg = config_by_id(1)
    layer = make_layer(cfg)
    x, _ = make_activations(cfg)
    stats = {}
    r = moe.block_for_config(cfg, layer, x, stats=stats)
    assert stats["gate_clamped"] / stats["elements"] > 0.1
    assert stats["up_clamped"] / stats["elements"] > 0.1
    unclamped = moe.moe_block(layer, x, cfg.k, cfg.alpha, 1e30, cfg.up_offset)
    assert np.max(np.abs(unclamped["delta"] - r["delta"])) > 1.0


def test_clamps_are_hit_on_large_shapes():
    for cid in (2, 5):
        cfg = scaled(config_by_id(cid), T=2, E=4, k=2, n_shared=0)
        layer = make_layer(cfg)
        x, _ = make_activations(cfg, rows=2)
        stats = {}
        moe.block_for_config(cfg, layer, x, stats=stats)
        assert stats["gate_clamped"] > 0 and stats["up_clamped"] > 0


# ---------------------------------------------------------------- permutation
def test_permutation_invariants():
    rng = np.random.default_rng(13)
    T, E, k = 37, 8, 3
    idx = moe.top_k(rng.normal(size=(T, E)), k)
    counts, offsets, perm, inv = moe.permutation(idx, E)
    R = T * k
    assert counts.sum() == R and offsets[0] == 0 and offsets[-1] == R
    assert np.all(np.diff(offsets) == counts)
    assert sorted(perm.tolist()) == list(range(R))          # bijection
    assert np.all(perm[inv] == np.arange(R))
    flat = idx.reshape(-1)
    for e in range(E):
        seg = perm[offsets[e]:offsets[e + 1]]
        assert np.all(flat[seg] == e)
        assert np.all(np.diff(seg // k) > 0)                # ascending token, one slot each
    # brute count check against itertools
    for e in range(E):
        assert counts[e] == sum(1 for v in itertools.chain(*idx.tolist()) if v == e)


# ---------------------------------------------------------------- RMSNorm
def test_rmsnorm_constant_vector_closed_form():
    for c in (0.01, 1.0, 3.0, 250.0):
        x = np.full((1, 64), c)
        xn = moe.rms_norm(x, np.ones(64), 1e-5)
        assert np.allclose(xn, 1.0 / math.sqrt(1.0 + 1e-5 / c ** 2), rtol=1e-15, atol=0)
        assert np.allclose(moe.rms_norm(-x, 2 * np.ones(64), 1e-5), -2 * xn, rtol=1e-15, atol=0)


def test_rmsnorm_unit_mean_square():
    x = np.random.default_rng(2).normal(size=(5, 200)) * 40
    xn = moe.rms_norm(x, np.ones(200), 0.0)
    assert np.allclose(np.mean(xn ** 2, axis=1), 1.0, rtol=1e-14, atol=0)


# ---------------------------------------------------------------- constants
def test_config_constants_match_pages():
    with open(os.path.join(GOLDEN, "model_constants.json")) as f:
        pages = json.load(f)
    g, d = pages["gpt_oss"], pages["ds4_flash"]
    for cid in (2, 3, 4):
        c = config_by_id(cid)
        assert (c.H, c.F, c.E, c.k) == (g["HIDDEN"], g["EXPERT_HIDDEN"], g["EXPERTS"],
                                        g["ACTIVE_EXPERTS"])
        assert (c.alpha, c.limit) == (g["SWIGLU_ALPHA"], g["SWIGLU_LIMIT"])
    c4 = config_by_id(4)
    assert c4.layers == g["LAYERS"] and c4.rms_eps == g["EPSILON"]
    assert c4.T == g["PREFILL_EXPERT_PARALLEL_ROWS"] and config_by_id(3).T == g["PREFILL_BATCH_SIZE"]
    c5 = config_by_id(5)
    assert (c5.H, c5.F, c5.E, c5.k, c5.n_shared) == (d["n_embd"], d["n_ff_exp"], d["n_expert"],
                                                     d["n_expert_used"], d["n_expert_shared"])
    assert c5.route_scale == d["expert_weight_scale"] and c5.limit == d["swiglu_clamp_exp"]
    p, c6 = pages["ds4_pro"], config_by_id(6)
    assert (c6.H, c6.F, c6.E, c6.k, c6.n_shared) == (p["n_embd"], p["n_ff_exp"], p["n_expert"],
                                                     p["n_expert_used"], p["n_expert_shared"])
    assert c6.route_scale == p["expert_weight_scale"] and c6.limit == p["swiglu_clamp_exp"]
    assert (c6.alpha, c6.up_offset, c6.act_dtype, c6.router, c6.T) == (
        c5.alpha, c5.up_offset, c5.act_dtype, c5.router, c5.T)


def test_stack_chains_float32_outputs():
    rng = np.random.default_rng(21)
    layers = [_tiny_layer(rng, 64, 32, 4, norm=True) for _ in range(2)]
    x = rng.normal(size=(3, 64)).astype(np.float32)
    outs = moe.moe_stack(layers, x, 2, 1.702, 7.0, 1.0, rms_eps=1e-5)
    one = moe.moe_block(layers[0], x, 2, 1.702, 7.0, 1.0, rms_eps=1e-5)["out"]
    two = moe.moe_block(layers[1], one, 2, 1.702, 7.0, 1.0, rms_eps=1e-5)["out"]
    assert outs[1]["out"].tobytes() == two.tobytes()
