"""The C-ABI library: loads, exports what the header declares, packs blobs
per the documented layout, and rejects bad arguments on the host before
touching a GPU. No compute calls here (runs without a GPU)."""
import ctypes
import glob
import os
import re

import numpy as np
import pytest

import mxfp4_expert_ffn_amd as mx
from mxfp4_expert_ffn_amd import _lib
from workloads import config_by_id, make_layer, scaled

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"^\s*(?:int|size_t|const char \*)\s*(moe_\w+)\s*\(", text, re.M))
    return names


def test_header_declares_the_entry_points():
    names = declared_symbols()
    for n in ("moe_route", "moe_forward_decode", "moe_forward_prefill", "moe_blob_layout_get",
              "moe_workspace_bytes", "moe_dequant_debug", "moe_pack_experts", "moe_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    for n in declared_symbols():
        assert hasattr(lib, n), n
        assert n in _lib.SIGNATURES, f"binding lacks {n}"


def _shape(**kw):
    base = dict(T=4, H=256, F=128, E=8, k=2)
    base.update(kw)
    return mx.make_shape(**base)


def test_blob_layout_offsets_and_sizes():
    for H, F in ((256, 256), (2880, 2880), (4096, 2048), (320, 96)):
        L = mx.moe_blob_layout_get(_shape(H=H, F=F))
        planes = [("gate_q", F * H // 2), ("up_q", F * H // 2), ("down_q", H * F // 2),
                  ("gate_s", F * H // 32), ("up_s", F * H // 32), ("down_s", H * F // 32),
                  ("gate_b", 4 * F), ("up_b", 4 * F), ("down_b", 4 * H)]
        end = 0
        for name, size in planes:
            assert L[name] % 256 == 0 and L[name] >= end, name
            end = L[name] + size
        assert L["bytes"] == end and L["stride"] % 4096 == 0 and L["stride"] >= end
        # algorithmic bytes: 17 bytes per 32 weights plus fp32 biases, up to plane padding
        alg = 3 * F * H * 17 // 32 + 4 * (2 * F + H)
        assert alg <= L["bytes"] < alg + 9 * 256
    assert mx.moe_blob_layout_get(_shape(H=2880, F=2880))["bytes"] == 13254144
    assert mx.moe_blob_layout_get(_shape(H=4096, F=2048))["bytes"] == 13402112


def _tiled(codes, scales):
    """Row-major codes [rows, K/2] and scales [rows, K/32] laid out in the
    blob's tiled order, written from the header's offset formulas."""
    rows, nb = scales.shape
    q = np.zeros(rows * nb * 16, np.uint8)
    s = np.zeros(rows * nb, np.uint8)
    for r in range(rows):
        for c in range(nb):
            qo = (r // 16) * 256 * nb + (c // 4) * 1024 + ((c % 4) * 16 + r % 16) * 16
            q[qo:qo + 16] = codes[r, 16 * c:16 * c + 16]
            s[(r // 16) * 16 * nb + (c // 4) * 64 + (c % 4) * 16 + r % 16] = scales[r, c]
    return q, s


def test_tiled_order_puts_a_wavefront_load_in_one_kilobyte():
    # the 64 lanes (block g = lane // 16, row = lane % 16) of a 128-wide step
    # read 64 distinct 16-byte blocks covering one contiguous kilobyte
    codes = np.arange(32 * 256 // 2, dtype=np.int64).reshape(32, 128).astype(np.uint8)
    scales = np.arange(32 * 8, dtype=np.int64).reshape(32, 8).astype(np.uint8)
    q, s = _tiled(codes, scales)
    for tile in range(2):
        for step in range(2):
            base = tile * 256 * 8 + step * 1024
            for lane in range(64):
                r, c = 16 * tile + lane % 16, 4 * step + lane // 16
                assert np.array_equal(q[base + 16 * lane:base + 16 * lane + 16], codes[r, 16 * c:16 * c + 16])
                assert s[tile * 16 * 8 + step * 64 + lane] == scales[r, c]


def test_pack_places_every_plane():
    cfg = scaled(config_by_id(1), E=3)
    layer = make_layer(cfg)
    shape = mx.make_shape(**cfg.shape_kwargs())
    L = mx.moe_blob_layout_get(shape)
    blob = mx.moe_pack_experts(shape, layer.experts)
    assert blob.size == 3 * L["stride"]
    H, F = cfg.H, cfg.F
    for e in range(3):
        b = blob[e * L["stride"]:(e + 1) * L["stride"]]
        ex = layer.experts

        def plane(name, n):
            return b[L[name]:L[name] + n]
        for m in ("gate", "up", "down"):
            q, sc = _tiled(getattr(ex, f"{m}_codes")[e], getattr(ex, f"{m}_scales")[e])
            assert np.array_equal(plane(f"{m}_q", F * H // 2), q), m
            assert np.array_equal(plane(f"{m}_s", F * H // 32), sc), m
        assert np.array_equal(plane("up_b", 4 * F).view(np.float32), ex.up_bias[e])
        assert np.array_equal(plane("down_b", 4 * H).view(np.float32), ex.down_bias[e])
        assert not b[L["bytes"]:].any()


def test_workspace_bytes():
    assert mx.moe_workspace_bytes(_shape()) > 0
    big = mx.moe_workspace_bytes(_shape(T=2048, H=4096, F=2048, E=256, k=6, n_shared=1))
    # FP8 terms of the SwiGLU output (4 codes + scales per value) and the
    # fp32 down output per routed row dominate
    rows = 2048 * 6 + 2048
    act = rows * 2048 * 4 * 33 // 32 + rows * 4096 * 4
    assert act < big < act + 2048 * 4096 * (12 + 5) + 16 * 2048 * 256 * 8 + (1 << 22)
    with pytest.raises(mx.MoeError):
        mx.moe_workspace_bytes(_shape(k=9))


FAKE = 1 << 20  # a non-NULL, aligned address; validation fails before any use


def _call(fn_name, shape, **over):
    lib = _lib.load()
    args = dict(hidden=FAKE, norm_w=None, router_w=FAKE, router_b=FAKE, routing=None,
                experts=FAKE, shared=None, out=FAKE, ro=None, ws=FAKE, ws_bytes=1 << 40,
                stream=None)
    args.update(over)
    fn = getattr(lib, fn_name)
    return fn(ctypes.byref(shape), args["hidden"], args["norm_w"], args["router_w"],
              args["router_b"], args["routing"], args["experts"], args["shared"], args["out"],
              args["ro"], args["ws"], args["ws_bytes"], args["stream"])


def _routing(**kw):
    r = _lib.MoeRouting()
    for k, v in kw.items():
        setattr(r, k, v)
    return ctypes.byref(r)


@pytest.mark.parametrize("fn", ["moe_forward_decode", "moe_forward_prefill"])
@pytest.mark.parametrize("case", [
    ("k > E", dict(k=9, E=8), {}, _lib.MOE_ERR_INVALID_ARG),
    ("k = 0", dict(k=0), {}, _lib.MOE_ERR_INVALID_ARG),
    ("E > 512", dict(E=513), {}, _lib.MOE_ERR_INVALID_ARG),
    ("H % 32", dict(H=100), {}, _lib.MOE_ERR_INVALID_ARG),
    ("F % 32", dict(F=40), {}, _lib.MOE_ERR_INVALID_ARG),
    ("null hidden", {}, dict(hidden=None), _lib.MOE_ERR_INVALID_ARG),
    ("null experts", {}, dict(experts=None), _lib.MOE_ERR_INVALID_ARG),
    ("misaligned hidden", {}, dict(hidden=FAKE + 4), _lib.MOE_ERR_INVALID_ARG),
    ("misaligned blob", {}, dict(experts=FAKE + 16), _lib.MOE_ERR_INVALID_ARG),
    ("shared missing", dict(n_shared=1), {}, _lib.MOE_ERR_INVALID_ARG),
    ("bad dtype", dict(act_dtype="x"), {}, None),
    ("small workspace", {}, dict(ws_bytes=1024), _lib.MOE_ERR_WORKSPACE),
    ("null workspace", {}, dict(ws=None), _lib.MOE_ERR_WORKSPACE),
    ("act_quant 3", dict(act_quant=3), {}, _lib.MOE_ERR_INVALID_ARG),
    ("table without ids", {}, dict(routing=_routing(tid2eid=FAKE, vocab=10)), _lib.MOE_ERR_INVALID_ARG),
    ("table with vocab 0", {}, dict(routing=_routing(tid2eid=FAKE, token_ids=FAKE)),
     _lib.MOE_ERR_INVALID_ARG),
    ("misaligned table", {}, dict(routing=_routing(tid2eid=FAKE + 2, token_ids=FAKE, vocab=4)),
     _lib.MOE_ERR_INVALID_ARG),
    ("misaligned bias", {}, dict(routing=_routing(sel_bias=FAKE + 1)), _lib.MOE_ERR_INVALID_ARG),
    ("act_quant -1", dict(act_quant=-1), {}, _lib.MOE_ERR_INVALID_ARG),
    ("misaligned workspace", {}, dict(ws=FAKE + 64), _lib.MOE_ERR_WORKSPACE),
    ("nonpositive limit", dict(limit=0.0), {}, _lib.MOE_ERR_INVALID_ARG),
    ("nonpositive scale", dict(route_scale=-1.0), {}, _lib.MOE_ERR_INVALID_ARG),
], ids=lambda c: c[0] if isinstance(c, tuple) else c)
def test_host_validation_errors(fn, case):
    _, skw, over, code = case
    shape = _shape(**skw)
    if code is None:  # make_shape maps unknown dtypes to f32; poke an invalid value directly
        shape.act_dtype = 7
        code = _lib.MOE_ERR_INVALID_ARG
    rc = _call(fn, shape, **over)
    assert rc == code
    assert mx.moe_last_error()


def test_decode_rejects_large_T_and_bf16_alias():
    assert _call("moe_forward_decode", _shape(T=65)) == _lib.MOE_ERR_UNSUPPORTED
    assert _call("moe_forward_decode", _shape(H=16384)) == _lib.MOE_ERR_UNSUPPORTED
    assert _call("moe_forward_prefill", _shape(act_dtype="bf16"), out=FAKE, hidden=FAKE) == \
        _lib.MOE_ERR_INVALID_ARG


def test_zero_tokens_is_ok_without_pointers():
    shape = _shape(T=0)
    assert _call("moe_forward_prefill", shape, hidden=None, out=None, ws=None) == 0
    assert _call("moe_forward_decode", shape, hidden=None, out=None, ws=None) == 0


def test_dequant_debug_rejects_bad_arguments():
    lib = _lib.load()
    s = _shape()
    assert lib.moe_dequant_debug(ctypes.byref(s), FAKE, 3, 0, FAKE, None) == _lib.MOE_ERR_INVALID_ARG
    assert lib.moe_dequant_debug(ctypes.byref(s), FAKE, 0, 3, FAKE, None) == _lib.MOE_ERR_INVALID_ARG
    assert lib.moe_dequant_debug(ctypes.byref(s), FAKE + 8, 0, 0, FAKE, None) == _lib.MOE_ERR_INVALID_ARG


def test_noalloc_decode_rejects_shapes_past_its_scratch():
    # the size check runs before any device call, so it holds without a GPU
    lib = _lib.load()
    big = mx.make_shape(T=64, H=8192, F=8192, E=512, k=8, n_shared=1)
    assert mx.moe_workspace_bytes(big) > _lib.MOE_NOALLOC_SCRATCH_BYTES
    rc = lib.moe_forward_decode_noalloc(ctypes.byref(big), None, None, None, None, None, None, None,
                                        None, None, None)
    assert rc == _lib.MOE_ERR_UNSUPPORTED
    assert "MOE_NOALLOC_SCRATCH_BYTES" in mx.moe_last_error()
    bad = mx.make_shape(T=1, H=100, F=64, E=4, k=2)  # H not a multiple of 32
    assert lib.moe_forward_decode_noalloc(ctypes.byref(bad), None, None, None, None, None, None,
                                          None, None, None, None) == _lib.MOE_ERR_INVALID_ARG


def test_noalloc_scratch_covers_the_decode_workloads():
    for cid in (1, 2, 4, 5):
        cfg = config_by_id(cid)
        s = mx.make_shape(**cfg.shape_kwargs(64 if cid != 1 else cfg.T))
        assert mx.moe_workspace_bytes(s) <= _lib.MOE_NOALLOC_SCRATCH_BYTES, cid


@pytest.mark.parametrize("cid,tile,x_terms", [(1, 16, 4), (3, 16, 4), (4, 32, 3), (5, 64, 1), (6, 64, 1), (7, 64, 1), (8, 64, 1)])
def test_prefill_plan_of_the_workloads(cid, tile, x_terms):
    cfg = config_by_id(cid)
    plan = mx.moe_prefill_plan(mx.make_shape(**cfg.shape_kwargs()), with_norm=cfg.rms_eps is not None)
    assert plan["tile_rows"] == tile and plan["x_terms"] == x_terms
    assert plan["act_terms"] == 3
    # 16-row tiles and 32-row tiles with FP8 terms (4-wavefront workgroups),
    # 64-row tiles with the bfloat16 or MX-FP4 operand (two A fragments per
    # wavefront)
    narrow = tile == 16 or (tile == 32 and x_terms == 3) or (tile == 64 and x_terms <= 1)
    assert plan["gate_up_features"] == (128 if narrow else 256)
    assert plan["down_rows"] == (512 if tile == 64 else 256)


@pytest.mark.parametrize("cid", [3, 4, 5, 6])
def test_prefill_plan_of_the_quantised_mode(cid):
    cfg = config_by_id(cid)
    kw = cfg.shape_kwargs()
    exact = mx.moe_prefill_plan(mx.make_shape(**kw), with_norm=cfg.rms_eps is not None)
    quant = mx.moe_prefill_plan(mx.make_shape(**kw, act_quant=1), with_norm=cfg.rms_eps is not None)
    assert quant["x_terms"] == 0
    # same tiling; the gate/up workgroup width follows the operand (4-wavefront
    # workgroups only for 32-row tiles with FP8 terms)
    skip = ("x_terms", "gate_up_features")
    assert {k: v for k, v in quant.items() if k not in skip} == \
        {k: v for k, v in exact.items() if k not in skip}
    assert quant["gate_up_features"] == (256 if quant["tile_rows"] == 32 else 128)
    assert quant["down_rows"] == exact["down_rows"]
    both = mx.moe_prefill_plan(mx.make_shape(**kw, act_quant=2), with_norm=cfg.rms_eps is not None)
    assert both["x_terms"] == 0 and both["act_terms"] == 0
    assert both["tile_rows"] == exact["tile_rows"]
    # MX-FP4 down rows on 64-row tiles: two A fragments per wavefront
    assert both["down_rows"] == 256


def test_decode_rejects_the_quantised_mode():
    # the mode check runs before any device call
    assert _call("moe_forward_decode", _shape(act_quant=1)) == _lib.MOE_ERR_UNSUPPORTED
    assert _call("moe_forward_decode", _shape(act_quant=2)) == _lib.MOE_ERR_UNSUPPORTED
    assert _call("moe_forward_decode", _shape(T=64, act_quant=1)) == _lib.MOE_ERR_UNSUPPORTED


def test_act_quant_debug_rejects_bad_arguments():
    lib = _lib.load()
    s = _shape()
    fn = lib.moe_act_quant_debug
    assert fn(ctypes.byref(s), None, None, FAKE, FAKE, FAKE, 1 << 40, None) == _lib.MOE_ERR_INVALID_ARG
    assert fn(ctypes.byref(s), FAKE, None, None, FAKE, FAKE, 1 << 40, None) == _lib.MOE_ERR_INVALID_ARG
    assert fn(ctypes.byref(s), FAKE + 4, None, FAKE, FAKE, FAKE, 1 << 40, None) == _lib.MOE_ERR_INVALID_ARG
    assert fn(ctypes.byref(s), FAKE, None, FAKE, FAKE, FAKE, 16, None) == _lib.MOE_ERR_WORKSPACE
    assert fn(ctypes.byref(_shape(H=100)), FAKE, None, FAKE, FAKE, FAKE, 1 << 40, None) == \
        _lib.MOE_ERR_INVALID_ARG
    assert fn(ctypes.byref(_shape(T=0)), None, None, None, None, None, 0, None) == 0


def test_prefill_plan_rejects_bad_arguments():
    with pytest.raises(mx.MoeError):
        mx.moe_prefill_plan(mx.make_shape(T=4, H=100, F=64, E=4, k=2))
    lib = _lib.load()
    assert lib.moe_prefill_plan(ctypes.byref(_shape()), 0, None) == _lib.MOE_ERR_INVALID_ARG
