"""The allocation-free decode entry point (moe_forward_decode_noalloc), through
the C ABI: two calls in a row on the library's fixed per-GPU scratch, the
second with a smaller input, each against moe_forward_decode with a caller
workspace on the same input. Routing exports must be equal; outputs within
the parity bar (max |err| <= 2e-3 x RMS)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mxfp4_expert_ffn_amd as mx
from mxfp4_expert_ffn_amd import _lib
from mxfp4_expert_ffn_amd.device import workspace
from workloads import config_by_id, make_layer, scaled
from workloads.gen import make_activations

from gpu_util import TOL, device_input, rel_err, shape_of, upload

pytestmark = pytest.mark.gpu


def _route(T, k, E):
    i32 = dict(dtype=torch.int32, device="cuda")
    return dict(topk_idx=torch.full((T, k), -1, **i32),
                topk_w=torch.full((T, k), -1.0, dtype=torch.float32, device="cuda"),
                counts=torch.full((E,), -1, **i32), perm=torch.full((T * k,), -1, **i32))


def _case(cfg, T):
    layer = make_layer(cfg)
    x, xb = make_activations(cfg, rows=T)
    return dict(cfg=cfg, T=T, dl=upload(cfg, layer), shape=shape_of(cfg, T),
                xd=device_input(cfg, x, xb))


def _both(c):
    cfg, T, dl, shape, xd = c["cfg"], c["T"], c["dl"], c["shape"], c["xd"]
    assert mx.moe_workspace_bytes(shape) <= _lib.MOE_NOALLOC_SCRATCH_BYTES
    args = (shape, xd, dl.router_w, dl.router_b, dl.experts_copy(0))
    out_r = torch.full((T, cfg.H), float("nan"), dtype=torch.float32, device="cuda")
    ro_r = _route(T, cfg.k, cfg.E)
    mx.moe_forward_decode(*args, out_r, workspace(shape), norm_w=dl.norm_w,
                          shared=dl.shared_copy(0), route_out=ro_r)
    out_n = torch.full_like(out_r, float("nan"))
    ro_n = _route(T, cfg.k, cfg.E)
    mx.moe_forward_decode_noalloc(*args, out_n, norm_w=dl.norm_w, shared=dl.shared_copy(0),
                                  route_out=ro_n)
    torch.cuda.synchronize()
    for f in ro_r:
        assert torch.equal(ro_n[f], ro_r[f]), f
    a, b = out_n.cpu().numpy(), out_r.cpu().numpy()
    assert np.isfinite(a).all()
    err = rel_err(a, b)
    assert err <= TOL, f"max|err|/rms = {err:.3e}"
    return err


def test_noalloc_decode_two_calls_second_smaller():
    print("\n[case] no-alloc decode: DS4-shaped T=16 bf16 + shared, then gpt-oss T=2", flush=True)
    ds4 = scaled(config_by_id(5), E=16)          # H=4096, F=2048, top-6, shared expert, bf16
    big = _case(ds4, 16)
    small = _case(config_by_id(2), 2)              # H=F=2880, 32 experts, top-4, float32
    assert mx.moe_workspace_bytes(small["shape"]) < mx.moe_workspace_bytes(big["shape"])
    _both(big)
    _both(small)       # the scratch still holds the first call's contents
    _both(big)         # and back


def test_noalloc_decode_rejects_oversized_shape_on_gpu():
    print("\n[case] no-alloc decode: oversized shape rejected", flush=True)
    H = F = 8192
    shape = mx.make_shape(T=64, H=H, F=F, E=512, k=8, act_dtype="bf16", n_shared=1)
    assert mx.moe_workspace_bytes(shape) > _lib.MOE_NOALLOC_SCRATCH_BYTES
    # rejected on the host before any launch: the buffers are never read
    x = torch.zeros((64, H), dtype=torch.int16, device="cuda")
    out = torch.empty((64, H), dtype=torch.float32, device="cuda")
    w = torch.zeros((512, H), dtype=torch.float32, device="cuda")
    b = torch.zeros(512, dtype=torch.float32, device="cuda")
    ex = torch.empty(256, dtype=torch.uint8, device="cuda")
    with pytest.raises(mx.MoeError) as ei:
        mx.moe_forward_decode_noalloc(shape, x, w, b, ex, out, shared=ex)
    assert ei.value.code == _lib.MOE_ERR_UNSUPPORTED
    torch.cuda.synchronize()
