"""The prefill gate/up GEMM takes a bfloat16 expert input (no RMSNorm) as it
is, on the bfloat16 matrix cores, against weights decoded to bfloat16 in
registers. A float32 input holding the same values goes through FP8 terms
instead, which carry a bfloat16 value whole. Both forms multiply the same
values exactly and accumulate in float32, so the two block outputs may differ
only by float32 summation order (and where that moves an FP8-term rounding of
the SwiGLU output). Bar: max |bf16 path - float32 path| <= 2e-4 x RMS, ten
times tighter than the oracle bar; routing identical. Both results are also
held to the oracle bar.

Page: goosedump `gpt_oss.rs` `mixture_of_experts` (the block); antirez ds4.c
`DS4_SHAPE_FLASH` (bf16 activations, shared expert).
"""
import numpy as np
import pytest
import torch

import mxfp4_expert_ffn_amd as mx
from oracle import moe as omoe
from workloads import config_by_id, make_layer, scaled
from workloads.gen import make_activations

from gpu_util import TOL, device_input, rel_err, run_forward, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mx._lib.load()


# 16-, 32- and 64-row tiles of the bfloat16 operand (the plan picks them from
# the rows per expert), the last at the DeepSeek-V4-Flash shape
CASES = [
    (dict(T=24, H=512, F=256, E=16, k=4), 16),
    (dict(T=96, H=2880, F=352, E=8, k=4), 32),
    (dict(T=2048), 64),
]


@pytest.mark.parametrize("kw,tile", CASES, ids=["tile16", "tile32", "ds4_tile64"])
def test_bf16_operand_equals_fp8_terms(kw, tile):
    cfg = scaled(config_by_id(5), **kw)
    print(f"\n[case] bf16 operand vs FP8 terms, tile {tile}, {kw}", flush=True)
    assert cfg.act_dtype == "bf16" and not cfg.rms_eps
    layer = make_layer(cfg)
    x, xb = make_activations(cfg)           # x: the bf16 values widened exactly
    dl = upload(cfg, layer)
    kb = cfg.shape_kwargs()
    kf = dict(kb, act_dtype="f32")
    plan_b = mx.moe_prefill_plan(mx.make_shape(**kb), with_norm=False)
    plan_f = mx.moe_prefill_plan(mx.make_shape(**kf), with_norm=False)
    assert plan_b["x_terms"] == 1 and plan_b["tile_rows"] == tile
    assert plan_f["x_terms"] >= 3 and plan_f["tile_rows"] == tile
    out_b, ro_b = run_forward("prefill", mx.make_shape(**kb), dl, device_input(cfg, x, xb))
    xf = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    out_f, ro_f = run_forward("prefill", mx.make_shape(**kf), dl, xf)
    assert torch.equal(ro_b["topk_idx"], ro_f["topk_idx"])
    assert torch.equal(ro_b["perm"], ro_f["perm"])
    ob, of = out_b.cpu().numpy(), out_f.cpu().numpy()
    d = rel_err(ob, of)
    toks = np.arange(cfg.T) if cfg.T <= 96 else np.random.default_rng(tile).choice(cfg.T, 16, replace=False)
    ref = omoe.block_for_config(cfg, layer, x, tokens=toks)
    eb = rel_err(ob[toks], x[toks] + ref["delta"])
    ef = rel_err(of[toks], x[toks] + ref["delta"])
    print(f"tile {tile}: max|bf16 - fp32 path|/rms = {d:.2e}; vs oracle {eb:.2e} / {ef:.2e}")
    assert d <= 2e-4
    assert eb <= TOL and ef <= TOL
