"""The routed MoE feed-forward block, written plainly in numpy float64.

What one block computes (pages: turbospark-runtime `gptoss/mod.rs`, module
doc "One decoder layer"; goosedump `gpt_oss.rs`, `mixture_of_experts` and
`mixture_of_experts_batch`):

    xn     = rms_norm(x)                          (only where the layer has a norm)
    logits = xn @ router^T + router_bias
    idx    = top-k of logits (k largest; ties to the lower expert index), or of
             logits + a selection-only bias, or a hash table's row (DeepSeek-V4)
    w      = route_scale * softmax(logits[idx])   (softmax over the k selected)
    y_j    = down_j(swiglu(gate_j(xn) + bg_j, up_j(xn) + bu_j)) + bd_j
    out    = resid + sum_j w_j * y_j  (+ shared expert with weight 1)

All arithmetic is float64; contractions use numpy `@` (BLAS dgemm) on float64
operands. The block output is rounded once to float32. Top-k, the permutation
and the SwiGLU are explicit code.
"""
from __future__ import annotations

import numpy as np

from . import act_quant as act_quant_mod
from . import mxfp4


# --------------------------------------------------------------------------
# RMSNorm. Page: antirez `ds4.c`, `rms_norm_weight` (sum of squares in double,
# x * 1/sqrt(mean + eps) * weight); eps 1e-5 from the goosedump constants
# block and the turbospark layer doc. Pinned by the constant-vector closed form.
# --------------------------------------------------------------------------
def rms_norm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(gamma, dtype=np.float64)


# --------------------------------------------------------------------------
# Router. Page: goosedump `mixture_of_experts_batch` (router matmul, then
# `add_bias_batch`) and `mixture_of_experts` (matvec then `add_bias`).
# fp32 x fp32 products are exact in float64.
# --------------------------------------------------------------------------
def router_logits(xn: np.ndarray, router_w: np.ndarray, router_b: np.ndarray) -> np.ndarray:
    xn = np.asarray(xn, dtype=np.float64)
    return xn @ np.asarray(router_w, dtype=np.float64).T + np.asarray(router_b, dtype=np.float64)


# --------------------------------------------------------------------------
# Top-k. Page: goosedump `top_experts`: a slot is taken only by a strictly
# greater value, so among equal values the lower expert index wins, and the
# selected experts come out by descending value. Written here as k rounds of
# "take the first maximum of what is left" (np.argmax returns the first, i.e.
# lowest-index, maximum). Pinned by brute force over k-subsets and by the
# page's insertion rule restated in the tests.
# --------------------------------------------------------------------------
def top_k(logits: np.ndarray, k: int) -> np.ndarray:
    logits = np.asarray(logits, dtype=np.float64)
    T, E = logits.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    left = logits.copy()
    idx = np.empty((T, k), dtype=np.int32)
    rows = np.arange(T)
    for j in range(k):
        best = np.argmax(left, axis=1)
        idx[:, j] = best
        left[rows, best] = -np.inf
    return idx


# --------------------------------------------------------------------------
# Route weights. Page: goosedump `mixture_of_experts` applies `softmax` to the
# k values `top_experts` returned (selection first, softmax second); antirez
# `ds4.c` `DS4_SHAPE_FLASH` sets `expert_weight_scale` 1.5 and
# `config_validate_model` requires normalised expert weights. Reading: the
# weights are route_scale * softmax over the selected logits.
# --------------------------------------------------------------------------
def route_weights(logits: np.ndarray, idx: np.ndarray, route_scale: float) -> np.ndarray:
    sel = np.take_along_axis(np.asarray(logits, dtype=np.float64), idx.astype(np.int64), axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    return route_scale * z / z.sum(axis=1, keepdims=True)


# --------------------------------------------------------------------------
# Permutation. Page: goosedump `mixture_of_experts_batch` pushes each
# (token, slot) route onto its expert's list in ascending token order;
# `route_output_index` numbers a route token*k + slot; `mix_expert_outputs`
# requires every route to land exactly once. Here:
#   counts[e]  number of routes to expert e
#   offsets[e] exclusive prefix sum of counts (offsets[E] = T*k)
#   perm[p]    route id (t*k + j) at position p, grouped by expert, each
#              group in ascending route id (= ascending token)
#   inv[r]     position of route r, so perm[inv[r]] == r
# --------------------------------------------------------------------------
def permutation(idx: np.ndarray, E: int):
    flat = np.asarray(idx, dtype=np.int64).reshape(-1)
    R = flat.size
    counts = np.zeros(E, dtype=np.int32)
    for e in flat:
        counts[e] += 1
    offsets = np.zeros(E + 1, dtype=np.int32)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    perm = np.empty(R, dtype=np.int32)
    inv = np.empty(R, dtype=np.int32)
    for e in range(E):
        routes = np.nonzero(flat == e)[0]          # ascending route ids
        perm[offsets[e]:offsets[e + 1]] = routes
    inv[perm] = np.arange(R, dtype=np.int32)
    return counts, offsets, perm, inv


# --------------------------------------------------------------------------
# Clamped SwiGLU. Pages: goosedump `swiglu_inplace(gate, up, SWIGLU_ALPHA,
# SWIGLU_LIMIT)` with alpha 1.702 and limit 7.0; turbospark layer doc
# "clamped SwiGLU"; antirez `ds4.c` clamp 10. The body is on no page.
# Reading (parity unpinned by the pages): gate clamped above at `limit`, up
# clamped to [-limit, limit], a = g * sigmoid(alpha * g) * (u + up_offset).
# up_offset is 1 for gpt-oss and 0 (with alpha 1) for the DeepSeek shape.
# --------------------------------------------------------------------------
def sigmoid(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def swiglu(g: np.ndarray, u: np.ndarray, alpha: float, limit: float, up_offset: float) -> np.ndarray:
    gc = np.minimum(g, limit)
    uc = np.clip(u, -limit, limit)
    return gc * sigmoid(alpha * gc) * (uc + up_offset)


# --------------------------------------------------------------------------
# One expert on a batch of rows. Page: goosedump `expert_batch_output` and
# `mixture_of_experts`: gate/up pair product, add both biases, SwiGLU, down
# product, add the down bias (the route weight is applied after that).
# --------------------------------------------------------------------------
def dequant_expert(planes, e: int):
    wg = mxfp4.dequant(planes.gate_codes[e], planes.gate_scales[e])
    wu = mxfp4.dequant(planes.up_codes[e], planes.up_scales[e])
    wd = mxfp4.dequant(planes.down_codes[e], planes.down_scales[e])
    return wg, wu, wd


def expert_ffn(xr: np.ndarray, planes, e: int, alpha: float, limit: float, up_offset: float,
               stats: dict | None = None, quant_act: bool = False) -> np.ndarray:
    """quant_act: the SwiGLU output, as float32, goes through the MX-FP4 round
    trip (blocks of 32 along F) before the down projection; `stats["act"]`
    then collects {"e", "a", "clamped"}: the expert, its unrounded outputs and
    where both of their inputs were clamped (for the tests' rounding-edge
    bound; the block adds the rows' tokens and slots)."""
    wg, wu, wd = dequant_expert(planes, e)
    g = xr @ wg.T + planes.gate_bias[e].astype(np.float64)
    u = xr @ wu.T + planes.up_bias[e].astype(np.float64)
    if stats is not None:
        stats["gate_clamped"] = stats.get("gate_clamped", 0) + int(np.count_nonzero(g > limit))
        stats["up_clamped"] = stats.get("up_clamped", 0) + int(np.count_nonzero(np.abs(u) > limit))
        stats["elements"] = stats.get("elements", 0) + g.size
    a = swiglu(g, u, alpha, limit, up_offset)
    if quant_act:
        if stats is not None:
            # values whose gate and up were both clamped come out as one constant
            # (no accumulated product left in them)
            both = (g >= limit) & (np.abs(u) >= limit)
            stats.setdefault("act", []).append({"e": e, "a": a, "clamped": both})
        a = act_quant_mod.quantize_rows(a.astype(np.float32))[2]
    return a @ wd.T + planes.down_bias[e].astype(np.float64)


# --------------------------------------------------------------------------
# The block. Page: goosedump `mixture_of_experts` (weighted sum over the k
# selected experts, slot by slot) and `mix_expert_outputs`; the caller adds
# the result to the residual (`vector_add` after the MoE in `forward` and
# `prefill`). Shared expert: antirez `ds4.c` `DS4_SHAPE_FLASH`
# (`n_expert_shared` 1) with no gate tensor for it; reading: weight 1.
# --------------------------------------------------------------------------
def route(xn, router_w, router_b, k: int, route_scale: float, sel_bias=None, hash_rows=None):
    logits = router_logits(xn, router_w, router_b)
    idx, sel = select_experts(logits, k, sel_bias, hash_rows)
    w = route_weights(logits, idx, route_scale)
    return logits, idx, w, sel


# --------------------------------------------------------------------------
# DeepSeek-V4 routing variants. Page: antirez `ds4.c`: `ds4_layer_weights`
# holds `ffn_exp_probs_b` and `ffn_gate_tid2eid`; `weights_validate_layout`
# declares exp_probs_b F32 [n_expert] (optional) and tid2eid I32
# [n_expert_used, n_vocab] for layers il < n_hash_layer (ggml order: the
# first dimension is the contiguous one, so the table holds one row of k
# experts per token id); `DS4_SHAPE_FLASH` sets n_hash_layer 3 and n_vocab
# 129280. The routing arithmetic itself is cut off the page. Readings:
#  - selection-only bias: the experts are the top-k (ties to the lower index)
#    of logits + exp_probs_b, taken in float64; the bias takes no part in the
#    weights, which stay route_scale * softmax over the selected experts'
#    own logits, in selection order;
#  - hash routing: a token with id v takes the k experts of table row v, in
#    row order; the router still runs, and the weights are route_scale *
#    softmax over those experts' logits.
# Parity pinned by brute force over k-subsets (`brute.block`), closed forms
# on constructed routers and the invariances in the tests.
# --------------------------------------------------------------------------
def select_experts(logits: np.ndarray, k: int, sel_bias=None, hash_rows=None):
    """Returns (idx [T, k] int32, the values the selection ranked [T, E]).

    hash_rows [T, k]: the table rows of the tokens' ids (experts in [0, E));
    else the top-k of logits (+ sel_bias [E] when given)."""
    logits = np.asarray(logits, dtype=np.float64)
    T, E = logits.shape
    if hash_rows is not None:
        idx = np.asarray(hash_rows, dtype=np.int64)
        if idx.shape != (T, k) or idx.min(initial=0) < 0 or idx.max(initial=0) >= E:
            raise ValueError("hash rows must be [T, k] experts in [0, E)")
        return idx.astype(np.int32), logits
    sel = logits if sel_bias is None else logits + np.asarray(sel_bias, dtype=np.float64)[None, :]
    return top_k(sel, k), sel


def moe_block(layer, x: np.ndarray, k: int, alpha: float, limit: float, up_offset: float,
              route_scale: float = 1.0, rms_eps: float | None = None,
              tokens=None, stats: dict | None = None, act_quant: int = 0,
              token_ids=None) -> dict:
    """Run one block on x [T, H] (exact input values; the residual is x).

    Routing is computed for all T tokens; expert outputs only for `tokens`
    (all when None). Returns float64 `delta` (the MoE sum without residual)
    and the float32 `out` rows for `tokens`, plus the routing tensors.

    act_quant 1: the experts' input (not the router's) is the float32 input
    rounded through the MX-FP4 round trip of `act_quant.quantize_rows`, in
    blocks of 32 along H (antirez `ds4.c`, the FP4 activation round trip;
    goosedump `mixture_of_experts` quantises the expert input once,
    `Q8Activation`). Reading: routing keeps the unquantised input, and the
    SwiGLU output is not quantised.
    act_quant 2: as 1, and each expert's SwiGLU output (the down projection's
    input, float32) goes through the same round trip along F.

    A layer with `sel_bias` [E] selects with the selection-only bias; one with
    `tid2eid` [vocab, k] routes token t by table row token_ids[t] (see
    `select_experts`).
    """
    x = np.asarray(x, dtype=np.float64)
    T = x.shape[0]
    xn = x if layer.norm_w is None else rms_norm(x, layer.norm_w, rms_eps)
    sel_bias = getattr(layer, "sel_bias", None)
    tid2eid = getattr(layer, "tid2eid", None)
    hash_rows = None
    if tid2eid is not None:
        if token_ids is None or len(token_ids) != T:
            raise ValueError("hash routing needs one token id per row")
        hash_rows = np.asarray(tid2eid)[np.asarray(token_ids, dtype=np.int64)]
    logits, idx, w, sel = route(xn, layer.router_w, layer.router_b, k, route_scale, sel_bias,
                                hash_rows)
    xe = xn
    if act_quant:
        xe = act_quant_mod.quantize_rows(xn.astype(np.float32))[2]
    E = layer.router_w.shape[0]
    counts, offsets, perm, inv = permutation(idx, E)
    toks = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)

    delta = np.zeros((toks.size, x.shape[1]), dtype=np.float64)
    # route outputs y[t, j] for the requested tokens, one expert at a time
    y = np.zeros((toks.size, k, x.shape[1]), dtype=np.float64)
    for e in np.unique(idx[toks]):
        rows, slots = np.nonzero(idx[toks] == e)
        y[rows, slots] = expert_ffn(xe[toks[rows]], layer.experts, int(e),
                                    alpha, limit, up_offset, stats, quant_act=act_quant == 2)
        if act_quant == 2 and stats is not None:
            stats["act"][-1].update(tokens=toks[rows], slots=slots, shared=False)
    for j in range(k):                              # slot-ordered weighted sum
        delta += w[toks, j][:, None] * y[:, j]
    if layer.shared is not None:
        for s in range(layer.shared.n):
            delta += expert_ffn(xe[toks], layer.shared, s, alpha, limit, up_offset, stats,
                                quant_act=act_quant == 2)
            if act_quant == 2 and stats is not None:
                stats["act"][-1].update(tokens=toks, slots=None, shared=True)
    out = (x[toks] + delta).astype(np.float32)
    return dict(out=out, delta=delta, logits=logits, sel=sel, idx=idx, w=w, counts=counts,
                offsets=offsets, perm=perm, inv=inv, xn=xn, xe=xe, tokens=toks,
                hashed=hash_rows is not None)


def moe_stack(layers, x: np.ndarray, k: int, alpha: float, limit: float, up_offset: float,
              route_scale: float = 1.0, rms_eps: float | None = None, token_ids=None) -> list:
    """Chain blocks: each layer's float32 output is the next layer's input.

    Page: goosedump `prefill`/`forward` apply the MoE once per layer and carry
    the hidden state; the state is stored as float32 between layers.
    """
    outs = []
    h = np.asarray(x, dtype=np.float32)
    for layer in layers:
        r = moe_block(layer, h, k, alpha, limit, up_offset, route_scale, rms_eps,
                      token_ids=token_ids)
        outs.append(r)
        h = r["out"]
    return outs


def block_for_config(cfg, layer, x, tokens=None, stats=None, act_quant: int = 0,
                     token_ids=None) -> dict:
    return moe_block(layer, x, cfg.k, cfg.alpha, cfg.limit, cfg.up_offset, cfg.route_scale,
                     cfg.rms_eps, tokens=tokens, stats=stats, act_quant=act_quant,
                     token_ids=token_ids)
