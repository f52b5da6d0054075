"""The MoE block again, in pure Python loops (no numpy), for tiny inputs.

It is a second, independent formulation that pins `oracle.moe`:
- weights decode through the page's table of eight E2M1 magnitudes
  (antirez `ds4.c`, `dsv4_e2m1fn_value_cpu`) plus the sign bit, not through
  the closed form used by `oracle.mxfp4`;
- dot products use `math.fsum` (exactly rounded sums);
- top-k enumerates every k-subset of experts and keeps the one whose members
  all precede every non-member in the order (value descending, index
  ascending), the order goosedump `top_experts` produces;
- the combine walks tokens and slots one at a time.
Inputs are the same nested arrays (numpy arrays are read element by element).
"""
from __future__ import annotations

import itertools
import math

PAGE_E2M1_MAGNITUDES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def decode_code(code: int) -> float:
    mag = PAGE_E2M1_MAGNITUDES[code & 7]
    return -mag if code & 8 else mag


def decode_matrix(packed, scales, rows: int, K: int):
    w = []
    for r in range(rows):
        row = []
        for j in range(K):
            byte = int(packed[r][j // 2])
            code = byte & 15 if j % 2 == 0 else byte >> 4
            row.append(decode_code(code) * 2.0 ** (int(scales[r][j // 32]) - 127))
        w.append(row)
    return w


def precedes(a, b) -> bool:
    """(value, index) a comes before b: larger value, or equal value and lower index."""
    return a[0] > b[0] or (a[0] == b[0] and a[1] < b[1])


def top_k_bruteforce(logits, k: int):
    E = len(logits)
    items = [(float(logits[e]), e) for e in range(E)]
    found = None
    for subset in itertools.combinations(range(E), k):
        inside = [items[e] for e in subset]
        outside = [items[e] for e in range(E) if e not in subset]
        if all(precedes(a, b) for a in inside for b in outside):
            if found is not None:
                raise AssertionError("two top-k subsets")
            found = inside
    # order the winning subset: repeatedly pick the member preceding all others
    ordered = []
    rest = list(found)
    while rest:
        first = [a for a in rest if all(a is b or precedes(a, b) for b in rest)][0]
        ordered.append(first[1])
        rest.remove(first)
    return ordered


def swiglu_scalar(g: float, u: float, alpha: float, limit: float, up_offset: float) -> float:
    g = g if g < limit else limit
    u = -limit if u < -limit else (limit if u > limit else u)
    return g / (1.0 + math.exp(-alpha * g)) * (u + up_offset) if -alpha * g < 700 else 0.0


def expert(x, planes, e: int, H: int, F: int, alpha, limit, up_offset):
    wg = decode_matrix(planes.gate_codes[e], planes.gate_scales[e], F, H)
    wu = decode_matrix(planes.up_codes[e], planes.up_scales[e], F, H)
    wd = decode_matrix(planes.down_codes[e], planes.down_scales[e], H, F)
    a = []
    for f in range(F):
        g = math.fsum(wg[f][h] * float(x[h]) for h in range(H)) + float(planes.gate_bias[e][f])
        u = math.fsum(wu[f][h] * float(x[h]) for h in range(H)) + float(planes.up_bias[e][f])
        a.append(swiglu_scalar(g, u, alpha, limit, up_offset))
    return [math.fsum(wd[h][f] * a[f] for f in range(F)) + float(planes.down_bias[e][h])
            for h in range(H)]


def block(layer, x, k: int, alpha: float, limit: float, up_offset: float,
          route_scale: float = 1.0, rms_eps=None, token_ids=None):
    """A layer with `sel_bias` ranks logits + bias in the subset enumeration
    (weights from the logits alone); one with `tid2eid` takes row
    token_ids[t] of the table as the token's experts, in row order."""
    T, H = len(x), len(x[0])
    E = len(layer.router_w)
    F = len(layer.experts.gate_bias[0])
    outs, idxs, ws = [], [], []
    for t in range(T):
        xt = [float(v) for v in x[t]]
        if layer.norm_w is not None:
            ms = math.fsum(v * v for v in xt) / H
            inv = 1.0 / math.sqrt(ms + rms_eps)
            xt = [xt[h] * inv * float(layer.norm_w[h]) for h in range(H)]
        logits = [math.fsum(float(layer.router_w[e][h]) * xt[h] for h in range(H))
                  + float(layer.router_b[e]) for e in range(E)]
        sel_bias = getattr(layer, "sel_bias", None)
        tid2eid = getattr(layer, "tid2eid", None)
        if tid2eid is not None:
            sel = [int(e) for e in tid2eid[int(token_ids[t])]]
        elif sel_bias is not None:
            sel = top_k_bruteforce([logits[e] + float(sel_bias[e]) for e in range(E)], k)
        else:
            sel = top_k_bruteforce(logits, k)
        m = max(logits[e] for e in sel)
        z = [math.exp(logits[e] - m) for e in sel]
        s = math.fsum(z)
        w = [route_scale * v / s for v in z]
        acc = [0.0] * H
        for j in range(k):
            y = expert(xt, layer.experts, sel[j], H, F, alpha, limit, up_offset)
            acc = [acc[h] + w[j] * y[h] for h in range(H)]
        if layer.shared is not None:
            for si in range(len(layer.shared.gate_bias)):
                y = expert(xt, layer.shared, si, H, F, alpha, limit, up_offset)
                acc = [acc[h] + y[h] for h in range(H)]
        outs.append([float(x[t][h]) + acc[h] for h in range(H)])
        idxs.append(sel)
        ws.append(w)
    return outs, idxs, ws
