#!/usr/bin/env python3
"""Throughput of the routed MXFP4 MoE block on one MI355X (gfx950).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--route-profile]
                    [--route-locality]

A step is one pass of the whole block over one batch of seeded synthetic
input (weights and activations resident in HBM before timing):
  suite   (default) decode as the headline line, with prefill, stack, ds4,
          ds4_q4, ds4_selbias and ds4_hash measured after it and nested under
          "workloads"
  decode  gpt-oss-20b-shaped layer, 1000 tokens as T=1 calls
  prefill gpt-oss-20b-shaped layer, T=128, Zipf(1.1)-skewed expert loads
  stack   24 gpt-oss-20b-shaped layers (RMSNorm + MoE), T=512
  ds4     DeepSeek-V4-Flash-shaped layer, T=2048, 256 experts top-6 + shared
  ds4_q4  ds4 in the quantised expert-input mode (MX-FP4 expert input, FP4 x FP4
          gate/up products)
  ds4_q4a ds4 in quantised mode 2 (the SwiGLU output MX-FP4 too: FP4 x FP4 down)
  ds4_selbias  ds4 with the selection-only expert bias (exp_probs_b)
  ds4_hash     ds4 hash-routed by token id (tid2eid table over 129280 ids)
  ds4_pro DeepSeek-V4-Pro-shaped layer, T=2048, H=7168, F=3072, 384 experts top-6 + shared
  tiny    T=8, H=F=256, 8 experts top-2
  decode_stack  T=1 tokens through 24 gpt-oss-20b-shaped layers (RMSNorm + MoE),
          16 tokens per step, each layer's output the next layer's input
Each step's calls are captured once in a HIP graph and replayed; W warm-up
steps, then exactly K timed steps between two synchronisations (--steps and
--warmup set the headline workload's; nested workloads use their own step
counts). After the timed region, one more step is launched eagerly with the
library's moe_profile_next_launch hook armed on every call, so HIP events
stamped by the dominant kernel's own dispatches give its live average
duration for the roofline object; that step is not part of `value`. Expert
weights are held in several device copies, cycled between calls, so that the
256 MB Infinity Cache cannot serve them from one call to the next.

With --route-profile every call also adds its expert selections to a
[layers][E] uint64 table on the device (the route profile of the library's
route_out), so the timed steps include that recording. With --route-locality
(T=1 workloads) one more step runs after the timed region, eagerly, with each
call exporting its selections and route weights; the library's
moe_route_locality then reports that trace's adjacent-token overlap and the hit
rates of simulated per-layer expert caches.

Prints one JSON line (rank 0, N=1 only).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE block tokens/s (decode T=1, prefill T=128/512) + % HBM/MFMA peak"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
FP8_PEAK_TFLOPS = 5000.0        # MI355X dense FP8 MFMA: the rate of the FP4 x FP8 scaled MFMA used
FP4_PEAK_TFLOPS = 10100.0       # MI355X dense FP4 MFMA: the FP4 x FP4 rate (quantised expert input)
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA: a bfloat16 expert input taken as it is
DTYPE = "fp4xfp8"               # MXFP4 weights x FP8-term activations, float32 accumulation

WORKLOADS = {
    "decode": dict(config=2, name="gptoss20b_decode_T1_1000tok", kernel="decode_gate_up", copies=8,
                   steps=100),
    "prefill": dict(config=3, name="gptoss20b_prefill_T128_zipf", kernel="gate_up_gemm", copies=4,
                    steps=200),
    "stack": dict(config=4, name="gptoss20b_stack24_T512", kernel="gate_up_gemm", copies=1,
                  steps=20),
    "ds4": dict(config=5, name="ds4flash_T2048_E256_top6_shared", kernel="gate_up_gemm", copies=2,
                steps=50),
    # the same layer with the expert input rounded once to MX-FP4 (act_quant=1)
    "ds4_q4": dict(config=5, name="ds4flash_T2048_E256_top6_shared_mxfp4_input",
                   kernel="gate_up_gemm", copies=2, steps=50, act_quant=1),
    # and the SwiGLU output rounded to MX-FP4 too (act_quant=2)
    "ds4_q4a": dict(config=5, name="ds4flash_T2048_E256_top6_shared_mxfp4_input_and_act",
                    kernel="gate_up_gemm", copies=2, steps=50, act_quant=2),
    # DeepSeek-V4 routing variants on the same layer shape
    "ds4_selbias": dict(config=7, name="ds4flash_T2048_E256_top6_shared_selbias",
                        kernel="gate_up_gemm", copies=2, steps=50),
    "ds4_hash": dict(config=8, name="ds4flash_T2048_E256_top6_shared_hash129280",
                     kernel="gate_up_gemm", copies=2, steps=50),
    "tiny": dict(config=1, name="tiny_T8_H256_E8_top2", kernel="decode_gate_up", copies=1,
                 steps=200),
    # DeepSeek-V4-Pro-shaped layer (H=7168, F=3072, 384 experts top-6 + shared,
    # route scale 2.5), at the Flash workload's batch and recipe: 13.6 GB per copy
    "ds4_pro": dict(config=6, name="ds4pro_T2048_E384_top6_shared", kernel="gate_up_gemm",
                    copies=2, steps=20),
    # T=1 decode through the 24-layer stack's weights (RMSNorm + MoE per layer):
    # 16 independent tokens per step, each through all 24 layers in turn
    "decode_stack": dict(config=4, name="gptoss20b_decode_stack24_T1_16tok",
                         kernel="decode_gate_up", copies=1, steps=10, tokens=16),
}
KERNEL_SOURCES = {"decode_gate_up": "decode.hip", "decode_down": "decode.hip",
                  "gate_up_gemm": "prefill.hip", "down_gemm": "prefill.hip"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """Raw hipEvent_t handles from the HIP runtime the process already loaded."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so.7")
        self.lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.made = []

    def create(self) -> int:
        e = ctypes.c_void_p()
        rc = self.lib.hipEventCreateWithFlags(ctypes.byref(e), 0)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        self.made.append(e.value)
        return e.value

    def record(self, ev: int, stream: int):
        rc = self.lib.hipEventRecord(ctypes.c_void_p(ev), ctypes.c_void_p(stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_ms(self, a: int, b: int) -> float:
        f = ctypes.c_float()
        rc = self.lib.hipEventElapsedTime(ctypes.byref(f), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return f.value

    def destroy_all(self):
        for e in self.made:
            self.lib.hipEventDestroy(ctypes.c_void_p(e))
        self.made = []


def pad128(n: int) -> int:
    return (n + 127) // 128 * 128


def source_sha(kernel: str) -> str:
    h = hashlib.sha256()
    for f in ("common.hpp", "kernels.hpp", "mx_mfma.hpp", KERNEL_SOURCES[kernel]):
        with open(os.path.join(ROOT, "mxfp4_expert_ffn_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profile(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}__{workload}__pmc.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for ln in f:
            if ":" in ln and not ln.startswith("#"):
                k, v = ln.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_sha") != source_sha(kernel):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ---------------------------------------------------------------- workloads
class Setup:
    """Device-resident inputs and the per-step call lists of one workload."""

    def __init__(self, wl: str, copies: int | None):
        import numpy as np
        import torch

        import mxfp4_expert_ffn_amd as mx
        from mxfp4_expert_ffn_amd.device import upload_layer, workspace
        from workloads import config_by_id, make_layer, make_token_ids
        from workloads.gen import make_activations

        spec = WORKLOADS[wl]
        self.wl, self.spec = wl, spec
        self.cfg = cfg = config_by_id(spec["config"])
        self.copies = spec["copies"] if copies is None else copies
        self.mx = mx
        t0 = time.time()
        x, xb = make_activations(cfg)
        self.x_host = x
        self.token_ids = make_token_ids(cfg)   # hash-routed workloads only
        self.ids_dev = (None if self.token_ids is None
                        else torch.from_numpy(self.token_ids).cuda())
        n_layers = cfg.layers
        self.host_layers = []
        self.layers = []
        self.act_quant = spec.get("act_quant", 0)
        self.shape = mx.make_shape(**cfg.shape_kwargs(), act_quant=self.act_quant)
        for l in range(n_layers):
            layer = make_layer(cfg, l)
            self.layers.append(upload_layer(self.shape, layer, copies=self.copies))
            if l == 0:
                self.host_layers.append(layer)
            del layer
        log(f"[bench] {wl}: generated and uploaded {n_layers} layer(s) x {self.copies} "
            f"cop{'y' if self.copies == 1 else 'ies'} in {time.time() - t0:.1f}s")
        if cfg.act_dtype == "bf16":
            self.xd = torch.from_numpy(xb.view(np.int16).copy()).cuda()
        else:
            self.xd = torch.from_numpy(x).cuda()
        self.ws = workspace(self.shape)
        self.profile = None  # [layers][E] int64 route profile table, when recording
        self.trace = None    # (idx, w) [positions, layers, k] device tensors, when tracing
        self.tokens_per_step = cfg.T * cfg.calls
        # "calls": independent T=1 decode calls; "decode_stack": T=1 tokens
        # through every layer; "decode": one decode call; "prefill"
        if "tokens" in spec:
            self.mode = "decode_stack"
        elif cfg.path == "decode":
            self.mode = "calls" if cfg.T == 1 else "decode"
        else:
            self.mode = "prefill"
        if self.mode == "decode_stack":
            self.ntok = spec["tokens"]
            self.tokens_per_step = self.ntok
            self.step_shape = mx.make_shape(**cfg.shape_kwargs(1))
            self.ws = workspace(self.step_shape)
            self.out = torch.empty((self.ntok, 2, cfg.H), dtype=torch.float32, device="cuda")
            self.xrows = [self.xd[i:i + 1] for i in range(self.ntok)]
        elif self.mode == "calls":
            # one step = cfg.calls independent T=1 calls
            self.step_shape = mx.make_shape(**cfg.shape_kwargs(1))
            self.ws = workspace(self.step_shape)
            self.out = torch.empty((cfg.calls, cfg.H), dtype=torch.float32, device="cuda")
            self.xrows = [self.xd[i:i + 1] for i in range(cfg.calls)]
            self.orows = [self.out[i:i + 1] for i in range(cfg.calls)]
        else:
            self.step_shape = self.shape
            self.out = torch.empty((cfg.T, cfg.H), dtype=torch.float32, device="cuda")
            self.out2 = torch.empty_like(self.out)

    def _ro(self, layer: int, pos: int = 0):
        ro = {}
        if self.profile is not None:
            ro["route_counts"] = self.profile[layer]
        if self.trace is not None:
            ro["topk_idx"] = self.trace[0][pos, layer:layer + 1]
            ro["topk_w"] = self.trace[1][pos, layer:layer + 1]
        return ro or None

    def step_calls(self, step: int):
        """Closures making up one step (weights copy chosen per call/step)."""
        mx, cfg = self.mx, self.cfg
        calls = []
        if self.mode == "decode_stack":
            for i in range(self.ntok):
                src = self.xrows[i]
                for l, dl in enumerate(self.layers):
                    dst = self.out[i, l % 2].view(1, cfg.H)
                    calls.append(lambda dl=dl, src=src, dst=dst, l=l, i=i: mx.moe_forward_decode(
                        self.step_shape, src, dl.router_w, dl.router_b, dl.experts_copy(0), dst,
                        self.ws, norm_w=dl.norm_w, route_out=self._ro(l, i)))
                    src = dst
        elif self.mode == "calls":
            dl = self.layers[0]
            for i in range(cfg.calls):
                ex = dl.experts_copy(i)
                calls.append(lambda i=i, ex=ex: mx.moe_forward_decode(
                    self.step_shape, self.xrows[i], dl.router_w, dl.router_b, ex, self.orows[i],
                    self.ws, route_out=self._ro(0, i)))
        elif self.mode == "decode":
            dl = self.layers[0]
            calls.append(lambda: mx.moe_forward_decode(
                self.shape, self.xd, dl.router_w, dl.router_b, dl.experts_copy(step), self.out,
                self.ws, norm_w=dl.norm_w, shared=dl.shared_copy(step), route_out=self._ro(0)))
        else:
            src = self.xd
            bufs = (self.out, self.out2)
            for l, dl in enumerate(self.layers):
                dst = bufs[l % 2]
                calls.append(lambda dl=dl, src=src, dst=dst, l=l: mx.moe_forward_prefill(
                    self.shape, src, dl.router_w, dl.router_b, dl.experts_copy(step), dst,
                    self.ws, norm_w=dl.norm_w, shared=dl.shared_copy(step), route_out=self._ro(l),
                    routing=dl.routing(self.ids_dev)))
                src = dst
        return calls

    # algorithmic work of the dominant kernel per launch and of the block per step:
    # the expert weights it must read (codes + scales + biases) of every distinct
    # expert a call selects, once, plus its activation operands in and out in the
    # formats it uses (FP8 terms: 4 codes + 4 scale bytes per 32 values)
    def algorithmic(self, counts_per_call):
        cfg = self.cfg
        H, F, k, E = cfg.H, cfg.F, cfg.k, cfg.E
        mat = F * H * 17 // 32            # codes + scales of one [F,H] matrix
        terms = lambda n: 4 * pad128(n) + 4 * pad128(n) // 32
        if self.spec["kernel"] == "decode_gate_up":
            T = 1 if self.mode in ("calls", "decode_stack") else cfg.T
            routes = T * k + T * cfg.n_shared
            # T=1: the k selections are distinct experts; batches count them
            distinct = ([sum(1 for c in counts if c > 0) for counts in counts_per_call]
                        if counts_per_call else [T * k])
            active = sum(distinct) / len(distinct) + cfg.n_shared
            splits = (H + 511) // 512    # the router's split-K partials (512-wide slices)
            byts = active * 2 * (mat + 4 * F) + T * terms(H) + routes * terms(F) + T * splits * E * 8
            return dict(bytes=byts, flops=routes * 4 * H * F, units=routes,
                        unit="route (token, selected expert)", active_experts=active)
        # gate/up GEMM: weights of every active expert once, the expert input
        # once (its FP8 terms that take part, the bfloat16 rows themselves, or
        # the MX-FP4 codes + scales), the SwiGLU output's three FP8 terms (or
        # its MX-FP4 codes) out
        T = cfg.T
        active = [sum(1 for c in counts if c > 0) + cfg.n_shared for counts in counts_per_call]
        rows = T * k + T * cfg.n_shared
        xt = self.gate_up_x_terms()
        if self.act_quant:
            x_in = T * pad128(H) * 17 // 32
        elif xt == 1:
            x_in = T * H * 2
        else:
            x_in = T * terms(H) * xt // 4
        act_out = rows * pad128(F) * 17 // 32 if self.act_quant == 2 else rows * terms(F) * 3 // 4
        per = [a * 2 * (mat + 4 * F) + x_in + act_out for a in active]
        return dict(bytes=sum(per) / len(per), flops=4.0 * rows * H * F, units=rows,
                    unit="routed row (token, expert) of the grouped GEMM",
                    active_experts=sum(active) / len(active))

    def gate_up_x_terms(self):
        """The library's operand choice for the expert input of the gate/up
        GEMM: FP8 terms (3 or 4), 1 (the bfloat16 input itself) or 0 (MX-FP4)."""
        cfg = self.cfg
        return self.mx.moe_prefill_plan(self.shape, with_norm=cfg.rms_eps is not None)["x_terms"]

    def issued_flops(self, counts_per_call):
        """Matrix-core flops the dominant kernel issues per launch, from its
        structure: every 16x16x128 block-scaled instruction counts
        2 * 16 * 16 * 128 flops, the zero columns, padded rows and FP8 terms
        included."""
        cfg = self.cfg
        H, F, k = cfg.H, cfg.F, cfg.k
        per_mfma = 2 * 16 * 16 * 128
        if self.spec["kernel"] == "decode_gate_up":
            # per route: F/32 items x 8 wavefronts x their K-steps x 4 tiles;
            # a wavefront runs rounds of spw steps (steps past K run with a
            # zero operand but still issue)
            T = 1 if self.mode in ("calls", "decode_stack") else cfg.T
            routes = T * k + T * cfg.n_shared
            ns = pad128(H) // 128
            spw = min(4, max(1, -(-ns // 8)))
            steps = sum(spw for w in range(8) for s0 in range(w * spw, ns, 8 * spw))
            return routes * (F // 32) * steps * 4 * per_mfma
        # gate/up GEMM (the library's plan for this shape): per 16-row group of
        # an expert's rows, every gate and up weight tile of every feature block
        # of a work item, every 128-wide K-step, every FP8 term used (one
        # instruction for the MX-FP4 input, x_terms 0; four 16x16x32 bf16
        # instructions, the same flops, for the bfloat16 input, x_terms 1)
        plan = self.mx.moe_prefill_plan(self.shape, with_norm=cfg.rms_eps is not None)
        nt, fwg = plan["x_terms"] or 1, plan["gate_up_features"]
        tiles = -(-pad128(F) // fwg) * (2 * fwg // 16)
        tot = []
        for counts in counts_per_call:
            groups = sum(-(-c // 16) for c in counts)
            if cfg.n_shared:
                groups += -(-cfg.T // 16)
            tot.append(groups * tiles * (pad128(H) // 128) * nt * per_mfma)
        return sum(tot) / len(tot)

    def block_bytes_per_step(self, counts_per_call):
        cfg = self.cfg
        H, F, k = cfg.H, cfg.F, cfg.k
        expert = 3 * F * H * 17 // 32 + 4 * (2 * F + H)
        if self.mode == "calls":
            return cfg.calls * k * expert
        if self.mode == "decode_stack":
            return self.ntok * cfg.layers * k * expert
        tot = 0
        for counts in counts_per_call:
            tot += (sum(1 for c in counts if c > 0) + cfg.n_shared) * expert
        return tot


def route_counts(setup):
    """Per-call expert histograms of one step (for algorithmic byte counts):
    every layer of a prefill workload, or the one call of a batched decode."""
    import torch
    mx, cfg = setup.mx, setup.cfg
    res = []
    if setup.mode == "decode":
        dl = setup.layers[0]
        counts = torch.empty(cfg.E, dtype=torch.int32, device="cuda")
        mx.moe_forward_decode(setup.shape, setup.xd, dl.router_w, dl.router_b, dl.experts_copy(0),
                              setup.out, setup.ws, norm_w=dl.norm_w, shared=dl.shared_copy(0),
                              route_out={"counts": counts})
        torch.cuda.synchronize()
        return [counts.cpu().tolist()]
    if setup.mode != "prefill":
        return res
    src = setup.xd
    bufs = (setup.out, setup.out2)
    for l, dl in enumerate(setup.layers):
        counts = torch.empty(cfg.E, dtype=torch.int32, device="cuda")
        dst = bufs[l % 2]
        mx.moe_forward_prefill(setup.shape, src, dl.router_w, dl.router_b, dl.experts_copy(0), dst,
                               setup.ws, norm_w=dl.norm_w, shared=dl.shared_copy(0),
                               route_out={"counts": counts}, routing=dl.routing(setup.ids_dev))
        torch.cuda.synchronize()
        res.append(counts.cpu().tolist())
        src = dst
    return res


def capture(calls):
    """Capture one step's calls into a HIP graph."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c in calls:
            c()
    return g


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline_full(setup, budget_s: float) -> dict:
    """cpu_baseline with the host's CPU model and, for the single-layer
    gpt-oss workloads, the same oracle with its BLAS held to one thread (on
    half the budget)."""
    r = cpu_baseline(setup, budget_s)
    r["cpu_model"] = cpu_model()
    r["host_cpus"] = len(os.sched_getaffinity(0))
    if setup.cfg.config_id in (1, 2, 3):
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1, user_api="blas"):
            r1 = cpu_baseline(setup, budget_s / 2)
        r["one_thread"] = {"value": r1["value"], "sample": r1["sample"]}
    return r


def cpu_baseline(setup, budget_s: float):
    """The oracle, as it stands, on a bounded sample of the same workload.

    One unit of work is an oracle call of the workload's own shape: a T=1 call
    per token for the decode workloads, the batched call for the others. Units
    run until at least half the budget has gone, so the sample takes between
    budget / 2 and budget / 2 plus one unit. The host keeps layer 0 only: for a
    layer stack the rate is layer 0's divided by the layer count."""
    import numpy as np
    from oracle import moe as omoe
    cfg = setup.cfg
    layer = setup.host_layers[0]
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()
                     if p.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        cores = 1
    x = setup.x_host
    layers = cfg.layers

    def run_units(unit, tokens_per_unit):
        n_units, t0 = 0, time.time()
        while True:
            unit(n_units)
            n_units += 1
            dt = time.time() - t0
            if dt >= budget_s / 2:
                return n_units * tokens_per_unit, dt, n_units

    if setup.mode in ("calls", "decode_stack"):
        ntok = setup.ntok if setup.mode == "decode_stack" else cfg.calls
        n, dt, _ = run_units(lambda i: omoe.block_for_config(cfg, layer, x[i % ntok:i % ntok + 1]), 1)
        what = "RMSNorm + MoE " if layer.norm_w is not None else ""
        scaled = f", divided by {layers} layers" if layers > 1 else ""
        return dict(value=n / dt / layers, unit="tokens/s", cores=cores, kind="oracle",
                    sample=f"{n} T=1 fp64 oracle calls ({what}layer 0), one per decode token, "
                           f"in {dt:.1f} s{scaled}")
    # prefill-type: all T tokens of the first layer if the budget allows, else
    # the first n tokens. The oracle's time goes into dequantising each expert
    # the sample touches (about 0.08 s per expert at H*F = 4096*2048, measured
    # on the GPU host, scaled by the expert's size), so n is the largest count
    # whose expected number of distinct experts, E(1 - (1 - k/E)^n) plus the
    # shared one, fits the budget
    per_expert = 0.08 * cfg.H * cfg.F / (4096 * 2048)

    def experts_touched(m):
        return cfg.E * (1.0 - (1.0 - cfg.k / cfg.E) ** m) + cfg.n_shared

    n = cfg.T
    while n > 1 and experts_touched(n) * per_expert > budget_s:
        n = int(n * 0.9)
    toks = np.arange(n)
    ids = None if setup.token_ids is None else setup.token_ids[:cfg.T]
    done, dt, calls = run_units(lambda i: omoe.block_for_config(cfg, layer, x[:cfg.T], tokens=toks,
                                                                act_quant=setup.act_quant,
                                                                token_ids=ids), n)
    scaled = f", divided by {layers} layers" if layers > 1 else ""
    mode = ", MX-FP4 expert input" if setup.act_quant else ""
    return dict(value=done / dt / layers, unit="tokens/s", cores=cores, kind="oracle",
                sample=f"{calls} fp64 oracle call(s) of layer 0, each on {n} of {cfg.T} tokens "
                       f"(routing for all {cfg.T}){mode}, in {dt:.1f} s{scaled}")


def route_locality(setup) -> dict:
    """One untimed step with every call exporting its selections and route
    weights: the decode trace's locality, from the library's host profiler."""
    import torch
    mx, cfg = setup.mx, setup.cfg
    P = setup.ntok if setup.mode == "decode_stack" else cfg.calls
    L = len(setup.layers)
    setup.trace = (torch.full((P, L, cfg.k), -1, dtype=torch.int32, device="cuda"),
                   torch.zeros((P, L, cfg.k), dtype=torch.float32, device="cuda"))
    for c in setup.step_calls(0):
        c()
    torch.cuda.synchronize()
    idx, w = (t.cpu().numpy() for t in setup.trace)
    setup.trace = None
    r = mx.moe_route_locality(idx, w, cfg.E)
    sel = int(r["hist"].sum())
    tw = float(r["weight_hist"].sum())
    pairs = int(r["adjacent_pairs"].sum())
    order = mx.moe_route_hotlist(r["hist"], r["weight_hist"])
    return {
        "positions": P, "layers": L, "k": cfg.k, "selections": sel,
        "cache_sizes": r["caps"].tolist(),
        "hit_rate": [round(int(h) / sel, 6) for h in r["cache_hits"].sum(axis=1)],
        "weighted_hit_rate": [round(float(h) / tw, 6) for h in r["cache_weight_hits"].sum(axis=1)],
        "mean_adjacent_overlap": round(float(r["overlap_sum"].sum()) / pairs, 6) if pairs else 0.0,
        "mean_adjacent_jaccard": round(float(r["jaccard_sum"].sum()) / pairs, 6) if pairs else 0.0,
        "hottest": [[int(i) // cfg.E, int(i) % cfg.E, int(r["hist"].flat[i])] for i in order[:4]],
    }


# the default run: the decode headline, then these workloads nested under
# "workloads" (each with its own step count)
SUITE = (("prefill", "prefill_T128"), ("stack", "stack_T512"), ("ds4", "ds4"), ("ds4_q4", "ds4_q4"),
         ("ds4_q4a", "ds4_q4a"), ("ds4_selbias", "ds4_selbias"), ("ds4_hash", "ds4_hash"))


def measure(wl: str, args, steps: int, warmup: int) -> dict:
    """Time one workload: K graph-replayed steps, then one instrumented eager
    step for the dominant kernel's own duration. Frees its device memory."""
    import torch

    setup = Setup(wl, args.copies)
    spec, cfg, mx = setup.spec, setup.cfg, setup.mx
    ev = HipEvents()
    stream = torch.cuda.current_stream().cuda_stream

    counts = route_counts(setup)
    if args.route_profile:
        setup.profile = torch.zeros((cfg.layers, cfg.E), dtype=torch.int64, device="cuda")
    ncopies_graph = 1 if setup.mode in ("calls", "decode_stack") else setup.copies
    plain = [setup.step_calls(c) for c in range(ncopies_graph)]
    for calls in plain:          # eager run once (validates arguments, warms code objects)
        for c in calls:
            c()
    torch.cuda.synchronize()

    kernel = spec["kernel"]
    inst_calls = setup.step_calls(steps % ncopies_graph)
    pairs = [(ev.create(), ev.create()) for _ in inst_calls]
    graphs = None if args.no_graph else [capture(calls) for calls in plain]
    torch.cuda.synchronize()

    def run_step(s):
        if graphs is None:
            for c in plain[s % ncopies_graph]:
                c()
        else:
            graphs[s % ncopies_graph].replay()

    for s in range(warmup):
        run_step(s)
    torch.cuda.synchronize()
    t_start, t_stop = ev.create(), ev.create()
    torch.cuda.synchronize()
    ev.record(t_start, stream)
    for s in range(steps):
        run_step(s)
    ev.record(t_stop, stream)
    torch.cuda.synchronize()
    total_ms = ev.elapsed_ms(t_start, t_stop)
    # outside the timed region: the dominant kernel's own duration, from HIP
    # events its dispatches stamp (eager, the hook armed on every call). A few
    # untimed replays go first, without a synchronisation, so the instrumented
    # calls queue behind them and run back to back on a busy GPU, as the timed
    # steps do, rather than one by one behind the host
    for s in range(3):
        run_step(steps + s)
    for i, c in enumerate(inst_calls):
        mx.moe_profile_next_launch(kernel, pairs[i][0], pairs[i][1])
        c()
    torch.cuda.synchronize()
    kern_ms = [ev.elapsed_ms(a, b) for a, b in pairs]
    kern_avg_ms = sum(kern_ms) / len(kern_ms)
    ms_per_step = total_ms / steps
    value = setup.tokens_per_step * steps / (total_ms / 1e3)
    alg = setup.algorithmic(counts)
    issued = setup.issued_flops(counts)
    kern_s = kern_avg_ms / 1e3
    traffic = traffic_from_profile(kernel, wl)
    # the matrix-core peak of the instruction the kernel issues: FP4 x FP8
    # (the FP8 rate), FP4 x FP4 with the MX-FP4 expert input, or bf16 x bf16
    # when the gate/up GEMM takes a bfloat16 input as it is
    if setup.act_quant:
        mfma_peak, mfma_dtype = FP4_PEAK_TFLOPS, "fp4 (fp4 x fp4 scaled MFMA)"
    elif kernel == "gate_up_gemm" and setup.gate_up_x_terms() == 1:
        mfma_peak, mfma_dtype = BF16_PEAK_TFLOPS, "bf16 (weights decoded to bf16 in registers x bf16 input)"
    else:
        mfma_peak, mfma_dtype = FP8_PEAK_TFLOPS, "fp8 (fp4 x fp8 scaled MFMA)"
    t_hbm = alg["bytes"] / (HBM_PEAK_GBPS * 1e9)
    t_mfma = alg["flops"] / (mfma_peak * 1e12)
    if kernel.startswith("decode") or t_hbm >= t_mfma:
        achieved, peak, unit, bound = alg["bytes"] / kern_s / 1e9, HBM_PEAK_GBPS, "GB/s", "hbm"
    else:
        achieved, peak, unit, bound = alg["flops"] / kern_s / 1e12, mfma_peak, "TFLOP/s", "mfma"
    # how the gate/up GEMM takes the expert input (decode: four FP8 terms)
    xt = setup.gate_up_x_terms() if setup.mode == "prefill" else None
    if setup.act_quant:
        expert_input = "mxfp4 (rounded once)"
    elif xt == 1:
        expert_input = "exact (bf16 as it is; weights decoded to bf16 in registers)"
    else:
        expert_input = "exact (fp8 terms)"
    # the arithmetic the path computes in: MXFP4 weights against FP8 terms,
    # the bfloat16 input (weights decoded to bf16), or MX-FP4 activations
    gate_dt = {1: "bf16", 0: "fp4xfp4"}.get(xt, DTYPE) if setup.mode == "prefill" else DTYPE
    down_dt = "fp4xfp4" if setup.act_quant == 2 else DTYPE
    dtype = gate_dt if gate_dt == down_dt else f"{gate_dt} (gate/up), {down_dt} (down)"
    block_bytes = setup.block_bytes_per_step(counts)
    block_gbps = block_bytes / (ms_per_step / 1e3) / 1e9
    nominal_tf = alg["flops"] / kern_s / 1e12
    issued_tf = issued / kern_s / 1e12

    result = {
        "value": round(value, 1),
        "unit": "tokens/s",
        "dtype": dtype,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 4),
        "config": {
            "workload": spec["name"], "T": int(setup.step_shape.T), "H": cfg.H, "F": cfg.F, "E": cfg.E,
            "k": cfg.k, "n_shared": cfg.n_shared, "layers": cfg.layers,
            "tokens_per_step": setup.tokens_per_step, "weights": "mxfp4 (e2m1 + e8m0/32) + fp32 bias",
            "activations": cfg.act_dtype, "weight_copies": setup.copies,
            "expert_input": expert_input,
            "swiglu_output": "mxfp4" if setup.act_quant == 2 else "exact (fp8 terms)",
            "launch": "eager" if graphs is None else "hip_graph",
            "route_profile": args.route_profile,
        },
        "roofline": {
            "kernel": kernel, "bound": bound, "achieved": round(achieved, 2), "peak": peak,
            "unit": unit, "frac": round(achieved / peak, 4),
            "traffic": traffic,
            "avg_launch_us": round(kern_avg_ms * 1e3, 3),
            "algorithmic_bytes_per_launch": int(alg["bytes"]),
            "algorithmic_flops_per_launch": int(alg["flops"]),
            "units_per_launch": alg["units"], "unit_of_work": alg["unit"],
            "active_experts_per_launch": round(alg["active_experts"], 2),
            # matrix-core view of the same launch: nominal = the block's own
            # 4*H*F (gate/up) flops per unit; issued = every instruction the
            # kernel runs (FP8 terms, zero columns, padded rows)
            "mfma": {
                "peak_TFLOPs": mfma_peak, "peak_dtype": mfma_dtype,
                "nominal_TFLOPs": round(nominal_tf, 2),
                "nominal_frac": round(nominal_tf / mfma_peak, 4),
                "issued_flops_per_launch": int(issued),
                "issued_TFLOPs": round(issued_tf, 2),
                "issued_frac": round(issued_tf / mfma_peak, 4),
            },
        },
        "block": {
            "expert_bytes_per_step": int(block_bytes),
            "achieved_GBps": round(block_gbps, 1),
            "frac_of_hbm_peak": round(block_gbps / HBM_PEAK_GBPS, 4),
        },
    }
    if setup.profile is not None:
        # every executed step recorded T*k selections per layer: the eager
        # validation pass(es), the warm-up, the timed steps, the three replays
        # and the instrumented step after them
        runs = ncopies_graph + warmup + steps + 3 + 1
        summ = mx.moe_route_profile_summary(setup.profile.cpu().numpy())
        summ["selections_expected"] = runs * setup.tokens_per_step * cfg.k * cfg.layers
        del summ["layer_unique"]
        result["route_profile"] = summ
    if args.route_locality:
        result["route_locality"] = route_locality(setup)
    ev.destroy_all()
    if not args.no_cpu_baseline:
        log(f"[bench] {wl}: timing the CPU oracle baseline")
        result["cpu_baseline"] = cpu_baseline_full(setup, args.cpu_budget)
    else:
        result["cpu_baseline"] = None
    del graphs, plain, inst_calls, setup
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    log(f"[bench] {wl}: {result['value']:.1f} tokens/s, {kernel} {result['roofline']['frac']:.3f} "
        f"of {bound} peak")
    return result


def calibrate(result: dict, gib: float):
    import torch
    n = int(gib * (1 << 30)) // 4
    a = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    result["calibration_copy_bytes"] = 2 * 4 * n
    # the copy's own rate (read + write bytes over its best of five runs):
    # what a plain streaming kernel sustains on this GPU
    best = None
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    result["calibration_copy_GBps"] = round(2 * 4 * n / (best / 1e3) / 1e9, 1)
    best = None  # a read-only stream: torch's sum over the same buffer
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        a.sum()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    result["calibration_read_GBps"] = round(4 * n / (best / 1e3) / 1e9, 1)
    del a, b


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default per workload)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", choices=["suite"] + sorted(WORKLOADS), default="suite")
    ap.add_argument("--copies", type=int, default=None, help="device copies of the expert weights")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of HIP graphs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds for the oracle sample")
    ap.add_argument("--route-profile", action="store_true",
                    help="record every call's expert selections into a device route profile")
    ap.add_argument("--route-locality", action="store_true",
                    help="after timing, one untimed step recording its decode trace, and the "
                         "trace's expert locality (T=1 workloads)")
    ap.add_argument("--calibrate-copy-gib", type=float, default=0.0,
                    help="also run one device copy of this many GiB (PMC byte calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    head = "decode" if args.workload == "suite" else args.workload
    if args.steps is None:
        args.steps = WORKLOADS[head]["steps"]
    if args.steps < 1:
        sys.exit("--steps must be >= 1")
    if args.route_locality and head not in ("decode", "decode_stack"):
        sys.exit("--route-locality needs a T=1 workload (decode, decode_stack)")
    if args.workload == "suite" and args.copies is not None:
        sys.exit("--copies applies to a single --workload")

    import torch
    import mxfp4_expert_ffn_amd as mx
    if not torch.cuda.is_available():
        sys.exit("no GPU visible")
    mx._lib.load()
    torch.cuda.set_device(0)

    r = measure(head, args, args.steps, args.warmup)
    result = {
        "metric": METRIC, "value": r.pop("value"), "unit": r.pop("unit"), "n_gpus": 1,
        "steps": r.pop("steps"), "warmup": r.pop("warmup"), "ms_per_step": r.pop("ms_per_step"),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": r.pop("dtype"),
        "data": "synthetic",
    }
    result.update(r)
    if args.workload == "suite":
        args.route_locality = False
        result["workloads"] = {}
        for wl, key in SUITE:
            result["workloads"][key] = measure(wl, args, WORKLOADS[wl]["steps"], args.warmup)
    if args.calibrate_copy_gib > 0:
        calibrate(result, args.calibrate_copy_gib)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
