"""Seeded synthetic inputs for the routed MoE block.

Recipe (identical for the oracle and the GPU harness):
- seed = 20261202 + config_id; every stream is a PCG64 generator keyed by
  (seed, stream, layer), streams 0 router, 1 experts, 2 activations, 3 norm.
- MXFP4 expert weights: code bytes uniform over 0..255 (two uniform 4-bit
  codes per byte), E8M0 scale bytes uniform over 123..127 (2^-4 .. 2^0),
  fp32 biases ~ N(0, 0.02).
- Router [E, H] fp32 with fp32 bias [E]:
    "normal":  W ~ N(0, w_std^2), b ~ N(0, b_std^2)
    "zipf":    W ~ N(0, (1.5/sqrt(H))^2), b_e = ln p_pi(e) with p_r ~ r^-s
               (r = 1..E, pi a seeded permutation), giving Zipf-like loads
    "uniform": W ~ U(-sqrt(3/H), sqrt(3/H)), b = 0 (near-balanced loads)
- Activations x ~ N(0, 1); for bf16 workloads x is drawn in fp32 and rounded
  to bf16 (nearest, ties to even); `x` then holds the exact widening.
- RMSNorm weight gamma ~ 1 + N(0, 0.1) when the workload has a norm.
- Routing variants (stream 4): selection-only bias [E] ~ N(0, sel_bias_std^2)
  in fp32; hash table tid2eid [vocab, k] int32, each row k distinct experts
  drawn uniformly without replacement. Token ids (stream 5) uniform over
  the vocabulary, one per activation row.

Arrays use the planar MXFP4 form: codes [E, rows, K/2] (element 2i in the low
nibble of byte i), scale bytes [E, rows, K/32], biases [E, rows].
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .configs import MoeConfig

BASE_SEED = 20261202
STREAM_ROUTER, STREAM_EXPERTS, STREAM_ACT, STREAM_NORM = 0, 1, 2, 3
STREAM_ROUTING, STREAM_TOKENS = 4, 5


def rng_for(config_id: int, stream: int, layer: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence(entropy=BASE_SEED + config_id, spawn_key=(stream, layer))
    return np.random.Generator(np.random.PCG64(ss))


@dataclass
class ExpertPlanes:
    """MXFP4 planes of n experts (gate/up: [n, F, H], down: [n, H, F])."""
    gate_codes: np.ndarray
    gate_scales: np.ndarray
    gate_bias: np.ndarray
    up_codes: np.ndarray
    up_scales: np.ndarray
    up_bias: np.ndarray
    down_codes: np.ndarray
    down_scales: np.ndarray
    down_bias: np.ndarray

    @property
    def n(self) -> int:
        return self.gate_codes.shape[0]

    def select(self, e: int) -> "ExpertPlanes":
        return ExpertPlanes(*[getattr(self, f)[e:e + 1] for f in PLANE_FIELDS])


PLANE_FIELDS = ("gate_codes", "gate_scales", "gate_bias", "up_codes", "up_scales",
                "up_bias", "down_codes", "down_scales", "down_bias")


@dataclass
class Layer:
    router_w: np.ndarray          # [E, H] f32
    router_b: np.ndarray          # [E] f32
    experts: ExpertPlanes
    shared: ExpertPlanes | None = None
    norm_w: np.ndarray | None = None  # [H] f32
    sel_bias: np.ndarray | None = None  # [E] f32 selection-only expert bias
    tid2eid: np.ndarray | None = None   # [vocab, k] int32 hash-routing table


@dataclass
class Workload:
    cfg: MoeConfig
    x: np.ndarray                 # [calls*T, H] f32 (exact values of the input)
    x_bf16: np.ndarray | None     # [calls*T, H] uint16 bf16 bits, bf16 workloads only
    layers: list = field(default_factory=list)


def _random_planes(rng: np.random.Generator, n: int, H: int, F: int) -> ExpertPlanes:
    def codes(rows, K):
        return np.frombuffer(rng.bytes(n * rows * K // 2), dtype=np.uint8).reshape(n, rows, K // 2)

    def scales(rows, K):
        return rng.integers(123, 128, size=(n, rows, K // 32), dtype=np.uint8)

    def bias(rows):
        return rng.normal(0.0, 0.02, size=(n, rows)).astype(np.float32)

    gc, gs, gb = codes(F, H), scales(F, H), bias(F)
    uc, us, ub = codes(F, H), scales(F, H), bias(F)
    dc, ds, db = codes(H, F), scales(H, F), bias(H)
    return ExpertPlanes(gc, gs, gb, uc, us, ub, dc, ds, db)


def _router(cfg: MoeConfig, rng: np.random.Generator):
    E, H = cfg.E, cfg.H
    if cfg.router == "normal":
        w = rng.normal(0.0, cfg.router_w_std, size=(E, H))
        b = rng.normal(0.0, cfg.router_b_std, size=E)
    elif cfg.router == "zipf":
        w = rng.normal(0.0, 1.5 / np.sqrt(H), size=(E, H))
        perm = rng.permutation(E)
        p = np.arange(1, E + 1, dtype=np.float64) ** (-cfg.zipf_s)
        p /= p.sum()
        b = np.log(p[perm])
    elif cfg.router == "uniform":
        a = np.sqrt(3.0 / H)
        w = rng.uniform(-a, a, size=(E, H))
        b = np.zeros(E)
    else:
        raise ValueError(cfg.router)
    return w.astype(np.float32), b.astype(np.float32)


def make_layer(cfg: MoeConfig, layer: int = 0) -> Layer:
    if cfg.H % 32 or cfg.F % 32:
        raise ValueError("H and F must be multiples of 32")
    rw, rb = _router(cfg, rng_for(cfg.config_id, STREAM_ROUTER, layer))
    erng = rng_for(cfg.config_id, STREAM_EXPERTS, layer)
    experts = _random_planes(erng, cfg.E, cfg.H, cfg.F)
    shared = _random_planes(erng, cfg.n_shared, cfg.H, cfg.F) if cfg.n_shared else None
    norm_w = None
    if cfg.rms_eps is not None:
        nrng = rng_for(cfg.config_id, STREAM_NORM, layer)
        norm_w = (1.0 + nrng.normal(0.0, 0.1, size=cfg.H)).astype(np.float32)
    sel_bias = tid2eid = None
    if cfg.sel_bias_std > 0 or cfg.hash_vocab > 0:
        rrng = rng_for(cfg.config_id, STREAM_ROUTING, layer)
        if cfg.sel_bias_std > 0:
            sel_bias = rrng.normal(0.0, cfg.sel_bias_std, size=cfg.E).astype(np.float32)
        if cfg.hash_vocab > 0:
            tid2eid = distinct_rows(rrng, cfg.hash_vocab, cfg.E, cfg.k)
    return Layer(rw, rb, experts, shared, norm_w, sel_bias, tid2eid)


def distinct_rows(rng: np.random.Generator, rows: int, n: int, k: int) -> np.ndarray:
    """[rows, k] int32: each row k distinct values of 0..n-1, uniformly without
    replacement (the j-th draw picks among the n - j values still free, then
    steps over the earlier picks in ascending order)."""
    out = np.empty((rows, k), dtype=np.int64)
    for j in range(k):
        c = rng.integers(0, n - j, size=rows)
        taken = np.sort(out[:, :j], axis=1)
        for i in range(j):
            c = c + (c >= taken[:, i])
        out[:, j] = c
    return out.astype(np.int32)


def make_token_ids(cfg: MoeConfig, rows: int | None = None) -> np.ndarray | None:
    """Token ids [rows] int32 for hash-routed workloads (None otherwise)."""
    if cfg.hash_vocab <= 0:
        return None
    rows = cfg.T * cfg.calls if rows is None else rows
    rng = rng_for(cfg.config_id, STREAM_TOKENS)
    return rng.integers(0, cfg.hash_vocab, size=rows).astype(np.int32)


def _round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    bits = x.astype(np.float32).view(np.uint32).astype(np.uint64)
    rounded = (bits + 0x7FFF + ((bits >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def make_activations(cfg: MoeConfig, rows: int | None = None):
    rows = cfg.T * cfg.calls if rows is None else rows
    rng = rng_for(cfg.config_id, STREAM_ACT)
    x = rng.normal(0.0, 1.0, size=(rows, cfg.H)).astype(np.float32)
    if cfg.act_dtype == "bf16":
        bits = _round_to_bf16_bits(x)
        return bf16_bits_to_f32(bits), bits
    return x, None


def make_workload(cfg: MoeConfig, layers: int | None = None) -> Workload:
    n_layers = cfg.layers if layers is None else layers
    x, xb = make_activations(cfg)
    return Workload(cfg, x, xb, [make_layer(cfg, l) for l in range(n_layers)])
