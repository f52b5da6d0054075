"""The workload configurations, as data: the five of the block, a sixth with
the DeepSeek-V4-Pro shape, and two DeepSeek-V4-Flash layers with the routing
variants (selection-only bias; hash routing).

Model constants come from the pages:
- gpt-oss-20b (goosedump 0.12.31 `src/engine/model/gpt_oss.rs`, constants block):
  H = F = 2880, 32 experts, top-4, SwiGLU alpha 1.702 and limit 7.0, RMSNorm
  eps 1e-5, 24 layers, prefill batch 128 with an expert-parallel threshold of
  4 x 128 rows.
- DeepSeek-V4-Flash (antirez `ds4.c`, `DS4_SHAPE_FLASH`): n_embd 4096,
  n_ff_exp 2048, 256 routed experts, 6 used, 1 shared expert, expert weight
  scale 1.5, SwiGLU clamp 10 (`DS4_DEFAULT_SWIGLU_CLAMP_EXP`).
- DeepSeek-V4 routing variants (`ds4_layer_weights`, `weights_validate_layout`,
  `DS4_SHAPE_FLASH`): the optional selection-only bias exp_probs_b [n_expert]
  and, for the first n_hash_layer = 3 layers, the tid2eid table of
  n_expert_used experts per token id over n_vocab = 129280 ids.
- DeepSeek-V4-Pro (`DS4_SHAPE_PRO`): n_embd 7168, n_ff_exp 3072, 384 routed
  experts, 6 used, 1 shared, expert weight scale 2.5, the same default clamp.
  Everything the page leaves open (batch, router, activations, SwiGLU alpha
  and offset) follows the Flash workload.

Value distributions (codes, scales, biases, router, activations) are the
synthetic recipe of the workload list; see `gen.py`.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass


@dataclass(frozen=True)
class MoeConfig:
    config_id: int
    name: str
    T: int                 # tokens per block call
    H: int                 # hidden size
    F: int                 # expert hidden size
    E: int                 # routed experts
    k: int                 # experts used per token
    alpha: float = 1.702   # SwiGLU gate slope
    limit: float = 7.0     # SwiGLU clamp
    up_offset: float = 1.0  # added to the clamped up projection
    route_scale: float = 1.0
    n_shared: int = 0
    act_dtype: str = "f32"  # "f32" or "bf16" hidden/residual
    layers: int = 1
    rms_eps: float | None = None  # RMSNorm before the router when set
    router: str = "normal"  # "normal" | "zipf" | "uniform"
    router_w_std: float = 0.05
    router_b_std: float = 0.05
    zipf_s: float = 1.1
    calls: int = 1          # independent block calls making up one pass
    path: str = "prefill"   # which entry point the workload exercises
    sel_bias_std: float = 0.0  # selection-only expert bias ~ N(0, std^2) when > 0
    hash_vocab: int = 0        # hash routing by token id over this vocabulary when > 0

    @property
    def R(self) -> int:
        return self.T * self.k

    def shape_kwargs(self, T: int | None = None) -> dict:
        """Keyword arguments describing one block call (T tokens) of this workload."""
        return dict(T=self.T if T is None else T, H=self.H, F=self.F, E=self.E, k=self.k,
                    act_dtype=self.act_dtype, n_shared=self.n_shared, alpha=self.alpha,
                    limit=self.limit, up_offset=self.up_offset, route_scale=self.route_scale,
                    rms_eps=self.rms_eps or 0.0)


CONFIGS = (
    MoeConfig(1, "tiny", T=8, H=256, F=256, E=8, k=2, router_b_std=0.05,
              path="decode"),
    MoeConfig(2, "gptoss_decode", T=1, H=2880, F=2880, E=32, k=4,
              router_b_std=0.5, calls=1000, path="decode"),
    MoeConfig(3, "gptoss_prefill", T=128, H=2880, F=2880, E=32, k=4,
              router="zipf", zipf_s=1.1),
    MoeConfig(4, "gptoss_stack24", T=512, H=2880, F=2880, E=32, k=4,
              router_b_std=0.5, layers=24, rms_eps=1e-5),
    MoeConfig(5, "ds4_flash", T=2048, H=4096, F=2048, E=256, k=6,
              alpha=1.0, limit=10.0, up_offset=0.0, route_scale=1.5,
              n_shared=1, act_dtype="bf16", router="uniform"),
    MoeConfig(6, "ds4_pro", T=2048, H=7168, F=3072, E=384, k=6,
              alpha=1.0, limit=10.0, up_offset=0.0, route_scale=2.5,
              n_shared=1, act_dtype="bf16", router="uniform"),
    # DeepSeek-V4-Flash layer with the selection-only expert bias (exp_probs_b)
    MoeConfig(7, "ds4_flash_selbias", T=2048, H=4096, F=2048, E=256, k=6,
              alpha=1.0, limit=10.0, up_offset=0.0, route_scale=1.5,
              n_shared=1, act_dtype="bf16", router="uniform", sel_bias_std=0.5),
    # DeepSeek-V4-Flash hash-routed layer (one of the first n_hash_layer = 3):
    # experts from the tid2eid table row of each token id, vocabulary 129280
    MoeConfig(8, "ds4_flash_hash", T=2048, H=4096, F=2048, E=256, k=6,
              alpha=1.0, limit=10.0, up_offset=0.0, route_scale=1.5,
              n_shared=1, act_dtype="bf16", router="uniform", hash_vocab=129280),
)


def config_by_id(config_id: int) -> MoeConfig:
    for c in CONFIGS:
        if c.config_id == config_id:
            return c
    raise KeyError(config_id)


def scaled(cfg: MoeConfig, **overrides) -> MoeConfig:
    """Same distributions and constants, other sizes (for small parity cases)."""
    return dataclasses.replace(cfg, **overrides)
