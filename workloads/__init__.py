"""Seeded synthetic workloads for the routed MoE block.

This package only draws random inputs of the shapes, value distributions and
routing structure of the pages' models (gpt-oss-20b and DeepSeek-V4-Flash).
It holds none of the block's arithmetic: no decoding of MXFP4, no routing,
no SwiGLU. Both the CPU oracle and the GPU path consume what it produces.
"""
from .configs import CONFIGS, MoeConfig, config_by_id, scaled  # noqa: F401
from .gen import make_workload, make_layer, make_token_ids, Layer, Workload  # noqa: F401
