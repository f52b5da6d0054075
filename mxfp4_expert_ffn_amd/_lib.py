"""ctypes declarations of libmoe_mxfp4.so (the C ABI in include/moe_mxfp4.h)."""
from __future__ import annotations

import ctypes
import os

# the in-tree build; MOE_MXFP4_LIB names another build of the same sources
LIB_PATH = os.environ.get("MOE_MXFP4_LIB") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libmoe_mxfp4.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_WORKSPACE = -3
MOE_ERR_HIP = -4
MOE_NOALLOC_SCRATCH_BYTES = 32 << 20  # the fixed device scratch per GPU
MOE_F32 = 0
MOE_BF16 = 1

# moe_kernel_id
KERNELS = {"rmsnorm": 0, "router": 1, "topk": 2, "permute": 3, "decode_gate_up": 4,
           "decode_down": 5, "gate_up_gemm": 6, "down_gemm": 7, "quantize": 8, "combine": 9}


class MoeShape(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int32), ("H", ctypes.c_int32), ("F", ctypes.c_int32),
        ("E", ctypes.c_int32), ("k", ctypes.c_int32), ("act_dtype", ctypes.c_int32),
        ("n_shared", ctypes.c_int32), ("swiglu_alpha", ctypes.c_float),
        ("swiglu_limit", ctypes.c_float), ("swiglu_up_offset", ctypes.c_float),
        ("route_scale", ctypes.c_float), ("rms_eps", ctypes.c_float),
        ("act_quant", ctypes.c_int32),
    ]


class MoeBlobLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in (
        "gate_q", "up_q", "down_q", "gate_s", "up_s", "down_s", "gate_b", "up_b", "down_b",
        "bytes", "stride")]


class MoeExpertPlanes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "gate_q", "up_q", "down_q", "gate_s", "up_s", "down_s", "gate_b", "up_b", "down_b")]


class MoeRouteOut(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "topk_idx", "topk_w", "counts", "offsets", "perm", "inv", "route_counts")]


class MoeRouting(ctypes.Structure):
    _fields_ = [("sel_bias", ctypes.c_void_p), ("tid2eid", ctypes.c_void_p),
                ("token_ids", ctypes.c_void_p), ("vocab", ctypes.c_int32)]


class MoePrefillPlan(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "tile_rows", "x_terms", "act_terms", "gate_up_features", "down_rows")]


class MoeLocalityOut(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "hist", "weight_hist", "cache_hits", "cache_weight_hits", "adjacent_pairs",
        "overlap_sum", "jaccard_sum")]


# every symbol the header declares, with its ctypes signature
_P = ctypes.c_void_p
SIGNATURES = {
    "moe_blob_layout_get": (ctypes.c_int, [ctypes.POINTER(MoeShape), ctypes.POINTER(MoeBlobLayout)]),
    "moe_pack_experts": (ctypes.c_int, [ctypes.POINTER(MoeShape), ctypes.c_int32,
                                        ctypes.POINTER(MoeExpertPlanes), _P]),
    "moe_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(MoeShape)]),
    "moe_route": (ctypes.c_int, [ctypes.POINTER(MoeShape), _P, _P, _P, _P,
                                 ctypes.POINTER(MoeRouting), ctypes.POINTER(MoeRouteOut), _P,
                                 ctypes.c_size_t, _P]),
    "moe_forward_decode": (ctypes.c_int, [ctypes.POINTER(MoeShape), _P, _P, _P, _P,
                                          ctypes.POINTER(MoeRouting), _P, _P, _P,
                                          ctypes.POINTER(MoeRouteOut), _P, ctypes.c_size_t, _P]),
    "moe_forward_prefill": (ctypes.c_int, [ctypes.POINTER(MoeShape), _P, _P, _P, _P,
                                           ctypes.POINTER(MoeRouting), _P, _P, _P,
                                           ctypes.POINTER(MoeRouteOut), _P, ctypes.c_size_t, _P]),
    "moe_forward_decode_noalloc": (ctypes.c_int, [ctypes.POINTER(MoeShape), _P, _P, _P, _P,
                                                  ctypes.POINTER(MoeRouting), _P, _P, _P,
                                                  ctypes.POINTER(MoeRouteOut), _P]),
    "moe_prefill_plan": (ctypes.c_int, [ctypes.POINTER(MoeShape), ctypes.c_int32,
                                        ctypes.POINTER(MoePrefillPlan)]),
    "moe_act_quant_debug": (ctypes.c_int, [ctypes.POINTER(MoeShape), _P, _P, _P, _P, _P,
                                           ctypes.c_size_t, _P]),
    "moe_dequant_debug": (ctypes.c_int, [ctypes.POINTER(MoeShape), _P, ctypes.c_int32,
                                         ctypes.c_int32, _P, _P]),
    "moe_profile_next_launch": (ctypes.c_int, [ctypes.c_int32, _P, _P]),
    "moe_route_profile_summary": (ctypes.c_int, [_P, ctypes.c_int32, ctypes.c_int32, _P, _P, _P]),
    "moe_route_locality": (ctypes.c_int, [_P, _P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_int32, _P, ctypes.c_int32,
                                          ctypes.POINTER(MoeLocalityOut)]),
    "moe_route_hotlist": (ctypes.c_int, [_P, _P, ctypes.c_int32, ctypes.c_int32, _P]),
    "moe_last_error": (ctypes.c_char_p, []),
}

_lib = None


def load() -> ctypes.CDLL:
    """Load the HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m mxfp4_expert_ffn_amd.build` (hipcc, gfx950)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib
