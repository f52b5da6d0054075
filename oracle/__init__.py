"""CPU oracle for the routed MXFP4 Mixture-of-Experts block.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
link this package: only the tests, the smoke check of the entry module and
the `cpu_baseline` leg of the benchmark use it. It shares no code with the
HIP library (no kernels, headers, tables, helpers or pre/post-processing);
the only thing both sides consume is the seeded input generator in
`workloads/`, which holds none of the block's arithmetic.

Modules:
- `mxfp4`  decoding of E2M1 codes and E8M0 scales (closed form), plane dequant.
- `act_quant`  the MX-FP4 round trip of activations (the quantised expert-input mode).
- `moe`    the block: RMSNorm, router, top-k, route weights, permutation,
           clamped SwiGLU, expert FFN, combine, layer stack. numpy float64.
- `brute`  the same block in pure Python loops (no numpy) for tiny inputs,
           with top-k by subset enumeration; it pins `moe`.
- `route_profile`  per-(layer, expert) selection counters and their summaries.
- `route_locality`  adjacent-token overlap and simulated per-layer expert caches
           over a decode trace, with the rankings of its reports.

Pins against what the pages and mathematics fix live in `tests/` (run with
`-m "not gpu"`). Parity status per function is stated in each docstring;
the clamped-SwiGLU body is a reading (no page prints it) and is marked
"parity unpinned by the pages" where it is defined.
"""
from . import mxfp4, act_quant, moe, brute, route_profile, route_locality  # noqa: F401
