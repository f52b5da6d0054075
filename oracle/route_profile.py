"""Expert-route profile: how often each expert of each layer is selected.

TEST INFRASTRUCTURE ONLY (see the package docstring): only the tests, the
smoke check of the entry module and the benchmark's `cpu_baseline` leg use it.

Page: goosedump `gpt_oss.rs`, `ExpertRouteProfile`. It holds one unsigned
64-bit counter per (layer, expert). `record(layer, experts)` is called once
per token and layer with the token's selected experts (from
`mixture_of_experts` and, token by token, `mixture_of_experts_batch`, right
after `top_experts`) and adds one to each selected expert's counter, with a
saturating add; a layer or expert index outside the table is skipped. The
summaries: `selections` (all counters summed, saturating),
`unique_layer_experts` (counters that are nonzero) and `layer_unique_counts`
(nonzero counters per layer).

Counters are Python integers, so the saturation at 2^64 - 1 is explicit.
Pinned in `tests/test_oracle_pins.py` by the route-count invariant (k per
token), the permutation histogram of `oracle.moe`, saturation, skipped
indices and constructed cases.
"""
from __future__ import annotations

U64_MAX = (1 << 64) - 1


class RouteProfile:
    def __init__(self, layers: int, experts: int):
        self.counts = [[0] * experts for _ in range(layers)]

    def record(self, layer: int, experts) -> None:
        if not 0 <= layer < len(self.counts):
            return
        row = self.counts[layer]
        for e in experts:
            e = int(e)
            if 0 <= e < len(row):
                row[e] = min(row[e] + 1, U64_MAX)

    def record_block(self, layer: int, idx) -> None:
        """One `record` per token of a block's top-k indices [T, k], in token order."""
        for token_experts in idx:
            self.record(layer, token_experts)

    def selections(self) -> int:
        total = 0
        for row in self.counts:
            for c in row:
                total = min(total + c, U64_MAX)
        return total

    def unique_layer_experts(self) -> int:
        return sum(1 for row in self.counts for c in row if c != 0)

    def layer_unique_counts(self) -> list:
        return [sum(1 for c in row if c != 0) for row in self.counts]

    def table(self):
        """The counters as a uint64 numpy array [layers, experts]."""
        import numpy as np
        return np.array(self.counts, dtype=np.uint64).reshape(len(self.counts), -1)
