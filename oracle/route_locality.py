"""Routed-expert locality of a decode trace: adjacent-token overlap and
simulated per-layer expert caches.

TEST INFRASTRUCTURE ONLY (see the package docstring): only the tests, the
smoke check of the entry module and the benchmark's `cpu_baseline` leg use it.

Page: antirez ds4.c, the Metal routed-expert locality profiler (its record
step, its cache-use step, and the layer, cache-summary and hotlist writers).
Per layer it keeps, over the tokens of a decode run in position order:
- a count and a route-weight sum per expert;
- for every token whose previous record in the same layer sits at the
  directly preceding position: the number of its selected experts that the
  previous token also selected (each previous slot counted once if some
  current slot holds the same expert), the overlap (that number over k) and
  the Jaccard index (that number over 2k minus it);
- for each cache size n from 1, 2, 4, ..., 256, 384 that does not exceed the
  expert count, a list of at most n experts, most recent first. A selection
  already in the list is a hit (its count and its route weight are added to
  the hits), and moves to the front. Otherwise it is put at the front,
  and the last entry drops out once the list would exceed n.
Slots are visited in order 0..k-1 within a token. A selection whose expert
lies outside 0..E-1 takes part in the adjacency comparison only.

The summaries follow the page's writers: per cache size, hits over all
selections and weighted hits over the total route weight; per layer,
unique experts, mean overlap and mean Jaccard over the adjacent pairs, and
the experts ranked by count (descending), then weight (descending), then
index; the hotlist ranks every (layer, expert) the same way, with the layer
before the expert as the last keys.

Pinned in `tests/test_route_locality.py`: hit counts against the LRU
stack-distance characterisation by brute force, the closed forms at n = 1 and
at n >= the distinct experts, the inclusion property, a worked trace, and
constructed overlap cases.
"""
from __future__ import annotations

CACHE_SIZES = (1, 2, 4, 8, 16, 32, 64, 128, 256, 384)


def cache_sizes_for(E: int) -> list:
    """The page's candidate cache sizes that do not exceed E."""
    return [n for n in CACHE_SIZES if n <= E]


class RouteLocality:
    def __init__(self, layers: int, experts: int, k: int, caps=None):
        self.L, self.E, self.k = layers, experts, k
        self.caps = list(caps) if caps is not None else cache_sizes_for(experts)
        self.hist = [[0] * experts for _ in range(layers)]
        self.weight_hist = [[0.0] * experts for _ in range(layers)]
        self.cache = [[[] for _ in range(layers)] for _ in self.caps]
        self.cache_hits = [[0] * layers for _ in self.caps]
        self.cache_weight_hits = [[0.0] * layers for _ in self.caps]
        self.records = [0] * layers
        self.prev = [None] * layers  # (position, selected experts)
        self.adjacent_pairs = [0] * layers
        self.overlap_sum = [0.0] * layers
        self.jaccard_sum = [0.0] * layers

    def _use(self, ci: int, layer: int, expert: int, weight: float) -> None:
        entries = self.cache[ci][layer]
        if expert in entries:
            self.cache_hits[ci][layer] += 1
            self.cache_weight_hits[ci][layer] += weight
            entries.remove(expert)
            entries.insert(0, expert)
            return
        entries.insert(0, expert)
        if len(entries) > self.caps[ci]:
            entries.pop()

    def record(self, layer: int, pos: int, selected, weights) -> None:
        """One token's k selected experts and route weights in one layer."""
        selected = [int(e) for e in selected]
        weights = [float(w) for w in weights]
        self.records[layer] += 1
        prev = self.prev[layer]
        if prev is not None and prev[0] + 1 == pos:
            inter = sum(1 for a in prev[1] if a in selected)
            self.adjacent_pairs[layer] += 1
            self.overlap_sum[layer] += inter / self.k
            union = 2 * self.k - inter
            if union:
                self.jaccard_sum[layer] += inter / union
        self.prev[layer] = (pos, selected)
        for e, w in zip(selected, weights):
            if not 0 <= e < self.E:
                continue
            self.hist[layer][e] += 1
            self.weight_hist[layer][e] += w
            for ci in range(len(self.caps)):
                self._use(ci, layer, e, w)

    def record_trace(self, idx, w) -> None:
        """A trace of consecutive decode positions: idx and w [P, layers, k]."""
        for p in range(len(idx)):
            for layer in range(self.L):
                self.record(layer, p, idx[p][layer], w[p][layer])

    # -- summaries ---------------------------------------------------------

    def selections(self) -> int:
        return sum(sum(row) for row in self.hist)

    def total_weight(self) -> float:
        return sum(sum(row) for row in self.weight_hist)

    def hit_rate(self, ci: int) -> float:
        s = self.selections()
        return sum(self.cache_hits[ci]) / s if s else 0.0

    def weighted_hit_rate(self, ci: int) -> float:
        tw = self.total_weight()
        return sum(self.cache_weight_hits[ci]) / tw if tw > 0.0 else 0.0

    def mean_overlap(self, layer: int) -> float:
        n = self.adjacent_pairs[layer]
        return self.overlap_sum[layer] / n if n else 0.0

    def mean_jaccard(self, layer: int) -> float:
        n = self.adjacent_pairs[layer]
        return self.jaccard_sum[layer] / n if n else 0.0

    def ranked_experts(self, layer: int) -> list:
        """Experts with a nonzero count: count desc, weight desc, index asc."""
        ids = [e for e in range(self.E) if self.hist[layer][e]]
        return sorted(ids, key=lambda e: (-self.hist[layer][e], -self.weight_hist[layer][e], e))

    def hotlist(self) -> list:
        """Every (layer, expert), zero counts included, ranked count desc,
        weight desc, layer asc, expert asc."""
        pairs = [(l, e) for l in range(self.L) for e in range(self.E)]
        return sorted(pairs, key=lambda p: (-self.hist[p[0]][p[1]], -self.weight_hist[p[0]][p[1]],
                                            p[0], p[1]))
