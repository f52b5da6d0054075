// Routed-expert locality of a decode trace, on the host: per-expert counts and
// route weights, adjacent-token overlap, and simulated most-recent-first expert
// caches of several sizes. The trace is small (k indices and weights per token
// and layer) and each cache is a sequential walk, so this stays host code.
//
// Page: antirez ds4.c, the Metal routed-expert locality profiler (record,
// cache use, and the sort orders of its layer and hotlist writers).
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <numeric>
#include <vector>

#include "host_status.hpp"
#include "moe_mxfp4.h"

namespace {

constexpr int kMaxCaps = 16;

// One cache: at most `cap` experts, most recent first.
struct RecentList {
    std::vector<int32_t> e;
    int32_t cap = 0;

    // true on a hit; the expert ends at the front either way
    bool use(int32_t expert) {
        auto it = std::find(e.begin(), e.end(), expert);
        const bool hit = it != e.end();
        if (hit) {
            e.erase(it);
        } else if (static_cast<int32_t>(e.size()) == cap) {
            e.pop_back();
        }
        e.insert(e.begin(), expert);
        return hit;
    }
};

}  // namespace

extern "C" int moe_route_locality(const int32_t *idx, const float *weights, int64_t positions,
                                  int32_t layers, int32_t k, int32_t E, const int32_t *caps,
                                  int32_t n_caps, const moe_locality_out *out) {
    if (!out || !out->hist || !out->weight_hist || !out->adjacent_pairs || !out->overlap_sum ||
        !out->jaccard_sum)
        return moe::host_fail(MOE_ERR_INVALID_ARG, "locality outputs must be non-NULL");
    if (positions < 0 || layers < 1 || k < 1 || E < 1)
        return moe::host_fail(MOE_ERR_INVALID_ARG, "need positions >= 0, layers >= 1, k >= 1, E >= 1");
    if (positions > 0 && (!idx || !weights))
        return moe::host_fail(MOE_ERR_INVALID_ARG, "idx and weights must be non-NULL");
    if (n_caps < 0 || n_caps > kMaxCaps)
        return moe::host_fail(MOE_ERR_INVALID_ARG, "n_caps outside [0, 16]");
    if (n_caps > 0 && (!caps || !out->cache_hits || !out->cache_weight_hits))
        return moe::host_fail(MOE_ERR_INVALID_ARG, "caps and the cache outputs must be non-NULL");
    for (int32_t c = 0; c < n_caps; ++c)
        if (caps[c] < 1 || caps[c] > E)
            return moe::host_fail(MOE_ERR_INVALID_ARG, "a cache size lies outside [1, E]");

    const size_t LE = static_cast<size_t>(layers) * E;
    std::fill(out->hist, out->hist + LE, uint64_t{0});
    std::fill(out->weight_hist, out->weight_hist + LE, 0.0);
    std::fill(out->adjacent_pairs, out->adjacent_pairs + layers, uint64_t{0});
    std::fill(out->overlap_sum, out->overlap_sum + layers, 0.0);
    std::fill(out->jaccard_sum, out->jaccard_sum + layers, 0.0);
    if (n_caps > 0) {
        const size_t CL = static_cast<size_t>(n_caps) * layers;
        std::fill(out->cache_hits, out->cache_hits + CL, uint64_t{0});
        std::fill(out->cache_weight_hits, out->cache_weight_hits + CL, 0.0);
    }

    std::vector<RecentList> lists(static_cast<size_t>(n_caps) * layers);
    for (int32_t c = 0; c < n_caps; ++c)
        for (int32_t l = 0; l < layers; ++l) {
            RecentList &r = lists[static_cast<size_t>(c) * layers + l];
            r.cap = caps[c];
            r.e.reserve(static_cast<size_t>(caps[c]) + 1);
        }

    const size_t row = static_cast<size_t>(k);
    for (int64_t p = 0; p < positions; ++p) {
        for (int32_t l = 0; l < layers; ++l) {
            const size_t at = (static_cast<size_t>(p) * layers + l) * row;
            const int32_t *sel = idx + at;
            const float *w = weights + at;
            if (p > 0) {  // the previous position's record of this layer is adjacent
                const int32_t *prev = idx + at - static_cast<size_t>(layers) * row;
                int32_t shared = 0;
                for (int32_t a = 0; a < k; ++a)
                    shared += std::find(sel, sel + k, prev[a]) != sel + k;
                out->adjacent_pairs[l] += 1;
                out->overlap_sum[l] += static_cast<double>(shared) / k;
                out->jaccard_sum[l] += static_cast<double>(shared) / (2 * k - shared);
            }
            for (int32_t j = 0; j < k; ++j) {
                const int32_t e = sel[j];
                if (e < 0 || e >= E) continue;
                const double wj = static_cast<double>(w[j]);
                out->hist[static_cast<size_t>(l) * E + e] += 1;
                out->weight_hist[static_cast<size_t>(l) * E + e] += wj;
                for (int32_t c = 0; c < n_caps; ++c) {
                    const size_t cl = static_cast<size_t>(c) * layers + l;
                    if (lists[cl].use(e)) {
                        out->cache_hits[cl] += 1;
                        out->cache_weight_hits[cl] += wj;
                    }
                }
            }
        }
    }
    return moe::host_ok();
}

extern "C" int moe_route_hotlist(const uint64_t *hist, const double *weight_hist, int32_t layers,
                                 int32_t E, int32_t *order) {
    if (!hist || !weight_hist || !order)
        return moe::host_fail(MOE_ERR_INVALID_ARG, "hist, weight_hist and order must be non-NULL");
    if (layers < 1 || E < 1 || static_cast<int64_t>(layers) * E > INT32_MAX)
        return moe::host_fail(MOE_ERR_INVALID_ARG, "need layers >= 1, E >= 1, layers * E < 2^31");
    const int32_t n = layers * E;
    for (int32_t i = 0; i < n; ++i)  // the ranking needs a strict order on the weights
        if (!std::isfinite(weight_hist[i]))
            return moe::host_fail(MOE_ERR_INVALID_ARG, "a route-weight sum is not finite");
    std::iota(order, order + n, 0);
    // the index is layer * E + expert, so ascending index is layer, then expert
    std::sort(order, order + n, [&](int32_t a, int32_t b) {
        if (hist[a] != hist[b]) return hist[a] > hist[b];
        if (weight_hist[a] != weight_hist[b]) return weight_hist[a] > weight_hist[b];
        return a < b;
    });
    return moe::host_ok();
}
