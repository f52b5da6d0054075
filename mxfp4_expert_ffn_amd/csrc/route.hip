// Routing kernels: RMSNorm, router logits (fp64), top-k + route weights,
// per-expert histogram / exclusive scan / stable permutation.
//
// Pages: goosedump `gpt_oss.rs` `mixture_of_experts_batch` (router matmul,
// add_bias_batch, top_experts, softmax, routes_by_expert in token order),
// `top_experts` (descending value, lower index on ties); antirez `ds4.c`
// `rms_norm_weight` (sum of squares accumulated in double).
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

template <int KIND>
__device__ __forceinline__ double load_in(const void *x, size_t i) {
    if constexpr (KIND == 0) return static_cast<double>(static_cast<const float *>(x)[i]);
    else if constexpr (KIND == 1) return static_cast<double>(bf16_bits_to_f32(static_cast<const uint16_t *>(x)[i]));
    else return static_cast<const double *>(x)[i];
}

// ---------------------------------------------------------------- RMSNorm
// One workgroup per token: fp64 sum of squares, inv = 1/sqrt(ss/H + eps),
// xn = x * inv * gamma kept in fp64 (for the router) and float32 (experts).
template <int KIND>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const void *x, const float *gamma, int H,
                                                      float eps, double *xn64, float *xn32) {
    const int t = blockIdx.x;
    const size_t row = static_cast<size_t>(t) * H;
    double ss = 0.0;
    for (int h = threadIdx.x; h < H; h += blockDim.x) {
        const double v = load_in<KIND>(x, row + h);
        ss = fma(v, v, ss);
    }
    __shared__ double part[4];
    ss = wave_sum_f64(ss);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
    __syncthreads();
    const double total = part[0] + part[1] + part[2] + part[3];
    const double inv = 1.0 / sqrt(total / H + static_cast<double>(eps));
    for (int h = threadIdx.x; h < H; h += blockDim.x) {
        const double v = load_in<KIND>(x, row + h) * inv * static_cast<double>(gamma[h]);
        xn64[row + h] = v;
        xn32[row + h] = static_cast<float>(v);
    }
}

// ---------------------------------------------------------------- router logits
// Both router kernels write split-K partial sums partial[s][t][e] (fp64) over
// hidden-dimension slices; consumers add the S partials in split order and
// the bias (gather_logits), so the logits are deterministic. fp32 x fp32
// products are exact in fp64.

// Few tokens: one wavefront per (expert, hidden slice of kRouterGemvSlice
// units); lane l holds the router weights of units 4(l + 64i) .. +3 of the
// slice in registers (all loads issued at once), then each token's
// activations are loaded the same way and reduced with a wave sum.
template <int KIND>
__device__ __forceinline__ void load4(const void *x, size_t i, double (&v)[4]) {
    if constexpr (KIND == 0) {
        const float4 f = *reinterpret_cast<const float4 *>(static_cast<const float *>(x) + i);
        v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
    } else if constexpr (KIND == 1) {
        const uint2 u = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(x) + i);
        v[0] = __uint_as_float(u.x << 16); v[1] = __uint_as_float(u.x & 0xffff0000u);
        v[2] = __uint_as_float(u.y << 16); v[3] = __uint_as_float(u.y & 0xffff0000u);
    } else {
        const double *d = static_cast<const double *>(x) + i;
        v[0] = d[0]; v[1] = d[1]; v[2] = d[2]; v[3] = d[3];
    }
}

// Workgroups past the router's own quantise the expert input into FP8 terms
// for the block-scaled decode kernels: one half-wavefront per 32-value block
// of k (the unit an E8M0 scale of the matrix core's operand B covers); codes
// go to xq[t][n][k] (zero past H), scales to xs[t][n][k / 32].
__device__ __forceinline__ void quantize_terms_group(const void *q_in, int q_bf16, int T, int H,
                                                     int Kp, uint8_t *xq, uint8_t *xs, int gidx) {
    const int lane = threadIdx.x & 63, i = lane & 31;
    const int nb = Kp / 32;  // blocks per token
    const bool on = gidx < T * nb;
    const int g = on ? gidx : 0;
    const int t = g / nb, blk = g - t * nb;
    const int kk = 32 * blk + i;
    float v = 0.f;
    if (on && kk < H) {
        const size_t at = static_cast<size_t>(t) * H + kk;
        v = q_bf16 ? bf16_bits_to_f32(static_cast<const uint16_t *>(q_in)[at])
                   : static_cast<const float *>(q_in)[at];
    }
    uint32_t codes, scales;
    fp8_terms_group(v, codes, scales);
    if (on) {
#pragma unroll
        for (int n = 0; n < kTerms; ++n) {
            xq[(static_cast<size_t>(t) * kTerms + n) * Kp + kk] = static_cast<uint8_t>(codes >> (8 * n));
            if (i == 0)
                xs[(static_cast<size_t>(t) * kTerms + n) * nb + blk] = static_cast<uint8_t>(scales >> (8 * n));
        }
    }
}

// Stand-alone form of the FP8-term quantisation, for batches the tiled router
// takes: 8 blocks of 32 values per workgroup and round, over a grid-stride
// loop (few, long-lived workgroups rather than one per 8 blocks). The loop
// runs per wavefront, both halves together, as the group maximum needs.
__global__ __launch_bounds__(256) void quantize_terms_kernel(const void *q_in, int q_bf16, int T,
                                                             int H, int Kp, uint8_t *xq,
                                                             uint8_t *xs) {
    const int total = T * (Kp / 32);
    const int half = (threadIdx.x >> 5) & 1;
    for (int g0 = blockIdx.x * 8 + 2 * (threadIdx.x >> 6); g0 < total; g0 += gridDim.x * 8)
        quantize_terms_group(q_in, q_bf16, T, H, Kp, xq, xs, g0 + half);
}

template <int KIND>
__global__ __launch_bounds__(256) void router_gemv_kernel(const void *x, const float *w, int T,
                                                          int H, int E, double *partial,
                                                          int router_wgs, const void *q_in,
                                                          int q_bf16, int Kp, uint8_t *xq,
                                                          uint8_t *xs) {
    constexpr int NV = kRouterGemvSlice / 256;  // float4 per lane
    const int lane = threadIdx.x & 63;
    if (static_cast<int>(blockIdx.x) >= router_wgs) {
        const int gidx = (blockIdx.x - router_wgs) * 8 + (threadIdx.x >> 5);
        quantize_terms_group(q_in, q_bf16, T, H, Kp, xq, xs, gidx);
        return;
    }
    const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int S = (H + kRouterGemvSlice - 1) / kRouterGemvSlice;
    if (item >= E * S) return;  // whole wavefront; no workgroup barrier below
    const int e = item / S, s = item - e * S;
    const int hbase = s * kRouterGemvSlice;
    float4 wr[NV];
    bool on[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int h = hbase + 4 * (lane + 64 * i);
        on[i] = h < H;
        wr[i] = *reinterpret_cast<const float4 *>(w + static_cast<size_t>(e) * H + (on[i] ? h : 0));
    }
    for (int t = 0; t < T; ++t) {
        double xv[NV][4];
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int h = hbase + 4 * (lane + 64 * i);
            load4<KIND>(x, static_cast<size_t>(t) * H + (on[i] ? h : 0), xv[i]);
        }
        double acc = 0.0;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            if (on[i]) {
                acc = fma(static_cast<double>(wr[i].x), xv[i][0], acc);
                acc = fma(static_cast<double>(wr[i].y), xv[i][1], acc);
                acc = fma(static_cast<double>(wr[i].z), xv[i][2], acc);
                acc = fma(static_cast<double>(wr[i].w), xv[i][3], acc);
            }
        }
        acc = wave_sum_f64(acc);
        if (lane == 0) partial[(static_cast<size_t>(s) * T + t) * E + e] = acc;
    }
}

// Tiled router for larger batches: a workgroup computes the fp64 partial
// logits of 64 tokens x 64 experts over one K slice on the fp64 matrix cores
// (v_mfma_f64_16x16x4_f64): each of its 4 wavefronts holds 32 tokens x 32
// experts as 2 x 2 result tiles. K advances 32 at a time through
// double-buffered LDS tiles kept in the inputs' own precision (widened
// exactly to fp64 when read), 4 per instruction; the next chunk's loads are
// in flight during the current chunk's instructions. Tokens and experts past
// T and E are clamped on load and not written.
//
// Instruction lanes (measured on gfx950): operand A lane l = A[l % 16][l / 16]
// (token, k), operand B lane l = B[l / 16][l % 16] (k, expert); result lane l
// holds D[4v + l / 16][l % 16], v = 0..3.
typedef double f64x4_t __attribute__((ext_vector_type(4)));

template <int KIND>
__global__ __launch_bounds__(256) void router_tiled_kernel(const void *x, const float *w, int T,
                                                           int H, int E, int slice,
                                                           double *partial) {
    typedef typename std::conditional<KIND == 2, double, float>::type XT;
    constexpr int kPad = 4;
    __shared__ __align__(16) XT xs[2][32][64 + kPad];     // [k][token]
    __shared__ __align__(16) float wsm[2][32][64 + kPad];  // [k][expert]
    const int tid = threadIdx.x;
    const int t0 = blockIdx.x * 64, e0 = blockIdx.y * 64, s = blockIdx.z;
    const int hbeg = s * slice, hend = min(H, hbeg + slice);
    // loads: thread -> (row tid / 4, k part 8 * (tid % 4)) of the 64 x 32 chunk
    const int lr = tid >> 2, lk = 8 * (tid & 3);
    const size_t xrow = static_cast<size_t>(min(t0 + lr, T - 1)) * H;
    const float *wrow = w + static_cast<size_t>(min(e0 + lr, E - 1)) * H;
    XT xv[8];
    float wv[8];
    auto load = [&](int h0) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (KIND == 1) xv[i] = bf16_bits_to_f32(static_cast<const uint16_t *>(x)[xrow + h0 + lk + i]);
            else xv[i] = static_cast<const XT *>(x)[xrow + h0 + lk + i];
        }
        const float4 a = *reinterpret_cast<const float4 *>(wrow + h0 + lk);
        const float4 b = *reinterpret_cast<const float4 *>(wrow + h0 + lk + 4);
        wv[0] = a.x; wv[1] = a.y; wv[2] = a.z; wv[3] = a.w;
        wv[4] = b.x; wv[5] = b.y; wv[6] = b.z; wv[7] = b.w;
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            xs[buf][lk + i][lr] = xv[i];
            wsm[buf][lk + i][lr] = wv[i];
        }
    };
    const int lane = tid & 63, wave = tid >> 6;
    const int tb = (wave & 1) * 32, eb = (wave >> 1) * 32;  // the wavefront's tokens, experts
    const int col = lane & 15, kq = lane >> 4;
    f64x4_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f64x4_t{0.0, 0.0, 0.0, 0.0};
    load(hbeg);
    int buf = 0;
    for (int h0 = hbeg; h0 < hend; h0 += 32) {
        store(buf);
        __syncthreads();
        if (h0 + 32 < hend) load(h0 + 32);
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const int kk = 4 * ks + kq;
            double a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) a[i] = static_cast<double>(xs[buf][kk][tb + 16 * i + col]);
#pragma unroll
            for (int j = 0; j < 2; ++j) b[j] = static_cast<double>(wsm[buf][kk][eb + 16 * j + col]);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        buf ^= 1;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int t = t0 + tb + 16 * i + 4 * v + kq;
                const int e = e0 + eb + 16 * j + col;
                if (t < T && e < E) partial[(static_cast<size_t>(s) * T + t) * E + e] = acc[i][j][v];
            }
}

// ---------------------------------------------------------------- top-k
// One wavefront per token: logits from the router partials, top-k, route
// weights; optionally copies the residual into `out` (the grouped down GEMM
// then adds into it).
__global__ __launch_bounds__(256) void topk_kernel(const double *partial, int S, const float *bias,
                                                   int T, int E, int k, float route_scale,
                                                   int32_t *idx, float *wts, int32_t *out_idx,
                                                   float *out_w, const void *resid,
                                                   int resid_bf16, int H, float *out) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    double v[4];
    if (E <= 64) gather_logits<1>(partial, S, T, t, E, bias, v);
    else if (E <= 128) gather_logits<2>(partial, S, T, t, E, bias, v);
    else gather_logits<4>(partial, S, T, t, E, bias, v);
    int sel[kMaxK];
    double val[kMaxK];
    wave_topk(v, E, k, sel, val);
    float w[kMaxK];
    route_softmax(val, k, route_scale, w);
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
        if (j < k && lane == j) {
            idx[t * k + j] = sel[j];
            wts[t * k + j] = w[j];
            if (out_idx) out_idx[t * k + j] = sel[j];
            if (out_w) out_w[t * k + j] = w[j];
        }
    }
    if (out) {
        float *o = out + static_cast<size_t>(t) * H;
        if (resid_bf16) {
            const uint16_t *r = static_cast<const uint16_t *>(resid) + static_cast<size_t>(t) * H;
            for (int h = lane; h < H; h += 64) o[h] = bf16_bits_to_f32(r[h]);
        } else {
            const float4 *r = reinterpret_cast<const float4 *>(static_cast<const float *>(resid) +
                                                               static_cast<size_t>(t) * H);
            float4 *o4 = reinterpret_cast<float4 *>(o);
            if (static_cast<const void *>(r) != static_cast<const void *>(o4))
                for (int h = lane; h < H / 4; h += 64) o4[h] = r[h];
        }
    }
}

// ---------------------------------------------------------------- permutation
// One workgroup of 1024 threads. Routes r = t*k + j are taken in chunks of
// 1024; inside a wavefront the lanes holding the same expert are found with
// eight bit-plane ballots and ranked by lane; per-wave counts are prefix-summed per expert in
// wave order, so a route's rank counts exactly the earlier routes of its
// expert: the permutation is stable (ascending token). Then counts, the
// exclusive scan and the M-tile prefix for the grouped GEMMs (a workgroup
// scan, one group per thread), perm and inv.
// Group E (when n_shared) is the shared expert: T rows, identity order.
__global__ __launch_bounds__(1024) void permute_kernel(
    const int32_t *idx, int T, int E, int k, int n_shared, int bm, int32_t *counts,
    int32_t *offsets, int32_t *perm, int32_t *inv, int32_t *rank, int32_t *mprefix,
    int32_t *out_counts, int32_t *out_offsets, int32_t *out_perm, int32_t *out_inv) {
    __shared__ int wcnt[16][kMaxE];
    __shared__ int base[kMaxE + 1];
    __shared__ int start[kMaxE + 2];
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int R = T * k;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int e = tid; e < E; e += 1024) base[e] = 0;
    __syncthreads();
    int e_next = tid < R ? idx[tid] : 0;  // the next chunk's experts load during this one
    for (int c0 = 0; c0 < R; c0 += 1024) {
        for (int i = tid; i < 16 * kMaxE; i += 1024) wcnt[i / kMaxE][i % kMaxE] = 0;
        const int r = c0 + tid;
        const bool valid = r < R;
        const int e = e_next;
        if (r + 1024 < R) e_next = idx[r + 1024];
        __syncthreads();
        // lanes holding the same expert: the intersection of the 8 bit-plane
        // ballots of the expert index
        static_assert(kMaxE <= 256, "expert indices fit 8 bit planes");
        uint64_t eq = __ballot(valid);
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const bool bit = (e >> b) & 1;
            const uint64_t plane = __ballot(bit);
            eq &= bit ? plane : ~plane;
        }
        const int myrank = __popcll(eq & lt_mask);
        if (valid && myrank == 0) wcnt[w][e] = __popcll(eq);  // the first lane of its expert
        __syncthreads();
        for (int ee = tid; ee < E; ee += 1024) {
            int run = base[ee];
            for (int ww = 0; ww < 16; ++ww) {
                const int c = wcnt[ww][ee];
                wcnt[ww][ee] = run;
                run += c;
            }
            base[ee] = run;
        }
        __syncthreads();
        if (valid) rank[r] = wcnt[w][e] + myrank;
        __syncthreads();
    }
    // counts, their exclusive scan and the tile prefix: one group per thread
    // (G <= kMaxE + 1 <= 1024), wavefront scans, then the totals of the
    // wavefronts before
    const int G = E + n_shared;
    __shared__ int wsum_c[16], wsum_t[16];
    {
        const int g = tid;
        const int c = g < G ? (g < E ? base[g] : T) : 0;
        const int nt = (c + bm - 1) / bm;
        int sc = c, st = nt;  // inclusive scans within the wavefront
        for (int d = 1; d < 64; d <<= 1) {
            const int oc = __shfl_up(sc, d), ot = __shfl_up(st, d);
            if (lane >= d) {
                sc += oc;
                st += ot;
            }
        }
        if (lane == 63) {
            wsum_c[w] = sc;
            wsum_t[w] = st;
        }
        __syncthreads();
        int pc = 0, pt = 0;
        for (int ww = 0; ww < w; ++ww) {
            pc += wsum_c[ww];
            pt += wsum_t[ww];
        }
        const int off = pc + sc - c, mt = pt + st - nt;
        if (g < G) {
            start[g] = off;
            offsets[g] = off;
            mprefix[g] = mt;
            counts[g] = c;
            if (out_counts && g < E) out_counts[g] = c;
            if (out_offsets && g < E) out_offsets[g] = off;
        }
        if (g == G - 1) {
            start[G] = off + c;
            offsets[G] = off + c;
            mprefix[G] = mt + nt;
        }
        if (out_offsets && g == 0) out_offsets[E] = R;
    }
    __syncthreads();
    for (int r = tid; r < R; r += 1024) {
        const int pos = start[idx[r]] + rank[r];
        perm[pos] = r;
        inv[r] = pos;
        if (out_perm) out_perm[pos] = r;
        if (out_inv) out_inv[r] = pos;
    }
}

}  // namespace

hipError_t launch_rmsnorm(const void *x, int x_bf16, const float *gamma, int T, int H, float eps,
                          double *xn64, float *xn32, hipStream_t s) {
    if (x_bf16)
        launch_kernel(rmsnorm_kernel<1>, T, 256, s, x, gamma, H, eps, xn64, xn32);
    else
        launch_kernel(rmsnorm_kernel<0>, T, 256, s, x, gamma, H, eps, xn64, xn32);
    return hipGetLastError();
}

RouterPlan router_plan(int T, int H, int E) {
    RouterPlan p;
    if (T <= kRouterGemvMaxT) {
        p.gemv = true;
        p.slice = kRouterGemvSlice;
        p.splits = (H + kRouterGemvSlice - 1) / kRouterGemvSlice;
        return p;
    }
    const int tiles = ((T + 63) / 64) * ((E + 63) / 64);
    int want = (512 + tiles - 1) / tiles;
    want = want < 1 ? 1 : (want > kRouterMaxSplits ? kRouterMaxSplits : want);
    const int units = H / 32;
    if (want > units) want = units;
    p.gemv = false;
    p.slice = 32 * ((units + want - 1) / want);
    p.splits = (H + p.slice - 1) / p.slice;
    return p;
}

hipError_t launch_router(const void *x, int in_kind, const float *w, int T, int H, int E,
                         double *partial, const TermsOut *terms, hipStream_t s) {
    const RouterPlan p = router_plan(T, H, E);
    if (p.gemv) {
        const int rwgs = (E * p.splits + 3) / 4;
        int qwgs = 0, Kp = 0;
        if (terms) {
            Kp = 128 * ((H + 127) / 128);
            qwgs = (T * (Kp / 32) + 7) / 8;
        }
        const void *qin = terms ? terms->in : nullptr;
        const int qbf = terms ? terms->in_bf16 : 0;
        uint8_t *xq = terms ? terms->q : nullptr;
        uint8_t *xs = terms ? terms->scales : nullptr;
        const int grid = rwgs + qwgs;
        if (in_kind == 0)
            launch_kernel(router_gemv_kernel<0>, grid, 256, s, x, w, T, H, E, partial, rwgs, qin,
                          qbf, Kp, xq, xs);
        else if (in_kind == 1)
            launch_kernel(router_gemv_kernel<1>, grid, 256, s, x, w, T, H, E, partial, rwgs, qin,
                          qbf, Kp, xq, xs);
        else
            launch_kernel(router_gemv_kernel<2>, grid, 256, s, x, w, T, H, E, partial, rwgs, qin,
                          qbf, Kp, xq, xs);
    } else {
        if (terms) return hipErrorInvalidValue;  // see router_quantizes
        const dim3 grid((T + 63) / 64, (E + 63) / 64, p.splits);
        if (in_kind == 0)
            launch_kernel(router_tiled_kernel<0>, grid, 256, s, x, w, T, H, E, p.slice, partial);
        else if (in_kind == 1)
            launch_kernel(router_tiled_kernel<1>, grid, 256, s, x, w, T, H, E, p.slice, partial);
        else
            launch_kernel(router_tiled_kernel<2>, grid, 256, s, x, w, T, H, E, p.slice, partial);
    }
    return hipGetLastError();
}

bool router_quantizes(int T) { return T <= kRouterGemvMaxT; }

hipError_t launch_quantize(const TermsOut &terms, int T, int H, hipStream_t s) {
    const int Kp = pad128(H);
    const int wgs = (T * (Kp / 32) + 7) / 8;
    launch_kernel(quantize_terms_kernel, wgs < 2048 ? wgs : 2048, 256, s, terms.in, terms.in_bf16,
                  T, H, Kp, terms.q, terms.scales);
    return hipGetLastError();
}

hipError_t launch_topk(const double *partial, int S, const float *bias, int T, int E, int k,
                       float route_scale, int32_t *idx, float *wts, int32_t *out_idx, float *out_w,
                       const void *resid, int resid_bf16, int H, float *out, hipStream_t s) {
    launch_kernel(topk_kernel, (T + 3) / 4, 256, s, partial, S, bias, T, E, k, route_scale, idx,
                  wts, out_idx, out_w, resid, resid_bf16, H, out);
    return hipGetLastError();
}

hipError_t launch_permute(const int32_t *idx, int T, int E, int k, int n_shared, int tile_rows,
                          int32_t *counts,
                          int32_t *offsets, int32_t *perm, int32_t *inv, int32_t *rank,
                          int32_t *mprefix, int32_t *out_counts, int32_t *out_offsets,
                          int32_t *out_perm, int32_t *out_inv, hipStream_t s) {
    launch_kernel(permute_kernel, 1, 1024, s, idx, T, E, k, n_shared, tile_rows, counts, offsets,
                  perm, inv, rank, mprefix, out_counts, out_offsets, out_perm, out_inv);
    return hipGetLastError();
}

}  // namespace moe
