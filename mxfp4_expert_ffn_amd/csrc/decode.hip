// Decode (T <= 64): per route, GEMVs over the selected expert's MXFP4 planes
// on the block-scaled matrix cores, after the router launch: gate/up over
// (route, 32-feature block), then down over (token, 16-row block of H) with
// every route of the token inside one workgroup.
//
// gate/up: a work item is 32 weight rows (two 16-row tiles) of gate and up of
// one route, for one workgroup; its 8 wavefronts split K into 128-wide steps.
// Every wavefront issues all of its loads (B first, then the weight tiles
// from a scalar base) before its first matrix-core instruction, with no branch
// in between, so each instruction waits only for its own operands. Weight
// tiles are read as whole contiguous kilobytes (the blob's tiled plane
// layout). The expert input arrives as FP8 terms in B columns 0..kTerms-1; the
// other 12 columns are zero, which costs nothing here: the GEMV is bound by
// weight bytes. The epilogue multiplies the SwiGLU output by the route weight
// before making its FP8 terms, so down can add all routes of a token in one
// accumulator.
//
// down: one workgroup owns 16 output rows of one token and runs the (route,
// K-step) fragments of all its routes, dealt over its wavefronts in a fixed
// order; the wavefronts' sums are added in wavefront order, then the
// route-weighted biases in slot order, into the residual already in out. Each
// output element has exactly one writer and a fixed summation order, so the
// result is the same on every run.
//
// Page: goosedump `gpt_oss.rs`, `mixture_of_experts` (gate/up pair with
// biases, clamped SwiGLU, down with bias, route weight, slot sum into the
// residual) and `mix_expert_outputs` (each route added once, in slot order).
#include "mx_mfma.hpp"

namespace moe {

namespace {

typedef uint32_t dec_u32x4 __attribute__((ext_vector_type(4)));

// B operand loaded straight from the FP8-term array (down, when a token's
// terms do not fit in LDS), through a buffer resource over the whole array,
// so that lanes whose column holds no term (n >= kTerms) and fragments past
// the end read zeros without touching memory:
// the row offset `row` is the byte offset of term row (row, n) in `q`, and
// `srow` that of its scale row in `sc`; `on` false gives a zero operand.
struct TermRows {
    __amdgpu_buffer_rsrc_t q, s;
};
__device__ __forceinline__ TermRows term_rows(const uint8_t *q, const uint8_t *sc, uint32_t qbytes,
                                              uint32_t sbytes) {
    // raw buffers (stride 0) over the arrays; loads past the size return 0
    constexpr int kRawFlags = 0x00020000;
    return TermRows{__builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(q), 0, qbytes, kRawFlags),
                    __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(sc), 0, sbytes, kRawFlags)};
}
typedef int dec_i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ BFrag load_bfrag_buf(const TermRows &tr, uint32_t row, uint32_t srow,
                                                int step, int h, bool on) {
    constexpr uint32_t kOff = 0x80000000u;  // past any array the library builds
    const uint32_t o = on ? row + 128u * step + 16u * h : kOff;
    const uint32_t so = on ? srow + 4u * step + h : kOff;
    const dec_i32x4 lo = __builtin_amdgcn_raw_buffer_load_b128(tr.q, o, 0, 0);
    const dec_i32x4 hi = __builtin_amdgcn_raw_buffer_load_b128(tr.q, o + 64u, 0, 0);
    BFrag b;
    b.lo = make_uint4(lo.x, lo.y, lo.z, lo.w);
    b.hi = make_uint4(hi.x, hi.y, hi.z, hi.w);
    b.s = __builtin_amdgcn_raw_buffer_load_b8(tr.s, so, 0, 0);
    return b;
}

// FP8-term rows staged in LDS: term row q (q = route * kTerms + n) holds
// Kp code bytes at q * (Kp + kRowPad) (the pad staggers the rows over the LDS
// banks), then the scale rows, Kp / 32 bytes each, packed, then 64 zero
// bytes that lanes without a term read. The staged rows are two runs of
// consecutive global term rows (a token's routed rows, then its shared-expert
// row), copied by the whole workgroup: codes in 16-byte chunks, CH per
// thread, scales in dwords, one per thread. Chunks past the end repeat the
// last one, so no branch sits between the loads.
constexpr int kRowPad = 16;
struct Staged {
    int Kp, nq;          // bytes per code row, rows
    __device__ __forceinline__ int stride() const { return Kp + kRowPad; }
    __device__ __forceinline__ int scale_off() const { return nq * stride(); }
    __device__ __forceinline__ int zero_off() const { return scale_off() + nq * (Kp / 32); }
};
__host__ __device__ constexpr int staged_bytes(int Kp, int nq) { return nq * (Kp + kRowPad + Kp / 32) + 64; }
// Source byte offsets (in the code and scale arrays) of staged code chunk c and
// scale dword c: rows [0, na) from global row ra, the rest from global row rb.
__device__ __forceinline__ size_t stage_code_src(const Staged &sg, int c, int na, int ra, int rb) {
    const int per = sg.Kp / 16, ca = na * per;
    return c < ca ? static_cast<size_t>(ra) * sg.Kp + 16u * c
                  : static_cast<size_t>(rb) * sg.Kp + 16u * (c - ca);
}
__device__ __forceinline__ size_t stage_scale_src(const Staged &sg, int c, int na, int ra, int rb) {
    const int per = sg.Kp / 128, ca = na * per;
    return c < ca ? static_cast<size_t>(ra) * (sg.Kp / 32) + 4u * c
                  : static_cast<size_t>(rb) * (sg.Kp / 32) + 4u * (c - ca);
}
__device__ __forceinline__ int stage_code_dst(const Staged &sg, int c) {
    const int per = sg.Kp / 16, q = c / per;
    return q * sg.stride() + 16 * (c - q * per);
}
// B operand of step s from staged term rows q0 .. q0 + kTerms - 1 (lane
// column n < kTerms reads row q0 + n; other columns read zeros).
__device__ __forceinline__ BFrag lds_bfrag(const uint8_t *lds, const Staged &sg, int q0, int s,
                                           int n, int h) {
    const bool on = n < kTerms;
    const int qo = on ? (q0 + n) * sg.stride() + 128 * s + 16 * h : sg.zero_off();
    const int so = on ? sg.scale_off() + (q0 + n) * (sg.Kp / 32) + 4 * s + h : sg.zero_off();
    BFrag b;
    b.lo = *reinterpret_cast<const uint4 *>(lds + qo);
    b.hi = *reinterpret_cast<const uint4 *>(lds + qo + (on ? 64 : 16));
    b.s = lds[so];
    return b;
}

// The experts of token t (top-k of its router logits - fp64 split-K partials
// + bias - or the routing variant's choice) by one wavefront: the selected
// experts and their logits, in every lane.
// `between`: the caller's loads, issued behind the partials' (gather_logits).
// SMALL_E: the kernel serves E <= 128 only (its registers are sized for that).
template <bool SMALL_E, typename Between = NoLoads>
__device__ __forceinline__ void route_token(const double *partial, int S, const float *router_b,
                                            const RouteSel &rs, int T, int t, int E, int k,
                                            int (&sel)[kMaxK], double (&val)[kMaxK],
                                            Between &&between = Between{}) {
    double v[kMaxQ];
    if constexpr (SMALL_E) {
        if (E <= 64) {
            gather_logits<1>(partial, S, T, t, E, router_b, v, between);
            select_routes<1>(v, rs, t, E, k, sel, val);
        } else {
            gather_logits<2>(partial, S, T, t, E, router_b, v, between);
            select_routes<2>(v, rs, t, E, k, sel, val);
        }
    } else if (E <= 256) {
        gather_logits<4>(partial, S, T, t, E, router_b, v, between);
        select_routes<4>(v, rs, t, E, k, sel, val);
    } else {
        gather_logits<8>(partial, S, T, t, E, router_b, v, between);
        select_routes<8>(v, rs, t, E, k, sel, val);
    }
}

// Expert blob of route r, selected by the calling wavefront itself (top-k of
// the token's logits), and the route's weight (1 for the shared expert;
// `need_weight` false: not made). `publish` (wave-uniform) writes the token's
// experts and route weights to idx / wts and the exports. `between`: the
// caller's loads, issued behind the router partials' (for the shared
// expert, at once).
template <bool SMALL_E, typename Between>
__device__ __forceinline__ const uint8_t *route_blob(const DecodeArgs &a, int r, bool publish,
                                                     bool need_weight, float &weight,
                                                     Between &&between) {
    const int R = a.T * a.k;
    weight = 1.0f;
    if (r >= R) {
        between();
        return a.sh.base;
    }
    const int lane = threadIdx.x & 63;
    const int t = r / a.k, j = r - t * a.k;
    int sel[kMaxK];
    double val[kMaxK];
    route_token<SMALL_E>(a.partial, a.S, a.router_b, a.rs, a.T, t, a.E, a.k, sel, val, between);
    int mine = sel[0];
#pragma unroll
    for (int jj = 1; jj < kMaxK; ++jj)
        if (jj == j) mine = sel[jj];
    mine = __builtin_amdgcn_readfirstlane(mine);  // equal in every lane; lets loads take a scalar base
    if (need_weight || publish) {  // wave-uniform: only the epilogue's wavefront needs it
        // lane jj takes slot jj's logit and expert; one exponential per lane
        double v = val[0];
        int e = sel[0];
#pragma unroll
        for (int jj = 1; jj < kMaxK; ++jj) {
            if (lane == jj) {
                v = val[jj];
                e = sel[jj];
            }
        }
        const float wl = route_weight_lanes(v, a.k, a.route_scale);
        weight = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), j));
        if (publish && lane < a.k) {
            a.idx[t * a.k + lane] = e;
            a.wts[t * a.k + lane] = wl;
            if (a.out_idx) a.out_idx[t * a.k + lane] = e;
            if (a.out_w) a.out_w[t * a.k + lane] = wl;
            // route profile (goosedump ExpertRouteProfile::record): one per selection
            if (a.route_counts)
                atomicAdd(reinterpret_cast<unsigned long long *>(a.route_counts + e), 1ull);
        }
    }
    return a.ex.base + static_cast<size_t>(mine) * a.ex.stride;
}

// gate/up + biases + clamped SwiGLU, times the route weight, for 32 features
// (block fb) of route r; writes the activation block's FP8 terms and scales (blocks past F write the
// zero padding of the down GEMV's operand). out[t] already holds the residual
// (seeded by the router launch's quantisation), so nothing here delays the
// router-partials load and the top-k. s_part: kDecodeWaves * 4 * 16 floats of
// LDS.
template <int SPW, int CH, bool SMALL_E>
__device__ __forceinline__ void gate_up_item(const DecodeArgs &a, int r, int fb, float *s_part,
                                             uint8_t *lds) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int R = a.T * a.k;
    const int t = r < R ? r / a.k : r - R;
    const int j = r < R ? r - t * a.k : -1;
    const int H = a.H, F = a.F;
    const int Kp = pad128(H), Fp = pad128(F), nbp = Fp / 32;
    uint8_t *aq = a.act_q + static_cast<size_t>(r) * kTerms * Fp;
    uint8_t *as = a.act_s + static_cast<size_t>(r) * kTerms * nbp;
    if (32 * fb >= F) {  // K padding of the down GEMV's operand: zero codes, by wavefront 0
        if (w == 0) {
            for (int e = lane; e < 32 * kTerms; e += 64) {
                const int n = e >> 5, i = e & 31;
                aq[n * Fp + 32 * fb + i] = 0;
                if (i == 0) as[n * nbp + fb] = 127;
            }
        }
        return;
    }
    // the token's input terms, staged through LDS by the whole workgroup;
    // their loads go out behind the router partials', so the top-k waits only
    // for the partials
    const Staged sg{Kp, kTerms};
    dec_u32x4 stv[CH];
    uint32_t stsv = 0;
    auto stage_loads = [&]() __attribute__((always_inline)) {
        const int tid = threadIdx.x, nthr = kDecodeWaves * 64;
        const int cq = kTerms * (Kp / 16), cs = kTerms * (Kp / 128);
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c = min(tid + nthr * i, cq - 1);
            stv[i] = *reinterpret_cast<const dec_u32x4 *>(a.xq + stage_code_src(sg, c, kTerms, t * kTerms, 0));
        }
        stsv = *reinterpret_cast<const uint32_t *>(a.xs + stage_scale_src(sg, min(tid, cs - 1), kTerms,
                                                                            t * kTerms, 0));
    };
    float route_w;
    const uint8_t *blob =
        route_blob<SMALL_E>(a, r, j == 0 && fb == 0 && w == 0, w == 0, route_w, stage_loads);
    // the epilogue's biases, loaded with the weights
    const int fe = 32 * fb + (lane & 31);
    const float bias_g = reinterpret_cast<const float *>(blob + a.ex.gate_b)[fe];
    const float bias_u = reinterpret_cast<const float *>(blob + a.ex.up_b)[fe];
    const int NS = Kp / 128, nblk = H / 32;
    // the four 16-row tiles: gate rows 32 fb.., 32 fb + 16.., then up
    const uint8_t *tq[4], *ts[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int tile = 2 * fb + (m & 1);
        tq[m] = blob + (m < 2 ? a.ex.gate_q : a.ex.up_q) + tile_code_base(tile, nblk);
        ts[m] = blob + (m < 2 ? a.ex.gate_s : a.ex.up_s) + tile_scale_base(tile, nblk);
    }
    const ALane al(nblk, lane);
    const int bn = lane & 15, bh = lane >> 4;
    const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
    const int wu = __builtin_amdgcn_readfirstlane(w);

    f32x4_t acc[4];  // gate tile 0, gate tile 1, up tile 0, up tile 1
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // rounds of SPW steps (one round unless K > 4096); every wavefront runs
    // the first round, whose weight loads go out before the staged terms are
    // stored and the workgroup barrier
    int s0 = wu * SPW;
    AFrag af[SPW][4];
#pragma unroll
    for (int i = 0; i < SPW; ++i)
#pragma unroll
        for (int m = 0; m < 4; ++m) af[i][m] = load_afrag(tq[m], ts[m], al, min(s0 + i, NS - 1));
    __builtin_amdgcn_sched_barrier(0);
    {
        const int tid = threadIdx.x, nthr = kDecodeWaves * 64;
        const int cq = kTerms * (Kp / 16), cs = kTerms * (Kp / 128);
#pragma unroll
        for (int i = 0; i < CH; ++i)
            *reinterpret_cast<dec_u32x4 *>(lds + stage_code_dst(sg, min(tid + nthr * i, cq - 1))) = stv[i];
        *reinterpret_cast<uint32_t *>(lds + sg.scale_off() + 4 * min(tid, cs - 1)) = stsv;
        if (tid < 4) reinterpret_cast<uint4 *>(lds + sg.zero_off())[tid] = make_uint4(0u, 0u, 0u, 0u);
        __syncthreads();
    }
    while (true) {
        // a step past K runs with a zero B operand
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            const BFrag b = lds_bfrag(lds, sg, 0, min(s0 + i, NS - 1), bn, bh);
            const bool on = s0 + i < NS;
            const uint4 blo = on ? b.lo : zero, bhi = on ? b.hi : zero;
#pragma unroll
            for (int m = 0; m < 4; ++m) acc[m] = mx_mfma(af[i][m], blo, bhi, b.s, acc[m]);
        }
        s0 += kDecodeWaves * SPW;
        if (s0 >= NS) break;
#pragma unroll
        for (int i = 0; i < SPW; ++i)
#pragma unroll
            for (int m = 0; m < 4; ++m) af[i][m] = load_afrag(tq[m], ts[m], al, min(s0 + i, NS - 1));
    }

#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[m][v] = quad_sum(acc[m][v]);
    if (bn == 0) {
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int v = 0; v < 4; ++v) s_part[(w * 4 + m) * 16 + 4 * bh + v] = acc[m][v];
    }
    __syncthreads();
    if (w == 0) {  // both half-waves hold the block; lanes 0..31 store it
        const int i = lane & 31, tile = i >> 4, row = i & 15;
        const int f = 32 * fb + i;
        float g = 0.f, u = 0.f;
#pragma unroll
        for (int ww = 0; ww < kDecodeWaves; ++ww) {
            g += s_part[(ww * 4 + tile) * 16 + row];
            u += s_part[(ww * 4 + 2 + tile) * 16 + row];
        }
        // times the route weight: down then sums the routes' products directly
        const float act =
            route_w * swiglu(g + bias_g, u + bias_u, a.sc.alpha, a.sc.limit, a.sc.up_offset);
        uint32_t codes, scales;
        fp8_terms_group(act, codes, scales);
        if (lane < 32) {
#pragma unroll
            for (int n = 0; n < kTerms; ++n) {
                aq[n * Fp + f] = static_cast<uint8_t>(codes >> (8 * n));
                if (lane == 0) as[n * nbp + fb] = static_cast<uint8_t>(scales >> (8 * n));
            }
        }
    }
}

// down for rows 16 hb .. 16 hb + 15 of token t: the sum over the token's
// routes j (slots 0..k-1, then the shared expert) of W_j . act_j, where act_j
// already carries the route weight, plus sum_j w_j * bias_j, added to the
// residual (which the router launch seeded into out). The NF = routes x
// K-steps fragments are dealt to the W wavefronts in rounds of SPF: wavefront
// w takes fragments w * SPF .. w * SPF + SPF - 1, then W * SPF further on;
// fragment f is route f / NS, step f % NS. A fragment past NF runs with a
// zero B operand. CH > 0: the token's activation terms are staged through
// LDS (CH 16-byte chunks per thread; every wavefront runs the first round,
// whose weight loads go out before the staged terms are stored and the
// workgroup barrier); CH = 0: each fragment's terms load directly.
template <int W, int SPF, int CH>
__device__ __forceinline__ void down_rows(const DecodeArgs &a, int t, int hb, float *s_part,
                                          uint8_t *lds) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int H = a.H, F = a.F, k = a.k, R = a.T * a.k;
    const int nr = k + a.n_shared;                    // routes of the token
    const int Fp = pad128(F), NS = Fp / 128, nblk = F / 32;
    const int NF = nr * NS;
    // staged rows: route j's terms come from act row t * k + j (the shared
    // expert's from row T * k + t)
    const Staged sg{Fp, nr * kTerms};
    constexpr int CHR = CH > 0 ? CH : 1;
    dec_u32x4 stv[CHR];
    uint32_t stsv = 0;
    if constexpr (CH > 0) {
        // the routed rows t*k .. t*k+k-1 (k * kTerms term rows), then the shared row
        const int tid = threadIdx.x, nthr = W * 64;
        const int cq = sg.nq * (Fp / 16), cs = sg.nq * (Fp / 128);
        const int ra = t * k * kTerms, rb = (R + t) * kTerms;
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c = min(tid + nthr * i, cq - 1);
            stv[i] = *reinterpret_cast<const dec_u32x4 *>(a.act_q + stage_code_src(sg, c, k * kTerms, ra, rb));
        }
        stsv = *reinterpret_cast<const uint32_t *>(a.act_s + stage_scale_src(sg, min(tid, cs - 1),
                                                                             k * kTerms, ra, rb));
    }
    // lane j loads slot j's expert and weight (one vector load each), then
    // every slot moves to scalar registers with readlane: no branch, no chain
    // (the staged terms' loads go first: measured faster than behind the
    // weights)
    const int lj = min(lane, k - 1);
    const int ev = a.idx[t * k + lj];
    const float wv = a.wts[t * k + lj];
    // blob of slot j (uniform j): its expert comes from lane j by readlane
    // (an array of pointers indexed at run time would leave the registers)
    auto slot_blob = [&](int j) __attribute__((always_inline)) {
        const int e = __builtin_amdgcn_readlane(ev, min(j, k - 1));
        return j < k ? a.ex.base + static_cast<size_t>(e) * a.ex.stride : a.sh.base;
    };
    // this lane's output row, the routes' weights and biases for it and its
    // residual (the epilogue's operands, read ahead of the tail)
    const int h = 16 * hb + (lane & 15);
    float rwt[kMaxK + 1], rbias[kMaxK + 1];
#pragma unroll
    for (int j = 0; j < kMaxK + 1; ++j) {
        const int jb = min(j, nr - 1);
        const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wv), min(j, k - 1)));
        rwt[j] = j < k ? wj : 1.0f;
        rbias[j] = reinterpret_cast<const float *>(slot_blob(jb) + a.ex.down_b)[h];
    }
    float *o = a.out + static_cast<size_t>(t) * H + h;
    const float resid = *o;
    const ALane al(nblk, lane);
    const int wu = __builtin_amdgcn_readfirstlane(w);
    const int bn = lane & 15, bh = lane >> 4;
    const int nn = min(bn, kTerms - 1);
    const bool bon = bn < kTerms;
    const uint64_t tcb = tile_code_base(hb, nblk), tsb = tile_scale_base(hb, nblk);
    const uint32_t nrows = static_cast<uint32_t>(R + a.T * a.n_shared);
    const TermRows tr = term_rows(a.act_q, a.act_s, nrows * kTerms * Fp, nrows * kTerms * (Fp / 32));
    (void)tr;
    (void)nn;

    f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
    int f0 = wu * SPF;
    AFrag af[SPF];
    BFrag b[SPF];
    int fj[SPF], fs[SPF];
    auto frags = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < SPF; ++i) {
            const int f = min(f0 + i, NF - 1);
            fj[i] = f / NS;
            fs[i] = f - fj[i] * NS;
        }
    };
    auto load_a = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < SPF; ++i) {
            const uint8_t *blob = slot_blob(fj[i]);
            af[i] = load_afrag(blob + a.ex.down_q + tcb, blob + a.ex.down_s + tsb, al, fs[i]);
        }
    };
    auto load_b_direct = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < SPF; ++i) {
            const int r = fj[i] < k ? t * k + fj[i] : R + t;  // act rows: routes, then shared
            b[i] = load_bfrag_buf(tr, (static_cast<uint32_t>(r) * kTerms + nn) * Fp,
                                  (static_cast<uint32_t>(r) * kTerms + nn) * (Fp / 32), fs[i], bh,
                                  bon && f0 + i < NF);
        }
    };
    auto mma = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < SPF; ++i) {
            if constexpr (CH > 0) {
                // one fragment's B read at a time (the reads hoisted together
                // would hold every fragment's operand in registers)
                const BFrag bl = lds_bfrag(lds, sg, fj[i] * kTerms, fs[i], bn, bh);
                const bool on = f0 + i < NF;
                const uint4 z = make_uint4(0u, 0u, 0u, 0u);
                acc = mx_mfma(af[i], on ? bl.lo : z, on ? bl.hi : z, bl.s, acc);
                __builtin_amdgcn_sched_barrier(0);
            } else {
                acc = mx_mfma(af[i], b[i], acc);  // zero where no term or past the fragments
            }
        }
    };
    frags();
    if constexpr (CH == 0) load_b_direct();
    __builtin_amdgcn_sched_barrier(0);
    load_a();
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (CH > 0) {
        const int tid = threadIdx.x, nthr = W * 64;
        const int cq = sg.nq * (Fp / 16), cs = sg.nq * (Fp / 128);
#pragma unroll
        for (int i = 0; i < CH; ++i)
            *reinterpret_cast<dec_u32x4 *>(lds + stage_code_dst(sg, min(tid + nthr * i, cq - 1))) = stv[i];
        *reinterpret_cast<uint32_t *>(lds + sg.scale_off() + 4 * min(tid, cs - 1)) = stsv;
        if (tid < 4) reinterpret_cast<uint4 *>(lds + sg.zero_off())[tid] = make_uint4(0u, 0u, 0u, 0u);
        __syncthreads();
    }
    while (true) {
        mma();
        f0 += W * SPF;
        if (f0 >= NF) break;
        frags();
        if constexpr (CH == 0) load_b_direct();
        __builtin_amdgcn_sched_barrier(0);
        load_a();
        __builtin_amdgcn_sched_barrier(0);
    }

#pragma unroll
    for (int v = 0; v < 4; ++v) acc[v] = quad_sum(acc[v]);
    if (bn == 0) {
#pragma unroll
        for (int v = 0; v < 4; ++v) s_part[w * 16 + 4 * bh + v] = acc[v];
    }
    __syncthreads();
    if (w == 0 && lane < 16) {
        float y = 0.f;
#pragma unroll
        for (int ww = 0; ww < W; ++ww) y += s_part[ww * 16 + lane];
        float bias_sum = 0.f;  // route-weighted biases in slot order, then the shared expert
#pragma unroll
        for (int j = 0; j < kMaxK + 1; ++j)
            if (j < nr) bias_sum = fmaf(rwt[j], rbias[j], bias_sum);
        *o = resid + (y + bias_sum);
    }
}

// grid.x = 32-wide feature blocks of pad128(F), grid.y = routes: consecutive
// workgroups (dealt round-robin over the dies) take blocks of one route, so
// every route's weights stream through all eight dies (0.8% faster per decode
// token than routes along x, which put each route on two dies)
template <int SPW, int CH, bool SMALL_E>
__global__ __launch_bounds__(kDecodeWaves * 64) void decode_gate_up_kernel(DecodeArgs a) {
    __shared__ float s_part[kDecodeWaves * 4 * 16];
    extern __shared__ __align__(16) uint8_t dyn_lds[];
    gate_up_item<SPW, CH, SMALL_E>(a, blockIdx.y, blockIdx.x, s_part, dyn_lds);
}

// grid.x = 16-row blocks of H, grid.y = tokens.
template <int W, int SPF, int CH>
__global__ __launch_bounds__(W * 64) void decode_down_kernel(DecodeArgs a) {
    __shared__ float s_part[W * 16];
    extern __shared__ __align__(16) uint8_t dyn_lds[];
    down_rows<W, SPF, CH>(a, blockIdx.y, blockIdx.x, s_part, dyn_lds);
}

// K-steps per wavefront per round (rounds repeat past 8 * 4 steps, K > 4096).
int decode_spw(int K) {
    const int ns = pad128(K) / 128;
    const int spw = (ns + kDecodeWaves - 1) / kDecodeWaves;
    return spw < 1 ? 1 : (spw > 4 ? 4 : spw);
}

}  // namespace

hipError_t launch_decode_gate_up(const DecodeArgs &a, hipStream_t s) {
    const dim3 grid(pad128(a.F) / 32, a.T * (a.k + a.n_shared));
    const dim3 block(kDecodeWaves * 64);
    const int Kp = pad128(a.H);
    const int ch = (Kp / 4 + kDecodeWaves * 64 - 1) / (kDecodeWaves * 64);  // 16-byte chunks per thread
    const size_t shm = staged_bytes(Kp, kTerms);
#define MOE_GU_DEC(SPW, CH)                                                                          \
    do {                                                                                             \
        if (a.E <= 128) launch_kernel_shm(decode_gate_up_kernel<SPW, CH, true>, grid, block, shm, s, a); \
        else launch_kernel_shm(decode_gate_up_kernel<SPW, CH, false>, grid, block, shm, s, a);         \
    } while (0)
    switch (decode_spw(a.H)) {  // K <= 1024: one chunk; <= 2048: one; <= 3072: two; else two or four
    case 1: MOE_GU_DEC(1, 1); break;
    case 2: MOE_GU_DEC(2, 1); break;
    case 3: MOE_GU_DEC(3, 2); break;
    default:
        if (ch <= 2) MOE_GU_DEC(4, 2);
        else MOE_GU_DEC(4, 4);
        break;
    }
#undef MOE_GU_DEC
    return hipGetLastError();
}

// A token's activation terms are staged through LDS when they fit this many bytes.
constexpr int kDownStageMax = 64 * 1024;

hipError_t launch_decode_down(const DecodeArgs &a, hipStream_t s) {
    const dim3 grid(a.H / 16, a.T);
    const int nr = a.k + a.n_shared, Fp = pad128(a.F);
    // fragments per wavefront and round: the token's routes x K-steps over
    // the wavefronts, at most 12 per round
    const int nf = nr * (Fp / 128);
    const int per = (nf + kDecodeWaves - 1) / kDecodeWaves;
    const dim3 block(kDecodeWaves * 64);
    const size_t shm = staged_bytes(Fp, nr * kTerms);
    const int ch = (nr * kTerms * Fp / 16 + kDecodeWaves * 64 - 1) / (kDecodeWaves * 64);
    constexpr int DW = kDecodeWaves;
#define MOE_DOWN(SPF)                                                                               \
    do {                                                                                            \
        if (shm > kDownStageMax) launch_kernel(decode_down_kernel<DW, SPF, 0>, grid, block, s, a);  \
        else if (ch <= 4) launch_kernel_shm(decode_down_kernel<DW, SPF, 4>, grid, block, shm, s, a); \
        else launch_kernel_shm(decode_down_kernel<DW, SPF, 8>, grid, block, shm, s, a);             \
    } while (0)
    if (per <= 4) MOE_DOWN(4);
    else if (per <= 8) MOE_DOWN(8);
    else MOE_DOWN(12);
#undef MOE_DOWN
    return hipGetLastError();
}

}  // namespace moe
