// Decode (T <= 64): per route, GEMVs over the selected expert's MXFP4 planes
// on the block-scaled matrix cores, after the router launch: gate/up over
// (route, feature block), then down over (route, 32-row block of H).
//
// A work item is 32 weight rows (two 16-row tiles) of one route, for one
// workgroup; its 8 wavefronts split K into 128-wide steps. Every wavefront
// issues all of its loads (B first, then the weight tiles from a scalar base)
// before its first matrix-core instruction, with no branch in between, so
// each instruction waits only for its own operands. Weight tiles are read as
// whole contiguous kilobytes (the blob's tiled plane layout). The expert input
// arrives as FP8 terms in B columns 0..kTerms-1; the other 12 columns are
// zero, which costs nothing here: the GEMV is bound by weight bytes.
//
// Page: goosedump `gpt_oss.rs`, `mixture_of_experts` (gate/up pair with
// biases, clamped SwiGLU, down with bias, route weight, slot sum into the
// residual).
#include "mx_mfma.hpp"

namespace moe {

namespace {

// Top-k of token t's router logits (fp64 split-K partials + bias) by one
// wavefront: the selected experts and their logits, in every lane.
__device__ __forceinline__ void route_token(const double *partial, int S, const float *router_b,
                                            int T, int t, int E, int k, int (&sel)[kMaxK],
                                            double (&val)[kMaxK]) {
    double v[kMaxQ];
    if (E <= 64) {
        gather_logits<1>(partial, S, T, t, E, router_b, v);
        wave_topk<1>(v, E, k, sel, val);
    } else if (E <= 128) {
        gather_logits<2>(partial, S, T, t, E, router_b, v);
        wave_topk<2>(v, E, k, sel, val);
    } else if (E <= 256) {
        gather_logits<4>(partial, S, T, t, E, router_b, v);
        wave_topk<4>(v, E, k, sel, val);
    } else {
        gather_logits<8>(partial, S, T, t, E, router_b, v);
        wave_topk<8>(v, E, k, sel, val);
    }
}

// Expert blob of route r, selected by the calling wavefront itself (top-k of
// the token's logits). `publish` (wave-uniform) writes the token's experts
// and route weights to idx / wts and the exports.
__device__ __forceinline__ const uint8_t *route_blob(const DecodeArgs &a, int r, bool publish) {
    const int R = a.T * a.k;
    if (r >= R) return a.sh.base;
    const int lane = threadIdx.x & 63;
    const int t = r / a.k, j = r - t * a.k;
    int sel[kMaxK];
    double val[kMaxK];
    route_token(a.partial, a.S, a.router_b, a.T, t, a.E, a.k, sel, val);
    int mine = sel[0];
#pragma unroll
    for (int jj = 1; jj < kMaxK; ++jj)
        if (jj == j) mine = sel[jj];
    mine = __builtin_amdgcn_readfirstlane(mine);  // equal in every lane; lets loads take a scalar base
    if (publish) {
        float wv[kMaxK];
        route_softmax(val, a.k, a.route_scale, wv);
#pragma unroll
        for (int jj = 0; jj < kMaxK; ++jj) {
            if (jj < a.k && lane == jj) {
                a.idx[t * a.k + jj] = sel[jj];
                a.wts[t * a.k + jj] = wv[jj];
                if (a.out_idx) a.out_idx[t * a.k + jj] = sel[jj];
                if (a.out_w) a.out_w[t * a.k + jj] = wv[jj];
                // route profile (goosedump ExpertRouteProfile::record): one per selection
                if (a.route_counts)
                    atomicAdd(reinterpret_cast<unsigned long long *>(a.route_counts + sel[jj]), 1ull);
            }
        }
    }
    return a.ex.base + static_cast<size_t>(mine) * a.ex.stride;
}

// gate/up + biases + clamped SwiGLU for 32 features (block fb) of route r;
// writes the activation block's FP8 terms and scales (blocks past F write the
// zero padding of the down GEMV's operand). out[t] already holds the residual
// (seeded by the router launch's quantisation), so nothing here delays the
// router-partials load and the top-k. s_part: kDecodeWaves * 4 * 16 floats of
// LDS.
template <int SPW>
__device__ __forceinline__ void gate_up_item(const DecodeArgs &a, int r, int fb, float *s_part) {
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
    const uint8_t *blob = route_blob(a, r, j == 0 && fb == 0 && w == 0);
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
    const int nn = min(bn, kTerms - 1);
    const bool bon = bn < kTerms;
    const uint8_t *xrow = a.xq + (static_cast<size_t>(t) * kTerms + nn) * Kp;
    const uint8_t *srow = a.xs + (static_cast<size_t>(t) * kTerms + nn) * (Kp / 32);
    const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
    const int wu = __builtin_amdgcn_readfirstlane(w);

    f32x4_t acc[4];  // gate tile 0, gate tile 1, up tile 0, up tile 1
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int s0 = wu * SPW; s0 < NS; s0 += kDecodeWaves * SPW) {  // one round unless K > 4096
        AFrag af[SPW][4];
        BFrag b[SPW];
        // B (small, cached) first, then every weight load: the memory counter
        // retires in order, so the first instruction waits only for its own data
#pragma unroll
        for (int i = 0; i < SPW; ++i) b[i] = load_bfrag(xrow, srow, min(s0 + i, NS - 1), bh);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < SPW; ++i)
#pragma unroll
            for (int m = 0; m < 4; ++m) af[i][m] = load_afrag(tq[m], ts[m], al, min(s0 + i, NS - 1));
        __builtin_amdgcn_sched_barrier(0);
        // no branch between the loads and the matrix-core instructions (a
        // branch there makes the compiler drain the loads step by step): a
        // step past K runs with a zero B operand
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            const bool on = bon && s0 + i < NS;
            const uint4 blo = on ? b[i].lo : zero, bhi = on ? b[i].hi : zero;
#pragma unroll
            for (int m = 0; m < 4; ++m) acc[m] = mx_mfma(af[i][m], blo, bhi, b[i].s, acc[m]);
        }
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
        const float act = swiglu(g + bias_g, u + bias_u, a.sc.alpha, a.sc.limit, a.sc.up_offset);
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

// down + bias, times the route weight, added into out[t] (which already holds
// the residual) for rows 32 hb .. 32 hb + 31 of route r; the expert and the
// weight come from idx / wts. s_part: kDecodeWaves * 2 * 16 floats of LDS.
template <int SPW>
__device__ __forceinline__ void down_item(const DecodeArgs &a, int r, int hb, float *s_part) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int R = a.T * a.k;
    const int t = r < R ? r / a.k : r - R;
    const int H = a.H, F = a.F;
    const uint8_t *blob = r < R ? a.ex.base + static_cast<size_t>(a.idx[r]) * a.ex.stride : a.sh.base;
    const float wt = r < R ? a.wts[r] : 1.0f;
    const float bias = reinterpret_cast<const float *>(blob + a.ex.down_b)[32 * hb + (lane & 31)];
    const int Fp = pad128(F), NS = Fp / 128, nblk = F / 32;
    const uint8_t *tq[2], *ts[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        tq[m] = blob + a.ex.down_q + tile_code_base(2 * hb + m, nblk);
        ts[m] = blob + a.ex.down_s + tile_scale_base(2 * hb + m, nblk);
    }
    const ALane al(nblk, lane);
    const int wu = __builtin_amdgcn_readfirstlane(w);
    const int bn = lane & 15, bh = lane >> 4;
    const int nn = min(bn, kTerms - 1);
    const bool bon = bn < kTerms;
    const uint8_t *xrow = a.act_q + (static_cast<size_t>(r) * kTerms + nn) * Fp;
    const uint8_t *srow = a.act_s + (static_cast<size_t>(r) * kTerms + nn) * (Fp / 32);
    const uint4 zero = make_uint4(0u, 0u, 0u, 0u);

    f32x4_t acc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
    for (int s0 = wu * SPW; s0 < NS; s0 += kDecodeWaves * SPW) {  // one round unless K > 4096
        AFrag af[SPW][2];
        BFrag b[SPW];
        // B (small, cached) first, then every weight load
#pragma unroll
        for (int i = 0; i < SPW; ++i) b[i] = load_bfrag(xrow, srow, min(s0 + i, NS - 1), bh);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            af[i][0] = load_afrag(tq[0], ts[0], al, min(s0 + i, NS - 1));
            af[i][1] = load_afrag(tq[1], ts[1], al, min(s0 + i, NS - 1));
        }
        __builtin_amdgcn_sched_barrier(0);
        // branch-free as in gate/up: a step past K runs with a zero B operand
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            const bool on = bon && s0 + i < NS;
            const uint4 blo = on ? b[i].lo : zero, bhi = on ? b[i].hi : zero;
            acc[0] = mx_mfma(af[i][0], blo, bhi, b[i].s, acc[0]);
            acc[1] = mx_mfma(af[i][1], blo, bhi, b[i].s, acc[1]);
        }
    }

#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[m][v] = quad_sum(acc[m][v]);
    if (bn == 0) {
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int v = 0; v < 4; ++v) s_part[(w * 2 + m) * 16 + 4 * bh + v] = acc[m][v];
    }
    __syncthreads();
    if (threadIdx.x < 32) {
        const int i = threadIdx.x, h = 32 * hb + i;
        float y = 0.f;
#pragma unroll
        for (int ww = 0; ww < kDecodeWaves; ++ww) y += s_part[(ww * 2 + (i >> 4)) * 16 + (i & 15)];
        unsafeAtomicAdd(a.out + static_cast<size_t>(t) * H + h, wt * (y + bias));
    }
}

// grid.x = 32-wide feature blocks of pad128(F), grid.y = routes: consecutive
// workgroups (dealt round-robin over the dies) take blocks of one route, so
// every route's weights stream through all eight dies (0.8% faster per decode
// token than routes along x, which put each route on two dies)
template <int SPW>
__global__ __launch_bounds__(kDecodeWaves * 64) void decode_gate_up_kernel(DecodeArgs a) {
    __shared__ float s_part[kDecodeWaves * 4 * 16];
    gate_up_item<SPW>(a, blockIdx.y, blockIdx.x, s_part);
}

// grid.x = 32-row blocks of H, grid.y = routes (as for gate/up).
template <int SPW>
__global__ __launch_bounds__(kDecodeWaves * 64) void decode_down_kernel(DecodeArgs a) {
    __shared__ float s_part[kDecodeWaves * 2 * 16];
    down_item<SPW>(a, blockIdx.y, blockIdx.x, s_part);
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
    switch (decode_spw(a.H)) {
    case 1: launch_kernel(decode_gate_up_kernel<1>, grid, block, s, a); break;
    case 2: launch_kernel(decode_gate_up_kernel<2>, grid, block, s, a); break;
    case 3: launch_kernel(decode_gate_up_kernel<3>, grid, block, s, a); break;
    default: launch_kernel(decode_gate_up_kernel<4>, grid, block, s, a); break;
    }
    return hipGetLastError();
}

hipError_t launch_decode_down(const DecodeArgs &a, hipStream_t s) {
    const dim3 grid(a.H / 32, a.T * (a.k + a.n_shared));
    const dim3 block(kDecodeWaves * 64);
    switch (decode_spw(a.F)) {
    case 1: launch_kernel(decode_down_kernel<1>, grid, block, s, a); break;
    case 2: launch_kernel(decode_down_kernel<2>, grid, block, s, a); break;
    case 3: launch_kernel(decode_down_kernel<3>, grid, block, s, a); break;
    default: launch_kernel(decode_down_kernel<4>, grid, block, s, a); break;
    }
    return hipGetLastError();
}

}  // namespace moe
