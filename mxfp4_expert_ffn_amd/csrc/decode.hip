// Decode path (few tokens): GEMV kernels that stream only the k selected
// experts' MXFP4 bytes with 128-bit loads.
//
// Page: goosedump `gpt_oss.rs` `mixture_of_experts`: per selected expert a
// gate/up matrix-vector pair on the same input, both biases, the clamped
// SwiGLU, the down matrix-vector product, the down bias, the route weight,
// and a slot-by-slot sum added to the residual.
//
// Lane mapping: in a row of K weights (K/32 MX blocks of 16 code bytes and
// one scale byte), lane l always takes blocks l, l+64, l+128, ... so the 32
// activations of each of its blocks are read once (from the workgroup's LDS
// copy) into registers and reused for every row the wavefront streams. A row
// sum is then one DPP reduction.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kMaxBlocks = 8192 / 32;  // MX blocks per row (K <= 8192)

// Stage a length-K vector (fp32 or bf16 bits) in LDS as float32, transposed
// to [32][K/32 + 1] so that lane l reading element i of block l hits
// consecutive addresses.
template <bool BF16>
__device__ __forceinline__ void stage_vec(const void *src, int K, float (*sv)[kMaxBlocks + 1]) {
    for (int i4 = threadIdx.x; i4 < K / 4; i4 += blockDim.x) {
        float v[4];
        if constexpr (BF16) {
            const uint2 u = reinterpret_cast<const uint2 *>(src)[i4];
            v[0] = __uint_as_float(u.x << 16); v[1] = __uint_as_float(u.x & 0xffff0000u);
            v[2] = __uint_as_float(u.y << 16); v[3] = __uint_as_float(u.y & 0xffff0000u);
        } else {
            const float4 f = reinterpret_cast<const float4 *>(src)[i4];
            v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
        }
        const int h = 4 * i4, b = h >> 5, i = h & 31;
#pragma unroll
        for (int j = 0; j < 4; ++j) sv[i + j][b] = v[j];
    }
}

// Lane l's blocks l, l+64, ... of the staged vector into registers.
template <int NB>
__device__ __forceinline__ void lane_blocks(const float (*sv)[kMaxBlocks + 1], int K, float (&v)[NB][32]) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int c = 0; c < NB; ++c) {
        const int b = lane + 64 * c;
#pragma unroll
        for (int i = 0; i < 32; ++i) v[c][i] = b < K / 32 ? sv[i][b] : 0.f;
    }
}

// gate/up GEMV + biases + clamped SwiGLU. grid.x = routes (T*k routed, then
// T*n_shared shared rows), grid.y = blocks of kDecodeRowsGU expert rows.
// Wavefront 0 recomputes the token's top-k from the router partials (every
// workgroup of a route agrees: same inputs, same order) while the others
// stage the activation row in LDS. Workgroups of slot 0 also seed out[t]
// with the residual, which the down kernel then accumulates into.
template <int NB, bool BF16>
__global__ __launch_bounds__(256) void decode_gate_up_kernel(
    const void *x, const double *partial, int S, const float *router_b, int T, int H, int F,
    int E, int k, float route_scale, ExpertPtrs ex, ExpertPtrs sh, SwigluConsts sc, int32_t *idx,
    float *wts, int32_t *out_idx, float *out_w, const void *resid, int resid_bf16, float *out,
    float *act) {
    constexpr int RPW = kDecodeRowsGU / 4;  // rows per wavefront
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int r = blockIdx.x, R = T * k;
    __shared__ int s_expert;
    __shared__ float s_x[32][kMaxBlocks + 1];
    const int t = r < R ? r / k : r - R;
    const int j = r < R ? r - t * k : -1;
    const void *xt = BF16 ? static_cast<const void *>(static_cast<const uint16_t *>(x) + static_cast<size_t>(t) * H)
                          : static_cast<const void *>(static_cast<const float *>(x) + static_cast<size_t>(t) * H);
    if (r < R && w == 0) {
        double v[4];
        if (E <= 64) gather_logits<1>(partial, S, T, t, E, router_b, v);
        else if (E <= 128) gather_logits<2>(partial, S, T, t, E, router_b, v);
        else gather_logits<4>(partial, S, T, t, E, router_b, v);
        int sel[kMaxK];
        double val[kMaxK];
        wave_topk(v, E, k, sel, val);
        int mine = sel[0];
#pragma unroll
        for (int jj = 1; jj < kMaxK; ++jj)
            if (jj == j) mine = sel[jj];
        if (lane == 0) s_expert = mine;
        if (j == 0 && blockIdx.y == 0) {
            float wv[kMaxK];
            route_softmax(val, k, route_scale, wv);
#pragma unroll
            for (int jj = 0; jj < kMaxK; ++jj) {
                if (jj < k && lane == jj) {
                    idx[t * k + jj] = sel[jj];
                    wts[t * k + jj] = wv[jj];
                    if (out_idx) out_idx[t * k + jj] = sel[jj];
                    if (out_w) out_w[t * k + jj] = wv[jj];
                }
            }
        }
    }
    stage_vec<BF16>(xt, H, s_x);
    float *o = out + static_cast<size_t>(t) * H;
    const float *rf = static_cast<const float *>(resid) + static_cast<size_t>(t) * H;
    if (j == 0 && (resid_bf16 || o != rf)) {
        // residual seed: this workgroup's share of out[t]
        const uint16_t *rb = static_cast<const uint16_t *>(resid) + static_cast<size_t>(t) * H;
        const int share = (H + gridDim.y - 1) / gridDim.y;
        const int h0 = blockIdx.y * share;
        for (int h = h0 + threadIdx.x; h < min(H, h0 + share); h += blockDim.x)
            o[h] = resid_bf16 ? bf16_bits_to_f32(rb[h]) : rf[h];
    }
    __syncthreads();
    const uint8_t *blob = r < R ? ex.base + static_cast<size_t>(s_expert) * ex.stride : sh.base;

    const int nblk = H / 32;
    const int f0 = blockIdx.y * kDecodeRowsGU + w * RPW;
    const uint8_t *gq = blob + ex.gate_q, *uq = blob + ex.up_q;
    const uint8_t *gs = blob + ex.gate_s, *us = blob + ex.up_s;
    const float *gb = reinterpret_cast<const float *>(blob + ex.gate_b);
    const float *ub = reinterpret_cast<const float *>(blob + ex.up_b);

    // Every load is unconditional (clamped to a valid row/block) so that all of
    // them are in flight together; out-of-range rows are never stored and
    // out-of-range blocks meet zero activations.
    uint4 qg[RPW][NB], qu[RPW][NB];
    uint32_t sg[RPW][NB], su[RPW][NB];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const int f = min(f0 + i, F - 1);
#pragma unroll
        for (int c = 0; c < NB; ++c) {
            const int b = min(lane + 64 * c, nblk - 1);
            const size_t qo = static_cast<size_t>(f) * (H / 2) + 16 * b;
            const size_t so = static_cast<size_t>(f) * nblk + b;
            qg[i][c] = *reinterpret_cast<const uint4 *>(gq + qo);
            qu[i][c] = *reinterpret_cast<const uint4 *>(uq + qo);
            sg[i][c] = gs[so];
            su[i][c] = us[so];
        }
    }
    float xv[NB][32];
    lane_blocks<NB>(s_x, H, xv);
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const int f = f0 + i;
        float ag = 0.f, au = 0.f;
#pragma unroll
        for (int c = 0; c < NB; ++c) {
            ag += mx_block_dot(qg[i][c], e8m0_scale(sg[i][c]), xv[c]);
            au += mx_block_dot(qu[i][c], e8m0_scale(su[i][c]), xv[c]);
        }
        ag = wave_sum(ag);
        au = wave_sum(au);
        if (f < F && lane == 0)
            act[static_cast<size_t>(r) * F + f] =
                swiglu(ag + gb[f], au + ub[f], sc.alpha, sc.limit, sc.up_offset);
    }
}

// down GEMV + bias, times the route weight, added into out[t] (seeded with
// the residual by the gate/up kernel). grid.x = (token, slot) pairs with the
// shared expert as the last slot, grid.y = blocks of kDecodeRowsDn rows.
template <int NB>
__global__ __launch_bounds__(256) void decode_down_kernel(
    int T, int H, int F, int k, int n_shared, ExpertPtrs ex, ExpertPtrs sh, const int32_t *idx,
    const float *wts, const float *act, float *out) {
    constexpr int RPW = kDecodeRowsDn / 4;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int nslots = k + n_shared;
    const int t = blockIdx.x / nslots, slot = blockIdx.x - t * nslots;
    const uint8_t *blob;
    size_t r;
    float wt;
    if (slot < k) {
        blob = ex.base + static_cast<size_t>(idx[t * k + slot]) * ex.stride;
        r = static_cast<size_t>(t) * k + slot;
        wt = wts[t * k + slot];
    } else {
        blob = sh.base;
        r = static_cast<size_t>(T) * k + t;
        wt = 1.0f;
    }
    __shared__ float s_a[32][kMaxBlocks + 1];
    stage_vec<false>(act + r * F, F, s_a);
    const int nblk = F / 32;
    const int h0 = blockIdx.y * kDecodeRowsDn + w * RPW;
    const uint8_t *dq = blob + ex.down_q, *ds = blob + ex.down_s;
    const float *db = reinterpret_cast<const float *>(blob + ex.down_b);
    uint4 q[RPW][NB];
    uint32_t sq[RPW][NB];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const int h = min(h0 + i, H - 1);
#pragma unroll
        for (int c = 0; c < NB; ++c) {
            const int b = min(lane + 64 * c, nblk - 1);  // clamped: see the gate/up kernel
            q[i][c] = *reinterpret_cast<const uint4 *>(dq + static_cast<size_t>(h) * (F / 2) + 16 * b);
            sq[i][c] = ds[static_cast<size_t>(h) * nblk + b];
        }
    }
    __syncthreads();
    float av[NB][32];
    lane_blocks<NB>(s_a, F, av);
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        float a = 0.f;
#pragma unroll
        for (int c = 0; c < NB; ++c) a += mx_block_dot(q[i][c], e8m0_scale(sq[i][c]), av[c]);
        a = wave_sum(a);
        const int h = h0 + i;
        if (lane == 0 && h < H)
            unsafeAtomicAdd(out + static_cast<size_t>(t) * H + h, wt * (a + db[h]));
    }
}

template <int NB>
hipError_t gate_up_nb(const void *x, int x_bf16, const double *partial, int S, const float *router_b,
                      int T, int H, int F, int E, int k, int n_shared, float route_scale,
                      const ExpertPtrs &ex, const ExpertPtrs &sh, SwigluConsts c, int32_t *idx,
                      float *wts, int32_t *out_idx, float *out_w, const void *resid,
                      int resid_bf16, float *out, float *act, hipStream_t s) {
    const dim3 grid(T * k + T * n_shared, (F + kDecodeRowsGU - 1) / kDecodeRowsGU);
    if (x_bf16)
        launch_kernel(decode_gate_up_kernel<NB, true>, grid, 256, s, x, partial, S, router_b, T, H,
                      F, E, k, route_scale, ex, sh, c, idx, wts, out_idx, out_w, resid,
                      resid_bf16, out, act);
    else
        launch_kernel(decode_gate_up_kernel<NB, false>, grid, 256, s, x, partial, S, router_b, T,
                      H, F, E, k, route_scale, ex, sh, c, idx, wts, out_idx, out_w, resid,
                      resid_bf16, out, act);
    return hipGetLastError();
}

template <int NB>
hipError_t down_nb(int T, int H, int F, int k, int n_shared, const ExpertPtrs &ex,
                   const ExpertPtrs &sh, const int32_t *idx, const float *wts, const float *act,
                   float *out, hipStream_t s) {
    const dim3 grid(T * (k + n_shared), (H + kDecodeRowsDn - 1) / kDecodeRowsDn);
    launch_kernel(decode_down_kernel<NB>, grid, 256, s, T, H, F, k, n_shared, ex, sh, idx, wts,
                  act, out);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_gate_up(const void *x, int x_bf16, const double *partial, int S,
                                 const float *router_b, int T, int H, int F, int E, int k,
                                 int n_shared, float route_scale, const ExpertPtrs &ex,
                                 const ExpertPtrs &sh, SwigluConsts c, int32_t *idx, float *wts,
                                 int32_t *out_idx, float *out_w, const void *resid,
                                 int resid_bf16, float *out, float *act, hipStream_t s) {
    switch ((H / 32 + 63) / 64) {
    case 1: return gate_up_nb<1>(x, x_bf16, partial, S, router_b, T, H, F, E, k, n_shared, route_scale, ex, sh, c, idx, wts, out_idx, out_w, resid, resid_bf16, out, act, s);
    case 2: return gate_up_nb<2>(x, x_bf16, partial, S, router_b, T, H, F, E, k, n_shared, route_scale, ex, sh, c, idx, wts, out_idx, out_w, resid, resid_bf16, out, act, s);
    case 3: return gate_up_nb<3>(x, x_bf16, partial, S, router_b, T, H, F, E, k, n_shared, route_scale, ex, sh, c, idx, wts, out_idx, out_w, resid, resid_bf16, out, act, s);
    case 4: return gate_up_nb<4>(x, x_bf16, partial, S, router_b, T, H, F, E, k, n_shared, route_scale, ex, sh, c, idx, wts, out_idx, out_w, resid, resid_bf16, out, act, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode_down(int T, int H, int F, int k, int n_shared, const ExpertPtrs &ex,
                              const ExpertPtrs &sh, const int32_t *idx, const float *wts,
                              const float *act, float *out, hipStream_t s) {
    switch ((F / 32 + 63) / 64) {
    case 1: return down_nb<1>(T, H, F, k, n_shared, ex, sh, idx, wts, act, out, s);
    case 2: return down_nb<2>(T, H, F, k, n_shared, ex, sh, idx, wts, act, out, s);
    case 3: return down_nb<3>(T, H, F, k, n_shared, ex, sh, idx, wts, act, out, s);
    case 4: return down_nb<4>(T, H, F, k, n_shared, ex, sh, idx, wts, act, out, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace moe
