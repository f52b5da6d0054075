// Decode (T <= 64): per route, GEMVs over the selected expert's MXFP4 planes
// on the block-scaled matrix cores.
//
// A workgroup takes 32 weight rows (two 16-row tiles) of one route; its 8
// wavefronts split K into 128-wide steps, and each issues every load of its
// steps before its first matrix-core instruction. Weight tiles are read as
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
    double v[4];
    if (E <= 64) gather_logits<1>(partial, S, T, t, E, router_b, v);
    else if (E <= 128) gather_logits<2>(partial, S, T, t, E, router_b, v);
    else gather_logits<4>(partial, S, T, t, E, router_b, v);
    wave_topk(v, E, k, sel, val);
}

// gate/up + biases + clamped SwiGLU for 32 features of one route; writes the
// activation block's FP8 terms and scales. grid.x = routes, grid.y = 32-wide
// feature blocks of pad128(F) (blocks past F write the zero padding).
// Every wavefront selects the route's expert itself (top-k of the token's
// logits), so its weight loads wait on no barrier. Workgroups of slot 0 also
// seed out[t] with the residual (a share each) and, in feature block 0,
// publish the token's experts and route weights.
template <int SPW>
__global__ __launch_bounds__(kDecodeWaves * 64) void decode_gate_up_kernel(
    const uint8_t *xq, const uint8_t *xs, const double *partial, int S, const float *router_b,
    int T, int H, int F, int E, int k, float route_scale, ExpertPtrs ex, ExpertPtrs sh,
    SwigluConsts sc, int32_t *idx, float *wts, int32_t *out_idx, float *out_w,
    const void *resid, int resid_bf16, float *out, uint8_t *act_q, uint8_t *act_s) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int r = blockIdx.x, R = T * k;
    const int t = r < R ? r / k : r - R;
    const int j = r < R ? r - t * k : -1;
    const int fb = blockIdx.y;
    const int Kp = pad128(H), Fp = pad128(F), nbp = Fp / 32;
    if (j == 0) {  // residual seed, unless out already is the float32 residual
        float *o = out + static_cast<size_t>(t) * H;
        const float *rf = static_cast<const float *>(resid) + static_cast<size_t>(t) * H;
        if (resid_bf16 || o != rf) {
            const uint16_t *rb = static_cast<const uint16_t *>(resid) + static_cast<size_t>(t) * H;
            const int share = (H + gridDim.y - 1) / gridDim.y;
            const int end = min(H, (fb + 1) * share);
            for (int h = fb * share + threadIdx.x; h < end; h += blockDim.x)
                o[h] = resid_bf16 ? bf16_bits_to_f32(rb[h]) : rf[h];
        }
    }
    uint8_t *aq = act_q + static_cast<size_t>(r) * kTerms * Fp;
    uint8_t *as = act_s + static_cast<size_t>(r) * kTerms * nbp;
    if (32 * fb >= F) {  // K padding of the down GEMV's operand: zero codes
        if (threadIdx.x < 32 * kTerms) {
            const int n = threadIdx.x >> 5, i = threadIdx.x & 31;
            aq[n * Fp + 32 * fb + i] = 0;
            if (i == 0) as[n * nbp + fb] = 127;
        }
        return;
    }
    const uint8_t *blob = sh.base;
    if (r < R) {
        int sel[kMaxK];
        double val[kMaxK];
        route_token(partial, S, router_b, T, t, E, k, sel, val);
        int mine = sel[0];
#pragma unroll
        for (int jj = 1; jj < kMaxK; ++jj)
            if (jj == j) mine = sel[jj];
        blob = ex.base + static_cast<size_t>(mine) * ex.stride;
        if (j == 0 && fb == 0 && w == 0) {
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
    // the epilogue's biases, loaded with the weights
    const int fe = 32 * fb + (lane & 31);
    const float bias_g = reinterpret_cast<const float *>(blob + ex.gate_b)[fe];
    const float bias_u = reinterpret_cast<const float *>(blob + ex.up_b)[fe];
    const uint8_t *gq = blob + ex.gate_q, *uq = blob + ex.up_q;
    const uint8_t *gs = blob + ex.gate_s, *us = blob + ex.up_s;
    const int NS = Kp / 128, nblk = H / 32;
    const int bn = lane & 15, bh = lane >> 4;
    const int nn = min(bn, kTerms - 1);
    const bool bon = bn < kTerms;
    const uint8_t *xrow = xq + (static_cast<size_t>(t) * kTerms + nn) * Kp;
    const uint8_t *srow = xs + (static_cast<size_t>(t) * kTerms + nn) * (Kp / 32);
    const uint4 zero = make_uint4(0u, 0u, 0u, 0u);

    f32x4_t acc[4];  // gate tile 0, gate tile 1, up tile 0, up tile 1
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int s0 = w * SPW; s0 < NS; s0 += kDecodeWaves * SPW) {  // one round unless K > 4096
        AFrag a[SPW][4];
        BFrag b[SPW];
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            const int s = min(s0 + i, NS - 1);
            a[i][0] = load_afrag(gq, gs, 2 * fb, s, nblk, lane);
            a[i][1] = load_afrag(gq, gs, 2 * fb + 1, s, nblk, lane);
            a[i][2] = load_afrag(uq, us, 2 * fb, s, nblk, lane);
            a[i][3] = load_afrag(uq, us, 2 * fb + 1, s, nblk, lane);
            b[i] = load_bfrag(xrow, srow, s, bh);
        }
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            if (s0 + i < NS) {
                const uint4 blo = bon ? b[i].lo : zero, bhi = bon ? b[i].hi : zero;
#pragma unroll
                for (int m = 0; m < 4; ++m) acc[m] = mx_mfma(a[i][m], blo, bhi, b[i].s, acc[m]);
            }
        }
    }

    __shared__ float s_part[kDecodeWaves][4][16];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[m][v] = quad_sum(acc[m][v]);
    if (bn == 0) {
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int v = 0; v < 4; ++v) s_part[w][m][4 * bh + v] = acc[m][v];
    }
    __syncthreads();
    if (w == 0) {  // both half-waves hold the block; lanes 0..31 store it
        const int i = lane & 31, tile = i >> 4, row = i & 15;
        const int f = 32 * fb + i;
        float g = 0.f, u = 0.f;
#pragma unroll
        for (int ww = 0; ww < kDecodeWaves; ++ww) {
            g += s_part[ww][tile][row];
            u += s_part[ww][2 + tile][row];
        }
        const float a = swiglu(g + bias_g, u + bias_u, sc.alpha, sc.limit, sc.up_offset);
        uint32_t codes, scales;
        fp8_terms_group(a, codes, scales);
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
// the residual). grid.x = routes, grid.y = 32-row blocks of H.
template <int SPW>
__global__ __launch_bounds__(kDecodeWaves * 64) void decode_down_kernel(
    const uint8_t *act_q, const uint8_t *act_s, int T, int H, int F, int k, const int32_t *idx,
    const float *wts, ExpertPtrs ex, ExpertPtrs sh, float *out) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int r = blockIdx.x, R = T * k;
    const int t = r < R ? r / k : r - R;
    const int hb = blockIdx.y;
    const uint8_t *blob = r < R ? ex.base + static_cast<size_t>(idx[r]) * ex.stride : sh.base;
    const uint8_t *dq = blob + ex.down_q, *ds = blob + ex.down_s;
    const float wt = r < R ? wts[r] : 1.0f;
    const float bias = reinterpret_cast<const float *>(blob + ex.down_b)[32 * hb + (lane & 31)];
    const int Fp = pad128(F), NS = Fp / 128, nblk = F / 32;
    const int bn = lane & 15, bh = lane >> 4;
    const int nn = min(bn, kTerms - 1);
    const bool bon = bn < kTerms;
    const uint8_t *xrow = act_q + (static_cast<size_t>(r) * kTerms + nn) * Fp;
    const uint8_t *srow = act_s + (static_cast<size_t>(r) * kTerms + nn) * (Fp / 32);
    const uint4 zero = make_uint4(0u, 0u, 0u, 0u);

    f32x4_t acc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
    for (int s0 = w * SPW; s0 < NS; s0 += kDecodeWaves * SPW) {
        AFrag a[SPW][2];
        BFrag b[SPW];
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            const int s = min(s0 + i, NS - 1);
            a[i][0] = load_afrag(dq, ds, 2 * hb, s, nblk, lane);
            a[i][1] = load_afrag(dq, ds, 2 * hb + 1, s, nblk, lane);
            b[i] = load_bfrag(xrow, srow, s, bh);
        }
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            if (s0 + i < NS) {
                const uint4 blo = bon ? b[i].lo : zero, bhi = bon ? b[i].hi : zero;
                acc[0] = mx_mfma(a[i][0], blo, bhi, b[i].s, acc[0]);
                acc[1] = mx_mfma(a[i][1], blo, bhi, b[i].s, acc[1]);
            }
        }
    }

    __shared__ float s_part[kDecodeWaves][2][16];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[m][v] = quad_sum(acc[m][v]);
    if (bn == 0) {
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int v = 0; v < 4; ++v) s_part[w][m][4 * bh + v] = acc[m][v];
    }
    __syncthreads();
    if (threadIdx.x < 32) {
        const int i = threadIdx.x, h = 32 * hb + i;
        float y = 0.f;
#pragma unroll
        for (int ww = 0; ww < kDecodeWaves; ++ww) y += s_part[ww][i >> 4][i & 15];
        unsafeAtomicAdd(out + static_cast<size_t>(t) * H + h, wt * (y + bias));
    }
}

// K-steps per wavefront per round (rounds repeat past 8 * 4 steps, K > 4096).
int decode_spw(int K) {
    const int ns = pad128(K) / 128;
    const int spw = (ns + kDecodeWaves - 1) / kDecodeWaves;
    return spw < 1 ? 1 : (spw > 4 ? 4 : spw);
}

}  // namespace

hipError_t launch_decode_gate_up(const uint8_t *xq, const uint8_t *xs, const double *partial, int S,
                                 const float *router_b, int T, int H, int F, int E, int k,
                                 int n_shared, float route_scale, const ExpertPtrs &ex,
                                 const ExpertPtrs &sh, SwigluConsts c, int32_t *idx, float *wts,
                                 int32_t *out_idx, float *out_w, const void *resid, int resid_bf16,
                                 float *out, uint8_t *act_q, uint8_t *act_s, hipStream_t s) {
    const dim3 grid(T * (k + n_shared), pad128(F) / 32);
    const dim3 block(kDecodeWaves * 64);
#define MOE_GU(SPW)                                                                              \
    launch_kernel(decode_gate_up_kernel<SPW>, grid, block, s, xq, xs, partial, S, router_b, T, H, \
                  F, E, k, route_scale, ex, sh, c, idx, wts, out_idx, out_w, resid, resid_bf16,   \
                  out, act_q, act_s)
    switch (decode_spw(H)) {
    case 1: MOE_GU(1); break;
    case 2: MOE_GU(2); break;
    case 3: MOE_GU(3); break;
    default: MOE_GU(4); break;
    }
#undef MOE_GU
    return hipGetLastError();
}

hipError_t launch_decode_down(const uint8_t *act_q, const uint8_t *act_s, int T, int H, int F,
                              int k, int n_shared, const int32_t *idx, const float *wts,
                              const ExpertPtrs &ex, const ExpertPtrs &sh, float *out,
                              hipStream_t s) {
    const dim3 grid(T * (k + n_shared), H / 32);
    const dim3 block(kDecodeWaves * 64);
#define MOE_DN(SPW)                                                                           \
    launch_kernel(decode_down_kernel<SPW>, grid, block, s, act_q, act_s, T, H, F, k, idx, wts, \
                  ex, sh, out)
    switch (decode_spw(F)) {
    case 1: MOE_DN(1); break;
    case 2: MOE_DN(2); break;
    case 3: MOE_DN(3); break;
    default: MOE_DN(4); break;
    }
#undef MOE_DN
    return hipGetLastError();
}

}  // namespace moe
