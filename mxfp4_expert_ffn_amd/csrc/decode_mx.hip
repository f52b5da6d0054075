// Decode path on the block-scaled matrix cores (v_mfma_scale_f32_16x16x128_f8f6f4).
//
// The weights stay MXFP4 all the way into the matrix core: as operand A, lane
// l supplies one whole MX block (16 code bytes) of weight row l%16, k-group
// l/16, and that block's E8M0 byte as its scale; the hardware applies it. No
// VALU decoding of weights at all, which is what limited the GEMV form.
//
// The activation vector is operand B as kTerms FP8 (E4M3) terms with their
// own E8M0 scales in columns 0..kTerms-1 (the other 12 columns are zero); the
// 16x16 result holds, per weight row, one partial sum per term, and a quad
// DPP sum over the term columns gives the row's dot product. Measured on
// gfx950 with FP4 A and FP8 B: B lane (column n, group h) holds k = 128s + 16h
// + [0,16) in bytes 0..15 and k = 128s + 64 + 16h + [0,16) in bytes 16..31 of
// K-step s, so a term vector stored in natural k order is read as two 16-byte
// pieces; the E8M0 scale that lane supplies applies to the k block
// 128s + 32h + [0,32) (blocks of 32 in natural k order, as for operand A).
//
// Work split: a workgroup takes 16 weight rows of one (token, expert) route;
// its 4 wavefronts split K, each issuing every load of its K-steps before the
// first MFMA, and combine their partial sums through LDS.
//
// Page: goosedump `gpt_oss.rs` `mixture_of_experts` (gate/up pair, biases,
// clamped SwiGLU, down, bias, route weight, slot sum into the residual).
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kMxRows = 16;  // weight rows per workgroup

__device__ __forceinline__ float quad_sum(float v) {
    v += __builtin_amdgcn_update_dpp(0.0f, v, 0xB1, 0xf, 0xf, false);  // quad_perm [1,0,3,2]
    v += __builtin_amdgcn_update_dpp(0.0f, v, 0x4E, 0xf, 0xf, false);  // quad_perm [2,3,0,1]
    return v;
}

__device__ __forceinline__ f32x4_t mx_mfma(const uint4 &a, const uint4 &b0, const uint4 &b1, bool bon,
                                           uint32_t sa, uint32_t sb, f32x4_t acc) {
    const i32x8_t A = {static_cast<int>(a.x), static_cast<int>(a.y), static_cast<int>(a.z),
                       static_cast<int>(a.w), 0, 0, 0, 0};
    const i32x8_t B = bon ? i32x8_t{static_cast<int>(b0.x), static_cast<int>(b0.y),
                                    static_cast<int>(b0.z), static_cast<int>(b0.w),
                                    static_cast<int>(b1.x), static_cast<int>(b1.y),
                                    static_cast<int>(b1.z), static_cast<int>(b1.w)}
                          : i32x8_t{0, 0, 0, 0, 0, 0, 0, 0};
    // cbsz 4: A is FP4 (E2M1); blgp 0: B is FP8 (E4M3); byte 0 of sa / sb is the E8M0 scale
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, acc, 4, 0, 0, static_cast<int>(sa),
                                                             0, static_cast<int>(sb));
}

// gate/up + biases + clamped SwiGLU; writes the activation's FP8 terms (fixed
// exponents act_e0 - 4n) for the down kernel. grid.x = routes, grid.y = row
// blocks of kMxRows.
template <int SPW>
__global__ __launch_bounds__(256) void decode_gate_up_mx_kernel(
    const uint8_t *xq, const uint8_t *xs, int Kp, const double *partial, int S,
    const float *router_b, int T, int H, int F, int E, int k, float route_scale, ExpertPtrs ex,
    ExpertPtrs sh, SwigluConsts sc, int act_e0, int Fp, int32_t *idx, float *wts,
    int32_t *out_idx, float *out_w, const void *resid, int resid_bf16, float *out,
    uint8_t *act_q) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int r = blockIdx.x, R = T * k;
    __shared__ int s_expert;
    __shared__ float s_part[4][2][kMxRows];
    const int t = r < R ? r / k : r - R;
    const int j = r < R ? r - t * k : -1;
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
    float *o = out + static_cast<size_t>(t) * H;
    const float *rf = static_cast<const float *>(resid) + static_cast<size_t>(t) * H;
    if (j == 0 && (resid_bf16 || o != rf)) {  // residual seed: this workgroup's share of out[t]
        const uint16_t *rb = static_cast<const uint16_t *>(resid) + static_cast<size_t>(t) * H;
        const int share = (H + gridDim.y - 1) / gridDim.y;
        const int h0 = blockIdx.y * share;
        for (int h = h0 + threadIdx.x; h < min(H, h0 + share); h += blockDim.x)
            o[h] = resid_bf16 ? bf16_bits_to_f32(rb[h]) : rf[h];
    }
    __syncthreads();
    const uint8_t *blob = r < R ? ex.base + static_cast<size_t>(s_expert) * ex.stride : sh.base;
    const uint8_t *gq = blob + ex.gate_q, *uq = blob + ex.up_q;
    const uint8_t *gs = blob + ex.gate_s, *us = blob + ex.up_s;

    const int NS = Kp / 128, nblk = H / 32;
    const int f0 = blockIdx.y * kMxRows;
    const int arow = lane & 15, ag = lane >> 4;   // A: weight row, k-group
    const int bn = lane & 15, bh = lane >> 4;     // B: column (term), k-group
    const int f = min(f0 + arow, F - 1);
    const int nn = min(bn, kTerms - 1);
    const uint8_t *xrow = xq + (static_cast<size_t>(t) * kTerms + nn) * Kp;
    const uint8_t *srow = xs + (static_cast<size_t>(t) * kTerms + nn) * (Kp / 32);

    // every load of this wavefront's K-steps first (indices clamped in range)
    uint4 wgq[SPW], wuq[SPW], xb0[SPW], xb1[SPW];
    uint32_t wgs[SPW], wus[SPW], xsc[SPW];
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
        const int s = min(w * SPW + i, NS - 1);
        const int blk = min(4 * s + ag, nblk - 1);
        const size_t qo = static_cast<size_t>(f) * (H / 2) + 16 * blk;
        const size_t so = static_cast<size_t>(f) * nblk + blk;
        wgq[i] = *reinterpret_cast<const uint4 *>(gq + qo);
        wuq[i] = *reinterpret_cast<const uint4 *>(uq + qo);
        wgs[i] = gs[so];
        wus[i] = us[so];
        xb0[i] = *reinterpret_cast<const uint4 *>(xrow + 128 * s + 16 * bh);
        xb1[i] = *reinterpret_cast<const uint4 *>(xrow + 128 * s + 64 + 16 * bh);
        xsc[i] = srow[4 * s + bh];
    }
    f32x4_t accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
    const bool bon = bn < kTerms;
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
        if (w * SPW + i < NS) {
            accg = mx_mfma(wgq[i], xb0[i], xb1[i], bon, wgs[i], xsc[i], accg);
            accu = mx_mfma(wuq[i], xb0[i], xb1[i], bon, wus[i], xsc[i], accu);
        }
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        accg[v] = quad_sum(accg[v]);
        accu[v] = quad_sum(accu[v]);
    }
    if (bn == 0) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            s_part[w][0][4 * ag + v] = accg[v];
            s_part[w][1][4 * ag + v] = accu[v];
        }
    }
    __syncthreads();
    if (threadIdx.x < kMxRows) {
        const int ff = f0 + threadIdx.x;
        if (ff < F) {
            float gsum = 0.f, usum = 0.f;
#pragma unroll
            for (int ww = 0; ww < 4; ++ww) {
                gsum += s_part[ww][0][threadIdx.x];
                usum += s_part[ww][1][threadIdx.x];
            }
            const float gb = reinterpret_cast<const float *>(blob + ex.gate_b)[ff];
            const float ub = reinterpret_cast<const float *>(blob + ex.up_b)[ff];
            const float a = swiglu(gsum + gb, usum + ub, sc.alpha, sc.limit, sc.up_offset);
            const uint32_t q = fp8_terms_fixed(a, act_e0);
#pragma unroll
            for (int n = 0; n < kTerms; ++n)
                act_q[(static_cast<size_t>(r) * kTerms + n) * Fp + ff] = static_cast<uint8_t>(q >> (8 * n));
        }
    }
    if (blockIdx.y == gridDim.y - 1) {  // zero the K padding of this route's terms
        const int pad = Fp - F;
        for (int i = threadIdx.x; i < kTerms * pad; i += blockDim.x)
            act_q[(static_cast<size_t>(r) * kTerms + i / pad) * Fp + F + i % pad] = 0;
    }
}

// down + bias, times the route weight, added into out[t] (seeded with the
// residual by the gate/up kernel). grid.x = (token, slot) pairs with the
// shared expert as the last slot, grid.y = row blocks of kMxRows.
template <int SPW>
__global__ __launch_bounds__(256) void decode_down_mx_kernel(
    const uint8_t *act_q, int Fp, int act_e0, int T, int H, int F, int k, int n_shared,
    ExpertPtrs ex, ExpertPtrs sh, const int32_t *idx, const float *wts, float *out) {
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
    __shared__ float s_part[4][kMxRows];
    const uint8_t *dq = blob + ex.down_q, *ds = blob + ex.down_s;
    const int NS = Fp / 128, nblk = F / 32;
    const int h0 = blockIdx.y * kMxRows;
    const int arow = lane & 15, ag = lane >> 4;
    const int bn = lane & 15, bh = lane >> 4;
    const int hr = min(h0 + arow, H - 1);
    const int nn = min(bn, kTerms - 1);
    const uint8_t *arow_q = act_q + (r * kTerms + nn) * Fp;
    const uint32_t bsc = static_cast<uint32_t>(act_e0 - 4 * nn + 127);

    uint4 wq[SPW], ab0[SPW], ab1[SPW];
    uint32_t wsc[SPW];
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
        const int s = min(w * SPW + i, NS - 1);
        const int blk = min(4 * s + ag, nblk - 1);
        wq[i] = *reinterpret_cast<const uint4 *>(dq + static_cast<size_t>(hr) * (F / 2) + 16 * blk);
        wsc[i] = ds[static_cast<size_t>(hr) * nblk + blk];
        ab0[i] = *reinterpret_cast<const uint4 *>(arow_q + 128 * s + 16 * bh);
        ab1[i] = *reinterpret_cast<const uint4 *>(arow_q + 128 * s + 64 + 16 * bh);
    }
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    const bool bon = bn < kTerms;
#pragma unroll
    for (int i = 0; i < SPW; ++i)
        if (w * SPW + i < NS) acc = mx_mfma(wq[i], ab0[i], ab1[i], bon, wsc[i], bsc, acc);
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[v] = quad_sum(acc[v]);
    if (bn == 0) {
#pragma unroll
        for (int v = 0; v < 4; ++v) s_part[w][4 * ag + v] = acc[v];
    }
    __syncthreads();
    if (threadIdx.x < kMxRows) {
        const int h = h0 + threadIdx.x;
        if (h < H) {
            const float y = s_part[0][threadIdx.x] + s_part[1][threadIdx.x] +
                            s_part[2][threadIdx.x] + s_part[3][threadIdx.x];
            const float bias = reinterpret_cast<const float *>(blob + ex.down_b)[h];
            unsafeAtomicAdd(out + static_cast<size_t>(t) * H + h, wt * (y + bias));
        }
    }
}

}  // namespace

int mx_steps_per_wave(int K) {
    const int ns = (K + 127) / 128;
    const int need = (ns + 3) / 4;
    for (int spw : {1, 2, 4, 6, 8})
        if (need <= spw) return spw;
    return 0;
}

hipError_t launch_decode_gate_up_mx(const uint8_t *xq, const uint8_t *xs, const double *partial,
                                    int S, const float *router_b, int T, int H, int F, int E, int k,
                                    int n_shared, float route_scale, const ExpertPtrs &ex,
                                    const ExpertPtrs &sh, SwigluConsts c, int act_e0,
                                    int32_t *idx, float *wts, int32_t *out_idx, float *out_w,
                                    const void *resid, int resid_bf16, float *out, uint8_t *act_q,
                                    hipStream_t s) {
    const int Kp = 128 * ((H + 127) / 128), Fp = 128 * ((F + 127) / 128);
    const dim3 grid(T * k + T * n_shared, (F + kMxRows - 1) / kMxRows);
#define MOE_GU(SPW)                                                                               \
    launch_kernel(decode_gate_up_mx_kernel<SPW>, grid, 256, s, xq, xs, Kp, partial, S, router_b, \
                  T, H, F, E, k, route_scale, ex, sh, c, act_e0, Fp, idx, wts, out_idx, out_w,   \
                  resid, resid_bf16, out, act_q)
    switch (mx_steps_per_wave(H)) {
    case 1: MOE_GU(1); break;
    case 2: MOE_GU(2); break;
    case 4: MOE_GU(4); break;
    case 6: MOE_GU(6); break;
    case 8: MOE_GU(8); break;
    default: return hipErrorInvalidValue;
    }
#undef MOE_GU
    return hipGetLastError();
}

hipError_t launch_decode_down_mx(const uint8_t *act_q, int act_e0, int T, int H, int F, int k,
                                 int n_shared, const ExpertPtrs &ex, const ExpertPtrs &sh,
                                 const int32_t *idx, const float *wts, float *out, hipStream_t s) {
    const int Fp = 128 * ((F + 127) / 128);
    const dim3 grid(T * (k + n_shared), (H + kMxRows - 1) / kMxRows);
#define MOE_DN(SPW)                                                                              \
    launch_kernel(decode_down_mx_kernel<SPW>, grid, 256, s, act_q, Fp, act_e0, T, H, F, k,    \
                  n_shared, ex, sh, idx, wts, out)
    switch (mx_steps_per_wave(F)) {
    case 1: MOE_DN(1); break;
    case 2: MOE_DN(2); break;
    case 4: MOE_DN(4); break;
    case 6: MOE_DN(6); break;
    case 8: MOE_DN(8); break;
    default: return hipErrorInvalidValue;
    }
#undef MOE_DN
    return hipGetLastError();
}

}  // namespace moe
