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
// activations of each of its blocks are loaded once into registers and reused
// for every row the wavefront streams. A row sum is then one DPP reduction.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

template <int NB, bool BF16>
__device__ __forceinline__ void load_vec_blocks(const void *src, int K, float (&v)[NB][32]) {
    const int lane = threadIdx.x & 63;
    const int nblk = K / 32;
#pragma unroll
    for (int c = 0; c < NB; ++c) {
        const int b = lane + 64 * c;
        if (b < nblk) {
            if constexpr (BF16) {
                const uint4 *p = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(src) + 32 * b);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint4 u = p[i];
                    const uint32_t d[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        v[c][8 * i + 2 * j] = __uint_as_float(d[j] << 16);
                        v[c][8 * i + 2 * j + 1] = __uint_as_float(d[j] & 0xffff0000u);
                    }
                }
            } else {
                const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(src) + 32 * b);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float4 f = p[i];
                    v[c][4 * i] = f.x; v[c][4 * i + 1] = f.y; v[c][4 * i + 2] = f.z; v[c][4 * i + 3] = f.w;
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < 32; ++i) v[c][i] = 0.f;
        }
    }
}

// gate/up GEMV + biases + clamped SwiGLU. grid.x = routes (T*k routed, then
// T*n_shared shared rows), grid.y = blocks of kDecodeRowsGU expert rows.
template <int NB, bool BF16>
__global__ __launch_bounds__(256) void decode_gate_up_kernel(
    const void *x, const double *logits, int T, int H, int F, int E, int k, float route_scale,
    ExpertPtrs ex, ExpertPtrs sh, SwigluConsts sc, int32_t *idx, float *wts, int32_t *out_idx,
    float *out_w, float *act) {
    constexpr int RPW = kDecodeRowsGU / 4;  // rows per wavefront
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int r = blockIdx.x, R = T * k;
    __shared__ int s_expert;
    const uint8_t *blob;
    int t;
    if (r < R) {
        t = r / k;
        const int j = r - t * k;
        if (w == 0) {
            int sel[kMaxK];
            double val[kMaxK];
            wave_topk(logits + static_cast<size_t>(t) * E, E, k, sel, val);
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
        __syncthreads();
        blob = ex.base + static_cast<size_t>(s_expert) * ex.stride;
    } else {
        t = r - R;
        blob = sh.base;
    }

    float xv[NB][32];
    if constexpr (BF16)
        load_vec_blocks<NB, true>(static_cast<const uint16_t *>(x) + static_cast<size_t>(t) * H, H, xv);
    else
        load_vec_blocks<NB, false>(static_cast<const float *>(x) + static_cast<size_t>(t) * H, H, xv);

    const int nblk = H / 32;
    const int f0 = blockIdx.y * kDecodeRowsGU + w * RPW;
    const uint8_t *gq = blob + ex.gate_q, *uq = blob + ex.up_q;
    const uint8_t *gs = blob + ex.gate_s, *us = blob + ex.up_s;
    const float *gb = reinterpret_cast<const float *>(blob + ex.gate_b);
    const float *ub = reinterpret_cast<const float *>(blob + ex.up_b);

    uint4 qg[RPW][NB], qu[RPW][NB];
    uint32_t sg[RPW][NB], su[RPW][NB];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const int f = f0 + i;
#pragma unroll
        for (int c = 0; c < NB; ++c) {
            const int b = lane + 64 * c;
            if (f < F && b < nblk) {
                const size_t qo = static_cast<size_t>(f) * (H / 2) + 16 * b;
                const size_t so = static_cast<size_t>(f) * nblk + b;
                qg[i][c] = *reinterpret_cast<const uint4 *>(gq + qo);
                qu[i][c] = *reinterpret_cast<const uint4 *>(uq + qo);
                sg[i][c] = gs[so];
                su[i][c] = us[so];
            } else {
                qg[i][c] = qu[i][c] = make_uint4(0, 0, 0, 0);
                sg[i][c] = su[i][c] = 127;
            }
        }
    }
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

// down GEMV + bias + route-weighted, slot-ordered combine with the residual.
// grid.x = tokens, grid.y = blocks of kDecodeRowsDn hidden rows; wavefront w
// takes slots w, w+4, ... (routed slots, then the shared expert).
template <int NB, bool RBF16>
__global__ __launch_bounds__(256) void decode_down_kernel(
    const void *resid, int T, int H, int F, int k, int n_shared, ExpertPtrs ex, ExpertPtrs sh,
    const int32_t *idx, const float *wts, const float *act, float *out) {
    constexpr int ROWS = kDecodeRowsDn;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int t = blockIdx.x, h0 = blockIdx.y * ROWS;
    const int nslots = k + n_shared, nblk = F / 32;
    __shared__ float ys[kMaxK + 1][ROWS];
    for (int slot = w; slot < nslots; slot += 4) {
        const uint8_t *blob;
        size_t r;
        if (slot < k) {
            blob = ex.base + static_cast<size_t>(idx[t * k + slot]) * ex.stride;
            r = static_cast<size_t>(t) * k + slot;
        } else {
            blob = sh.base;
            r = static_cast<size_t>(T) * k + t;
        }
        float av[NB][32];
        load_vec_blocks<NB, false>(act + r * F, F, av);
        const uint8_t *dq = blob + ex.down_q, *ds = blob + ex.down_s;
        const float *db = reinterpret_cast<const float *>(blob + ex.down_b);
        uint4 q[ROWS][NB];
        uint32_t s[ROWS][NB];
#pragma unroll
        for (int i = 0; i < ROWS; ++i) {
            const int h = h0 + i;
#pragma unroll
            for (int c = 0; c < NB; ++c) {
                const int b = lane + 64 * c;
                if (h < H && b < nblk) {
                    q[i][c] = *reinterpret_cast<const uint4 *>(dq + static_cast<size_t>(h) * (F / 2) + 16 * b);
                    s[i][c] = ds[static_cast<size_t>(h) * nblk + b];
                } else {
                    q[i][c] = make_uint4(0, 0, 0, 0);
                    s[i][c] = 127;
                }
            }
        }
#pragma unroll
        for (int i = 0; i < ROWS; ++i) {
            float a = 0.f;
#pragma unroll
            for (int c = 0; c < NB; ++c) a += mx_block_dot(q[i][c], e8m0_scale(s[i][c]), av[c]);
            a = wave_sum(a);
            const int h = h0 + i;
            if (lane == 0 && h < H) ys[slot][i] = a + db[h];
        }
    }
    __syncthreads();
    if (threadIdx.x < ROWS) {
        const int i = threadIdx.x, h = h0 + i;
        if (h < H) {
            const size_t o = static_cast<size_t>(t) * H + h;
            float acc = RBF16 ? bf16_bits_to_f32(static_cast<const uint16_t *>(resid)[o])
                              : static_cast<const float *>(resid)[o];
            for (int j = 0; j < k; ++j) acc = fmaf(wts[t * k + j], ys[j][i], acc);
            if (n_shared) acc += ys[k][i];
            out[o] = acc;
        }
    }
}

template <int NB>
hipError_t gate_up_nb(const void *x, int x_bf16, const double *logits, int T, int H, int F, int E,
                      int k, int n_shared, float route_scale, const ExpertPtrs &ex,
                      const ExpertPtrs &sh, SwigluConsts c, int32_t *idx, float *wts,
                      int32_t *out_idx, float *out_w, float *act, hipStream_t s) {
    dim3 grid(T * k + T * n_shared, (F + kDecodeRowsGU - 1) / kDecodeRowsGU);
    if (x_bf16)
        launch_kernel(decode_gate_up_kernel<NB, true>, grid, 256, s, x, logits, T, H, F, E, k,
                      route_scale, ex, sh, c, idx, wts, out_idx, out_w, act);
    else
        launch_kernel(decode_gate_up_kernel<NB, false>, grid, 256, s, x, logits, T, H, F, E, k,
                      route_scale, ex, sh, c, idx, wts, out_idx, out_w, act);
    return hipGetLastError();
}

template <int NB>
hipError_t down_nb(const void *resid, int resid_bf16, int T, int H, int F, int k, int n_shared,
                   const ExpertPtrs &ex, const ExpertPtrs &sh, const int32_t *idx, const float *wts,
                   const float *act, float *out, hipStream_t s) {
    dim3 grid(T, (H + kDecodeRowsDn - 1) / kDecodeRowsDn);
    if (resid_bf16)
        launch_kernel(decode_down_kernel<NB, true>, grid, 256, s, resid, T, H, F, k, n_shared, ex,
                      sh, idx, wts, act, out);
    else
        launch_kernel(decode_down_kernel<NB, false>, grid, 256, s, resid, T, H, F, k, n_shared, ex,
                      sh, idx, wts, act, out);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_gate_up(const void *x, int x_bf16, const double *logits, int T, int H,
                                 int F, int E, int k, int n_shared, float route_scale,
                                 const ExpertPtrs &ex, const ExpertPtrs &sh, SwigluConsts c,
                                 int32_t *idx, float *wts, int32_t *out_idx, float *out_w,
                                 float *act, hipStream_t s) {
    const int nb = (H / 32 + 63) / 64;
    switch (nb) {
    case 1: return gate_up_nb<1>(x, x_bf16, logits, T, H, F, E, k, n_shared, route_scale, ex, sh, c, idx, wts, out_idx, out_w, act, s);
    case 2: return gate_up_nb<2>(x, x_bf16, logits, T, H, F, E, k, n_shared, route_scale, ex, sh, c, idx, wts, out_idx, out_w, act, s);
    case 3: return gate_up_nb<3>(x, x_bf16, logits, T, H, F, E, k, n_shared, route_scale, ex, sh, c, idx, wts, out_idx, out_w, act, s);
    case 4: return gate_up_nb<4>(x, x_bf16, logits, T, H, F, E, k, n_shared, route_scale, ex, sh, c, idx, wts, out_idx, out_w, act, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode_down(const void *resid, int resid_bf16, int T, int H, int F, int k,
                              int n_shared, const ExpertPtrs &ex, const ExpertPtrs &sh,
                              const int32_t *idx, const float *wts, const float *act, float *out,
                              hipStream_t s) {
    const int nb = (F / 32 + 63) / 64;
    switch (nb) {
    case 1: return down_nb<1>(resid, resid_bf16, T, H, F, k, n_shared, ex, sh, idx, wts, act, out, s);
    case 2: return down_nb<2>(resid, resid_bf16, T, H, F, k, n_shared, ex, sh, idx, wts, act, out, s);
    case 3: return down_nb<3>(resid, resid_bf16, T, H, F, k, n_shared, ex, sh, idx, wts, act, out, s);
    case 4: return down_nb<4>(resid, resid_bf16, T, H, F, k, n_shared, ex, sh, idx, wts, act, out, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace moe
