// Prefill path: grouped GEMMs over the expert-sorted rows on the CDNA4 matrix
// cores (v_mfma_f32_32x32x16_bf16).
//
// Page: goosedump `gpt_oss.rs` `expert_batch_output`: per active expert, the
// routed rows are gathered, multiplied by the gate/up pair, biased, passed
// through the clamped SwiGLU, multiplied by down, biased, and scaled by the
// route weight; `mix_expert_outputs` sums each token's routes.
//
// Operands. MXFP4 weights are exact in bfloat16. Float32 activations are split
// as x = hi + lo (two bfloat16), so each product takes two MFMAs sharing the
// decoded weight tile and keeps float32-level accuracy; bfloat16 inputs need
// only the hi term.
//
// K order. A 32x32x16 MFMA has lane l supply 8 consecutive k values for row
// (or column) l%32 from k-group l/32. Any permutation of k applied to both
// operands leaves the sum unchanged, so in a 64-wide k step lane group g takes
// MX block (2s + g) and the four MFMAs j = 0..3 walk its 32 elements 8 at a
// time. One 128-bit load per lane is then exactly one MX block (16 code bytes
// and one scale), decoded in registers: no LDS round trip for the weights.
// The activation tile (32 rows x 64 k) is staged in LDS as bfloat16 hi/lo and
// read back in the same permuted order.
//
// Tiles. The permutation kernel leaves mprefix[g] = number of 32-row tiles of
// groups < g. Tiles are numbered group-major, then by weight tile, then by row
// tile, and dealt so that each XCD sweeps a contiguous range: consecutive
// workgroups on one L2 share an expert's weight tile and its rows.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kBM = kGemmBM;
constexpr int kLdsPitch = 72;  // bf16 per staged row: 64 + 8 pad (144 B rows)

struct TileInfo {
    int g, nt, row0, rows;
};

__device__ __forceinline__ TileInfo find_tile(int tile, int NT, int G, const int32_t *mprefix,
                                              const int32_t *offsets) {
    int lo = 0, hi = G - 1;  // largest g with mprefix[g] * NT <= tile
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (mprefix[mid] * NT <= tile) lo = mid;
        else hi = mid - 1;
    }
    TileInfo ti;
    ti.g = lo;
    const int mt_g = mprefix[lo + 1] - mprefix[lo];
    const int local = tile - mprefix[lo] * NT;
    ti.nt = local / mt_g;
    const int mt = local - ti.nt * mt_g;
    ti.row0 = offsets[lo] + mt * kBM;
    ti.rows = min(kBM, offsets[lo + 1] - ti.row0);
    return ti;
}

// Activation staging: 256 threads, thread -> row tid/8, 8 consecutive k.
template <bool BF16>
struct AStage {
    float4 f[2];
    uint4 b;
    __device__ __forceinline__ void load(const void *src, int ld, int srow, int col, int K) {
        const bool ok = srow >= 0 && col < K;
        if constexpr (BF16) {
            b = ok ? *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(src) +
                                                      static_cast<size_t>(srow) * ld + col)
                   : make_uint4(0, 0, 0, 0);
        } else {
            if (ok) {
                const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(src) +
                                                                   static_cast<size_t>(srow) * ld + col);
                f[0] = p[0];
                f[1] = p[1];
            } else {
                f[0] = f[1] = make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
    }
    __device__ __forceinline__ void store(__bf16 *hi, __bf16 *lo) const {
        if constexpr (BF16) {
            *reinterpret_cast<uint4 *>(hi) = b;
        } else {
            const float v[8] = {f[0].x, f[0].y, f[0].z, f[0].w, f[1].x, f[1].y, f[1].z, f[1].w};
            bf16x8_t h, l;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                __bf16 a, c;
                split_bf16(v[i], a, c);
                h[i] = a;
                l[i] = c;
            }
            *reinterpret_cast<bf16x8_t *>(hi) = h;
            *reinterpret_cast<bf16x8_t *>(lo) = l;
        }
    }
};

__device__ __forceinline__ void load_mx(const uint8_t *q, const uint8_t *sc, int row, int K, int kb,
                                        uint4 &code, uint32_t &scale) {
    if (kb < K / 32) {
        code = *reinterpret_cast<const uint4 *>(q + static_cast<size_t>(row) * (K / 2) + 16 * kb);
        scale = sc[static_cast<size_t>(row) * (K / 32) + kb];
    } else {
        code = make_uint4(0, 0, 0, 0);
        scale = 127;
    }
}

__device__ __forceinline__ uint32_t dword(const uint4 &q, int j) {
    return j == 0 ? q.x : j == 1 ? q.y : j == 2 ? q.z : q.w;
}

// ---------------------------------------------------------------- gate/up
// Workgroup tile: 32 rows of one expert x 128 features (4 waves x 32), both
// gate and up; epilogue adds the biases, applies the clamped SwiGLU and
// stores the float32 activation row of each (token, slot) route.
template <bool BF16>
__global__ __launch_bounds__(256) void gate_up_gemm_kernel(
    const void *x, int T, int H, int F, int E, int n_shared, int k, ExpertPtrs ex,
    ExpertPtrs sh, SwigluConsts sc, const int32_t *offsets, const int32_t *perm,
    const int32_t *mprefix, float *act) {
    const int G = E + n_shared;
    const int NT = (F + kGateUpBN - 1) / kGateUpBN;
    int tile;
    if (!xcd_tile(blockIdx.x, mprefix[G] * NT, tile)) return;
    const TileInfo ti = find_tile(tile, NT, G, mprefix, offsets);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int gsel = lane >> 5, l32 = lane & 31;
    const uint8_t *blob = ti.g < E ? ex.base + static_cast<size_t>(ti.g) * ex.stride : sh.base;

    __shared__ int s_src[kBM];
    __shared__ __align__(16) __bf16 s_a[2][2][kBM][kLdsPitch];
    if (threadIdx.x < kBM) {
        const int m = threadIdx.x;
        int src = -1;
        if (m < ti.rows) {
            const int p = ti.row0 + m;
            src = ti.g < E ? perm[p] / k : p - offsets[E];
        }
        s_src[m] = src;
    }
    __syncthreads();

    const int n = ti.nt * kGateUpBN + 32 * w + l32;  // feature of this lane's B column
    const bool wave_on = ti.nt * kGateUpBN + 32 * w < F;
    const uint8_t *gq = blob + ex.gate_q, *uq = blob + ex.up_q;
    const uint8_t *gs = blob + ex.gate_s, *us = blob + ex.up_s;

    const int arow = threadIdx.x >> 3, acol = (threadIdx.x & 7) * 8;
    const int asrc = s_src[arow];
    AStage<BF16> ast;
    uint4 qg_n, qu_n;
    uint32_t sg_n, su_n;
    const int nsteps = (H + 63) / 64;

    ast.load(x, H, asrc, acol, H);
    if (wave_on) {
        load_mx(gq, gs, n, H, gsel, qg_n, sg_n);
        load_mx(uq, us, n, H, gsel, qu_n, su_n);
    }
    f32x16_t acc_g = {}, acc_u = {};
    for (int s = 0; s < nsteps; ++s) {
        const int buf = s & 1;
        ast.store(&s_a[buf][0][arow][acol], &s_a[buf][1][arow][acol]);
        const uint4 qg = qg_n, qu = qu_n;
        const uint32_t sg = sg_n, su = su_n;
        __syncthreads();
        if (s + 1 < nsteps) {
            ast.load(x, H, asrc, 64 * (s + 1) + acol, H);
            if (wave_on) {
                load_mx(gq, gs, n, H, 2 * (s + 1) + gsel, qg_n, sg_n);
                load_mx(uq, us, n, H, 2 * (s + 1) + gsel, qu_n, su_n);
            }
        }
        if (wave_on) {
            const float fsg = e8m0_scale(sg), fsu = e8m0_scale(su);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bf16x8_t bg = fp4x8_to_bf16(dword(qg, j), fsg);
                const bf16x8_t bu = fp4x8_to_bf16(dword(qu, j), fsu);
                const bf16x8_t ah = *reinterpret_cast<const bf16x8_t *>(&s_a[buf][0][l32][gsel * 32 + 8 * j]);
                acc_g = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bg, acc_g, 0, 0, 0);
                acc_u = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bu, acc_u, 0, 0, 0);
                if constexpr (!BF16) {
                    const bf16x8_t al = *reinterpret_cast<const bf16x8_t *>(&s_a[buf][1][l32][gsel * 32 + 8 * j]);
                    acc_g = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bg, acc_g, 0, 0, 0);
                    acc_u = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bu, acc_u, 0, 0, 0);
                }
            }
        }
    }
    if (!wave_on) return;
    const float bgate = reinterpret_cast<const float *>(blob + ex.gate_b)[n];
    const float bup = reinterpret_cast<const float *>(blob + ex.up_b)[n];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int m = 8 * (v >> 2) + 4 * gsel + (v & 3);
        if (m < ti.rows)
            act[static_cast<size_t>(ti.row0 + m) * F + n] =
                swiglu(acc_g[v] + bgate, acc_u[v] + bup, sc.alpha, sc.limit, sc.up_offset);
    }
}

// ---------------------------------------------------------------- down
// Workgroup tile: 32 rows of one expert x 256 hidden units (4 waves x 2 x 32);
// epilogue adds the down bias, multiplies by the route weight and adds into
// the token's output row (which already holds the residual).
__global__ __launch_bounds__(256) void down_gemm_kernel(
    int T, int H, int F, int E, int n_shared, int k, ExpertPtrs ex, ExpertPtrs sh,
    const int32_t *offsets, const int32_t *perm, const float *wts, const int32_t *mprefix,
    const float *act, float *out) {
    constexpr int NSUB = kDownBN / 128;
    const int G = E + n_shared;
    const int NT = (H + kDownBN - 1) / kDownBN;
    int tile;
    if (!xcd_tile(blockIdx.x, mprefix[G] * NT, tile)) return;
    const TileInfo ti = find_tile(tile, NT, G, mprefix, offsets);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int gsel = lane >> 5, l32 = lane & 31;
    const uint8_t *blob = ti.g < E ? ex.base + static_cast<size_t>(ti.g) * ex.stride : sh.base;

    __shared__ int s_src[kBM];
    __shared__ int s_tok[kBM];
    __shared__ float s_wt[kBM];
    __shared__ __align__(16) __bf16 s_a[2][2][kBM][kLdsPitch];
    if (threadIdx.x < kBM) {
        const int m = threadIdx.x;
        int src = -1, tok = 0;
        float wt = 0.f;
        if (m < ti.rows) {
            const int p = ti.row0 + m;
            src = p;
            if (ti.g < E) {
                const int r = perm[p];
                tok = r / k;
                wt = wts[r];
            } else {
                tok = p - offsets[E];
                wt = 1.0f;
            }
        }
        s_src[m] = src;
        s_tok[m] = tok;
        s_wt[m] = wt;
    }
    __syncthreads();

    const uint8_t *dq = blob + ex.down_q, *ds = blob + ex.down_s;
    int hrow[NSUB];
    bool on[NSUB];
#pragma unroll
    for (int i = 0; i < NSUB; ++i) {
        const int base = ti.nt * kDownBN + (w * NSUB + i) * 32;
        on[i] = base < H;
        hrow[i] = base + l32;
    }
    const int arow = threadIdx.x >> 3, acol = (threadIdx.x & 7) * 8;
    const int asrc = s_src[arow];
    AStage<false> ast;
    uint4 q_n[NSUB];
    uint32_t s_n[NSUB];
    const int nsteps = (F + 63) / 64;

    ast.load(act, F, asrc, acol, F);
#pragma unroll
    for (int i = 0; i < NSUB; ++i)
        if (on[i]) load_mx(dq, ds, hrow[i], F, gsel, q_n[i], s_n[i]);
    f32x16_t acc[NSUB];
#pragma unroll
    for (int i = 0; i < NSUB; ++i) acc[i] = f32x16_t{};
    for (int s = 0; s < nsteps; ++s) {
        const int buf = s & 1;
        ast.store(&s_a[buf][0][arow][acol], &s_a[buf][1][arow][acol]);
        uint4 q[NSUB];
        uint32_t sc[NSUB];
#pragma unroll
        for (int i = 0; i < NSUB; ++i) {
            q[i] = q_n[i];
            sc[i] = s_n[i];
        }
        __syncthreads();
        if (s + 1 < nsteps) {
            ast.load(act, F, asrc, 64 * (s + 1) + acol, F);
#pragma unroll
            for (int i = 0; i < NSUB; ++i)
                if (on[i]) load_mx(dq, ds, hrow[i], F, 2 * (s + 1) + gsel, q_n[i], s_n[i]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bf16x8_t ah = *reinterpret_cast<const bf16x8_t *>(&s_a[buf][0][l32][gsel * 32 + 8 * j]);
            const bf16x8_t al = *reinterpret_cast<const bf16x8_t *>(&s_a[buf][1][l32][gsel * 32 + 8 * j]);
#pragma unroll
            for (int i = 0; i < NSUB; ++i) {
                if (on[i]) {
                    const bf16x8_t b = fp4x8_to_bf16(dword(q[i], j), e8m0_scale(sc[i]));
                    acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, b, acc[i], 0, 0, 0);
                    acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, b, acc[i], 0, 0, 0);
                }
            }
        }
    }
    const float *db = reinterpret_cast<const float *>(blob + ex.down_b);
#pragma unroll
    for (int i = 0; i < NSUB; ++i) {
        if (!on[i]) continue;
        const float bias = db[hrow[i]];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int m = 8 * (v >> 2) + 4 * gsel + (v & 3);
            if (m < ti.rows)
                unsafeAtomicAdd(out + static_cast<size_t>(s_tok[m]) * H + hrow[i],
                                s_wt[m] * (acc[i][v] + bias));
        }
    }
}

}  // namespace

hipError_t launch_gate_up_gemm(const void *x, int x_bf16, int T, int H, int F, int E, int k,
                               int n_shared, const ExpertPtrs &ex, const ExpertPtrs &sh,
                               SwigluConsts c, const int32_t *offsets, const int32_t *perm,
                               const int32_t *mprefix, int max_mtiles, float *act,
                               hipStream_t s) {
    const int NT = (F + kGateUpBN - 1) / kGateUpBN;
    const long long tiles = static_cast<long long>(max_mtiles) * NT;
    const int grid = static_cast<int>((tiles + kXcds - 1) / kXcds * kXcds);
    if (grid == 0) return hipSuccess;
    if (x_bf16)
        launch_kernel(gate_up_gemm_kernel<true>, grid, 256, s, x, T, H, F, E, n_shared, k, ex, sh,
                      c, offsets, perm, mprefix, act);
    else
        launch_kernel(gate_up_gemm_kernel<false>, grid, 256, s, x, T, H, F, E, n_shared, k, ex, sh,
                      c, offsets, perm, mprefix, act);
    return hipGetLastError();
}

hipError_t launch_down_gemm(int T, int H, int F, int E, int k, int n_shared, const ExpertPtrs &ex,
                            const ExpertPtrs &sh, const int32_t *offsets, const int32_t *perm,
                            const float *wts, const int32_t *mprefix, int max_mtiles,
                            const float *act, float *out, hipStream_t s) {
    const int NT = (H + kDownBN - 1) / kDownBN;
    const long long tiles = static_cast<long long>(max_mtiles) * NT;
    const int grid = static_cast<int>((tiles + kXcds - 1) / kXcds * kXcds);
    if (grid == 0) return hipSuccess;
    launch_kernel(down_gemm_kernel, grid, 256, s, T, H, F, E, n_shared, k, ex, sh, offsets, perm,
                  wts, mprefix, act, out);
    return hipGetLastError();
}

}  // namespace moe
