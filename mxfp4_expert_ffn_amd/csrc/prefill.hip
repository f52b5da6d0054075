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
constexpr int kTiles = 4;  // B tiles (32 weight rows each) per wavefront
constexpr int kDepth = 2;  // K steps (64 wide) of loads kept in flight per thread

struct TileInfo {
    int g, nt, row0, rows;
};

// Tile -> (group, weight tile, row range). The M-tile prefix is first copied
// to LDS (one round of loads), then binary-searched there.
__device__ __forceinline__ TileInfo find_tile(int tile, int NT, int G, const int32_t *mprefix,
                                              const int32_t *offsets, int *s_pre) {
    for (int i = threadIdx.x; i <= G; i += blockDim.x) s_pre[i] = mprefix[i];
    __syncthreads();
    int lo = 0, hi = G - 1;  // largest g with s_pre[g] * NT <= tile
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_pre[mid] * NT <= tile) lo = mid;
        else hi = mid - 1;
    }
    TileInfo ti;
    ti.g = lo;
    const int mt_g = s_pre[lo + 1] - s_pre[lo];
    const int local = tile - s_pre[lo] * NT;
    ti.nt = local / mt_g;
    const int mt = local - ti.nt * mt_g;
    ti.row0 = offsets[lo] + mt * kBM;
    ti.rows = min(kBM, offsets[lo + 1] - ti.row0);
    return ti;
}

// Staged activation tile: [buffer][hi, lo][32 rows][64 bf16]. Each 128-byte
// row holds eight 16-byte chunks stored at chunk ^ (row & 7), so the MFMA
// operand reads (32 rows at one logical chunk) and the staging writes (one
// row, eight chunks) both touch every LDS bank once per 8 lanes.
typedef __bf16 ATile[2][2][kBM][64];

__device__ __forceinline__ int swz(int row, int chunk) { return ((chunk ^ (row & 7)) << 3); }

// Activation staging: 256 threads, thread -> row tid/8, 16-byte chunk tid%8
// (8 consecutive k). Loads are unconditional (invalid rows or k read row 0,
// column 0) and validity is applied when the registers are written to LDS,
// so loads stay in flight.
template <bool BF16>
struct AStage {
    float4 f[2];
    uint4 b;
    bool ok;
    __device__ __forceinline__ void load(const void *src, int ld, int srow, int col, int K) {
        ok = srow >= 0 && col < K;
        const size_t off = ok ? static_cast<size_t>(srow) * ld + col : 0;
        if constexpr (BF16) {
            b = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(src) + off);
        } else {
            const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(src) + off);
            f[0] = p[0];
            f[1] = p[1];
        }
    }
    __device__ __forceinline__ void store(ATile &sa, int buf, int row, int chunk) const {
        __bf16 *hi = &sa[buf][0][row][swz(row, chunk)];
        __bf16 *lo = &sa[buf][1][row][swz(row, chunk)];
        if constexpr (BF16) {
            *reinterpret_cast<uint4 *>(hi) = ok ? b : make_uint4(0, 0, 0, 0);
        } else {
            const float v[8] = {f[0].x, f[0].y, f[0].z, f[0].w, f[1].x, f[1].y, f[1].z, f[1].w};
            bf16x8_t h, l;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                __bf16 a, c;
                split_bf16(ok ? v[i] : 0.f, a, c);
                h[i] = a;
                l[i] = c;
            }
            *reinterpret_cast<bf16x8_t *>(hi) = h;
            *reinterpret_cast<bf16x8_t *>(lo) = l;
        }
    }
};

// One MX block (16 code bytes + scale) of a K-wide row. Unconditional: a
// block past the end of K reads the row's last block (finite weights), which
// meets zero activations.
__device__ __forceinline__ void load_mx(const uint8_t *q, const uint8_t *sc, int row, int K, int kb,
                                        uint4 &code, uint32_t &scale) {
    const int b = min(kb, K / 32 - 1);
    code = *reinterpret_cast<const uint4 *>(q + static_cast<size_t>(row) * (K / 2) + 16 * b);
    scale = sc[static_cast<size_t>(row) * (K / 32) + b];
}

__device__ __forceinline__ uint32_t dword(const uint4 &q, int j) {
    return j == 0 ? q.x : j == 1 ? q.y : j == 2 ? q.z : q.w;
}

// B tiles of one wavefront: tile i is the 32 weight rows row[i] (one per lane
// l%32) of the MXFP4 plane (q[i], sc[i]) with K-wide rows; on[i] is uniform.
struct BTiles {
    const uint8_t *q[kTiles];
    const uint8_t *sc[kTiles];
    int row[kTiles];
    bool on[kTiles];
};

// Shared main loop: 32 activation rows (staged from `src`, rows s_src[m], a
// row-major [*, K] matrix of float32 or bfloat16) times kTiles MXFP4 weight
// tiles per wavefront. Global loads run kDepth steps ahead through a register
// ring; the activation tile is double-buffered in LDS, one barrier per step.
template <bool BF16>
__device__ __forceinline__ void mx_gemm_mainloop(const void *src, int K, const int *s_src,
                                                 ATile &sa, BTiles bt, f32x16_t (&acc)[kTiles]) {
    const int lane = threadIdx.x & 63;
    const int gsel = lane >> 5, l32 = lane & 31;
    const int arow = threadIdx.x >> 3, achunk = threadIdx.x & 7;
    const int asrc = s_src[arow];
    const int nsteps = (K + 63) / 64;
#pragma unroll
    for (int i = 0; i < kTiles; ++i)
        if (!bt.on[i]) bt.row[i] = 0;  // disabled tiles load row 0: loads stay unconditional
    AStage<BF16> ast[kDepth];
    uint4 bq[kDepth][kTiles];
    uint32_t bs[kDepth][kTiles];
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
        const int sd = min(d, nsteps - 1);
        ast[d].load(src, K, asrc, 64 * sd + 8 * achunk, K);
#pragma unroll
        for (int i = 0; i < kTiles; ++i) load_mx(bt.q[i], bt.sc[i], bt.row[i], K, 2 * sd + gsel, bq[d][i], bs[d][i]);
    }
    for (int s0 = 0; s0 < nsteps; s0 += kDepth) {
#pragma unroll
        for (int d = 0; d < kDepth; ++d) {
            const int s = s0 + d;
            if (s < nsteps) {
                const int buf = s & 1;
                ast[d].store(sa, buf, arow, achunk);
                uint4 w[kTiles];
                float f[kTiles];
#pragma unroll
                for (int i = 0; i < kTiles; ++i) {
                    w[i] = bq[d][i];
                    f[i] = e8m0_scale(bs[d][i]);
                }
                __syncthreads();
                {
                    // refill the slot unconditionally (the last kDepth steps
                    // reload step nsteps-1; those values are never used)
                    const int sn = min(s + kDepth, nsteps - 1);
                    ast[d].load(src, K, asrc, 64 * sn + 8 * achunk, K);
#pragma unroll
                    for (int i = 0; i < kTiles; ++i)
                        load_mx(bt.q[i], bt.sc[i], bt.row[i], K, 2 * sn + gsel, bq[d][i], bs[d][i]);
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int off = swz(l32, gsel * 4 + j);
                    const bf16x8_t ah = *reinterpret_cast<const bf16x8_t *>(&sa[buf][0][l32][off]);
                    bf16x8_t al;
                    if constexpr (!BF16) al = *reinterpret_cast<const bf16x8_t *>(&sa[buf][1][l32][off]);
#pragma unroll
                    for (int i = 0; i < kTiles; ++i) {
                        if (bt.on[i]) {
                            const bf16x8_t bw = fp4x8_to_bf16(dword(w[i], j), f[i]);
                            acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bw, acc[i], 0, 0, 0);
                            if constexpr (!BF16)
                                acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bw, acc[i], 0, 0, 0);
                        }
                    }
                }
            }
        }
    }
}

// ---------------------------------------------------------------- gate/up
// Workgroup tile: 32 rows of one expert x kGateUpBN = 256 features (4 waves x
// 2 subtiles of 32), gate and up each; epilogue adds the biases, applies the
// clamped SwiGLU and stores the float32 activation row of each route.
template <bool BF16>
__global__ __launch_bounds__(256) void gate_up_gemm_kernel(
    const void *x, int T, int H, int F, int E, int n_shared, int k, ExpertPtrs ex,
    ExpertPtrs sh, SwigluConsts sc, const int32_t *offsets, const int32_t *perm,
    const int32_t *mprefix, float *act) {
    static_assert(kGateUpBN == 4 * 2 * 32, "gate/up tile: 4 waves x 2 subtiles x 32 features");
    const int G = E + n_shared;
    const int NT = (F + kGateUpBN - 1) / kGateUpBN;
    int tile;
    if (!xcd_tile(blockIdx.x, mprefix[G] * NT, tile)) return;
    __shared__ int s_pre[kMaxE + 2];
    const TileInfo ti = find_tile(tile, NT, G, mprefix, offsets, s_pre);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int gsel = lane >> 5, l32 = lane & 31;
    const uint8_t *blob = ti.g < E ? ex.base + static_cast<size_t>(ti.g) * ex.stride : sh.base;

    __shared__ int s_src[kBM];
    __shared__ __align__(16) ATile s_a;
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

    const int base = ti.nt * kGateUpBN + 64 * w;
    const int n0 = base + l32, n1 = base + 32 + l32;  // features of the two subtiles
    BTiles bt;
    bt.q[0] = blob + ex.gate_q; bt.sc[0] = blob + ex.gate_s; bt.row[0] = n0; bt.on[0] = base < F;
    bt.q[1] = blob + ex.up_q;   bt.sc[1] = blob + ex.up_s;   bt.row[1] = n0; bt.on[1] = base < F;
    bt.q[2] = blob + ex.gate_q; bt.sc[2] = blob + ex.gate_s; bt.row[2] = n1; bt.on[2] = base + 32 < F;
    bt.q[3] = blob + ex.up_q;   bt.sc[3] = blob + ex.up_s;   bt.row[3] = n1; bt.on[3] = base + 32 < F;
    f32x16_t acc[kTiles];
#pragma unroll
    for (int i = 0; i < kTiles; ++i) acc[i] = f32x16_t{};
    mx_gemm_mainloop<BF16>(x, H, s_src, s_a, bt, acc);
    const float *gb = reinterpret_cast<const float *>(blob + ex.gate_b);
    const float *ub = reinterpret_cast<const float *>(blob + ex.up_b);
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
        if (!bt.on[2 * sub]) continue;
        const int n = sub == 0 ? n0 : n1;
        const float bgate = gb[n], bup = ub[n];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int m = 8 * (v >> 2) + 4 * gsel + (v & 3);
            if (m < ti.rows)
                act[static_cast<size_t>(ti.row0 + m) * F + n] =
                    swiglu(acc[2 * sub][v] + bgate, acc[2 * sub + 1][v] + bup, sc.alpha, sc.limit,
                           sc.up_offset);
        }
    }
}

// ---------------------------------------------------------------- down
// Workgroup tile: 32 rows of one expert x kDownBN = 512 hidden units (4 waves
// x 4 subtiles of 32); epilogue adds the down bias, multiplies by the route
// weight and adds into the token's output row (which holds the residual).
__global__ __launch_bounds__(256) void down_gemm_kernel(
    int T, int H, int F, int E, int n_shared, int k, ExpertPtrs ex, ExpertPtrs sh,
    const int32_t *offsets, const int32_t *perm, const float *wts, const int32_t *mprefix,
    const float *act, float *out) {
    static_assert(kDownBN == 4 * kTiles * 32, "down tile: 4 waves x kTiles subtiles x 32 rows");
    const int G = E + n_shared;
    const int NT = (H + kDownBN - 1) / kDownBN;
    int tile;
    if (!xcd_tile(blockIdx.x, mprefix[G] * NT, tile)) return;
    __shared__ int s_pre[kMaxE + 2];
    const TileInfo ti = find_tile(tile, NT, G, mprefix, offsets, s_pre);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int gsel = lane >> 5, l32 = lane & 31;
    const uint8_t *blob = ti.g < E ? ex.base + static_cast<size_t>(ti.g) * ex.stride : sh.base;

    __shared__ int s_src[kBM];
    __shared__ int s_tok[kBM];
    __shared__ float s_wt[kBM];
    __shared__ __align__(16) ATile s_a;
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

    BTiles bt;
#pragma unroll
    for (int i = 0; i < kTiles; ++i) {
        const int base = ti.nt * kDownBN + (w * kTiles + i) * 32;
        bt.q[i] = blob + ex.down_q;
        bt.sc[i] = blob + ex.down_s;
        bt.row[i] = base + l32;
        bt.on[i] = base < H;
    }
    f32x16_t acc[kTiles];
#pragma unroll
    for (int i = 0; i < kTiles; ++i) acc[i] = f32x16_t{};
    mx_gemm_mainloop<false>(act, F, s_src, s_a, bt, acc);
    const float *db = reinterpret_cast<const float *>(blob + ex.down_b);
#pragma unroll
    for (int i = 0; i < kTiles; ++i) {
        if (!bt.on[i]) continue;
        const int hr = ti.nt * kDownBN + (w * kTiles + i) * 32 + l32;
        const float bias = db[hr];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int m = 8 * (v >> 2) + 4 * gsel + (v & 3);
            if (m < ti.rows)
                unsafeAtomicAdd(out + static_cast<size_t>(s_tok[m]) * H + hr,
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
