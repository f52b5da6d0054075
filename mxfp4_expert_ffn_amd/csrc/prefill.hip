// Prefill: grouped GEMMs over the routed rows in expert order, on the
// block-scaled matrix cores (MXFP4 weights as operand A, FP8-term activations
// as operand B).
//
// A work item is (weight-row block, tile of up to 32 rows of one expert). Its
// workgroup of 4 wavefronts streams the weight rows once per tile, each
// wavefront its own rows (4 A fragments per 128-wide step, read as contiguous
// kilobytes from the tiled plane), while the tile's 32 rows x kTerms terms
// are staged per step through LDS (double-buffered) and shared by the 4
// wavefronts: 8 B fragments, 32 matrix-core instructions per wavefront per
// step. Items are dealt so that the tiles of one expert and row block run
// back to back on one accelerator die and share its L2.
//
// gate/up: 32 features per wavefront for both matrices, epilogue adds the
// biases, applies the clamped SwiGLU and writes the FP8 terms of each
// 32-feature block per row (the down GEMM's operand). down: 64 hidden rows per
// wavefront, epilogue adds the bias and scatter-adds route weight x result
// into out[token] (which holds the residual).
//
// Page: goosedump `gpt_oss.rs`, `mixture_of_experts` and its grouped form over
// expert-sorted rows; DeepSeek-V4 shared expert (ungated, weight 1).
#include "mx_mfma.hpp"

namespace moe {

namespace {

constexpr int kRowGroups = kGemmBM / 4;         // B operands per step (4 rows each)
constexpr int kBRowBytes = 128 + 16;            // one (row, term) step in LDS, padded
constexpr int kBBufBytes = kGemmBM * kTerms * kBRowBytes;
constexpr int kThreads = kGemmWaves * 64;
static_assert(kGemmBM * kTerms * 128 / 16 == 4 * kThreads, "B staging: 4 x 16 bytes per thread");
static_assert(kGemmBM * kTerms == 128, "B scale staging: one dword per thread of the first 128");

struct Tile {
    int g;   // group: expert, or E for the shared expert
    int p0;  // first row position
    int n;   // rows in the tile (1..32)
};

// Work item of this workgroup, dealt XCD-major (items i and i+1 run back to
// back on one die); false when it is past the real tiles.
__device__ __forceinline__ bool find_item(int max_tiles, int nrb, const int32_t *offsets,
                                          const int *s_pre, int G, int &rb, Tile &tl) {
    const int per = gridDim.x / kXcds;
    const int item = (blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
    rb = item / max_tiles;
    const int tile = item - rb * max_tiles;
    if (rb >= nrb || tile >= s_pre[G]) return false;
    int lo = 0, hi = G - 1;  // last group whose first tile is <= tile
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_pre[mid] <= tile) lo = mid;
        else hi = mid - 1;
    }
    tl.g = lo;
    tl.p0 = offsets[lo] + (tile - s_pre[lo]) * kGemmBM;
    tl.n = min(kGemmBM, offsets[lo + 1] - tl.p0);
    return true;
}

// Main loop: acc[j][rg] += A fragment j x B row group rg over all K-steps.
// brow: per tile row, the FP8-term row index in bq / bs (row stride kTerms).
template <int NA>
__device__ __forceinline__ void gemm_mainloop(const uint8_t *const (&aq)[NA],
                                              const uint8_t *const (&as)[NA], const int (&atile)[NA],
                                              int nblk, int NS, const uint8_t *bq, const uint8_t *bs,
                                              int Kb, const int *s_brow, uint8_t *sB, uint32_t *sBs,
                                              f32x4_t (&acc)[NA][kRowGroups]) {
    const int tid = threadIdx.x, lane = tid & 63;
    // this thread's staging sources: 4 x 16 bytes of codes, one scale dword
    const uint8_t *src[4];
    int dst[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int q = tid + kThreads * i;
        const int row = q >> 5, term = (q >> 3) & 3, chunk = q & 7;
        src[i] = bq + (static_cast<size_t>(s_brow[row]) * kTerms + term) * Kb + 16 * chunk;
        dst[i] = (row * kTerms + term) * kBRowBytes + 16 * chunk;
    }
    const bool sc_on = tid < kGemmBM * kTerms;
    const int srow = sc_on ? tid >> 2 : 0, sterm = tid & 3;
    const uint32_t *ssrc = reinterpret_cast<const uint32_t *>(
        bs + (static_cast<size_t>(s_brow[srow]) * kTerms + sterm) * (Kb / 32));

    uint4 st[4];
    uint32_t sts = 0;
    AFrag an[NA];
#pragma unroll
    for (int i = 0; i < 4; ++i) st[i] = *reinterpret_cast<const uint4 *>(src[i]);
    if (sc_on) sts = ssrc[0];
#pragma unroll
    for (int j = 0; j < NA; ++j) an[j] = load_afrag(aq[j], as[j], atile[j], 0, nblk, lane);

    const int bn = lane & 15, bh = lane >> 4;
    const int brd = ((4 * 0 + (bn >> 2)) * kTerms + (bn & 3)) * kBRowBytes + 16 * bh;  // + group offset
    for (int s = 0; s < NS; ++s) {
        uint8_t *buf = sB + (s & 1) * kBBufBytes;
        uint32_t *sbuf = sBs + (s & 1) * (kGemmBM * kTerms);
#pragma unroll
        for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4 *>(buf + dst[i]) = st[i];
        if (sc_on) sbuf[tid] = sts;
        AFrag a[NA];
#pragma unroll
        for (int j = 0; j < NA; ++j) a[j] = an[j];
        if (s + 1 < NS) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                st[i] = *reinterpret_cast<const uint4 *>(src[i] + 128 * (s + 1));
            if (sc_on) sts = ssrc[s + 1];
#pragma unroll
            for (int j = 0; j < NA; ++j) an[j] = load_afrag(aq[j], as[j], atile[j], s + 1, nblk, lane);
        }
        __syncthreads();
#pragma unroll
        for (int rg = 0; rg < kRowGroups; ++rg) {
            const int off = brd + rg * 4 * kTerms * kBRowBytes;
            const uint4 blo = *reinterpret_cast<const uint4 *>(buf + off);
            const uint4 bhi = *reinterpret_cast<const uint4 *>(buf + off + 64);
            const uint32_t bsc = (sbuf[(4 * rg + (bn >> 2)) * kTerms + (bn & 3)] >> (8 * bh)) & 0xffu;
#pragma unroll
            for (int j = 0; j < NA; ++j) acc[j][rg] = mx_mfma(a[j], blo, bhi, bsc, acc[j][rg]);
        }
    }
}

__device__ __forceinline__ void load_pre(const int32_t *mprefix, int G, int *s_pre) {
    for (int i = threadIdx.x; i <= G; i += blockDim.x) s_pre[i] = mprefix[i];
    __syncthreads();
}

// gate/up: grid = kXcds-rounded (pad128(F) / 128) x max_tiles items.
__global__ __launch_bounds__(kThreads) void gate_up_gemm_kernel(
    const uint8_t *xq, const uint8_t *xs, int T, int H, int F, int E, int k, int n_shared,
    ExpertPtrs ex, ExpertPtrs sh, SwigluConsts sc, const int32_t *offsets, const int32_t *perm,
    const int32_t *mprefix, int max_tiles, uint8_t *act_q, uint8_t *act_s) {
    __shared__ int s_pre[kMaxE + 2];
    __shared__ int s_brow[kGemmBM];
    __shared__ __align__(16) uint8_t sB[2 * kBBufBytes];
    __shared__ uint32_t sBs[2 * kGemmBM * kTerms];
    __shared__ float sAct[kGemmWaves][kGemmBM][33];
    const int G = E + n_shared, R = T * k;
    load_pre(mprefix, G, s_pre);
    const int Fp = pad128(F), nrb = Fp / kGateUpRowsWG;
    int rb;
    Tile tl;
    if (!find_item(max_tiles, nrb, offsets, s_pre, G, rb, tl)) return;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    if (tid < kGemmBM) {
        const int p = tl.p0 + min(tid, tl.n - 1);
        s_brow[tid] = p < R ? perm[p] / k : p - R;  // the token (x row)
    }
    __syncthreads();
    const uint8_t *blob = tl.g < E ? ex.base + static_cast<size_t>(tl.g) * ex.stride : sh.base;
    const int f0 = rb * kGateUpRowsWG + 32 * w;  // this wavefront's 32 features
    const int last_tile = F / 16 - 1;
    const uint8_t *const aq[4] = {blob + ex.gate_q, blob + ex.gate_q, blob + ex.up_q, blob + ex.up_q};
    const uint8_t *const as[4] = {blob + ex.gate_s, blob + ex.gate_s, blob + ex.up_s, blob + ex.up_s};
    const int t0 = min(f0 / 16, last_tile), t1 = min(f0 / 16 + 1, last_tile);
    const int atile[4] = {t0, t1, t0, t1};
    f32x4_t acc[4][kRowGroups];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int rg = 0; rg < kRowGroups; ++rg) acc[j][rg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int Kp = pad128(H);
    gemm_mainloop<4>(aq, as, atile, H / 32, Kp / 128, xq, xs, Kp, s_brow, sB, sBs, acc);

    // epilogue: SwiGLU into LDS, then one 32-feature block per row to FP8 terms
    const bool live = f0 < F;  // F % 32 == 0: a wavefront is all features or all padding
    if (live) {
        const float *gb = reinterpret_cast<const float *>(blob + ex.gate_b);
        const float *ub = reinterpret_cast<const float *>(blob + ex.up_b);
        const int rq = (lane & 15) >> 2;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int fl = 16 * j + 4 * (lane >> 4) + v;
                const float bg = gb[f0 + fl], bu = ub[f0 + fl];
#pragma unroll
                for (int rg = 0; rg < kRowGroups; ++rg) {
                    // the quad sums run on every lane (DPP reads its neighbours)
                    const float g = quad_sum(acc[j][rg][v]), u = quad_sum(acc[2 + j][rg][v]);
                    if ((lane & 3) == 0)
                        sAct[w][4 * rg + rq][fl] = swiglu(g + bg, u + bu, sc.alpha, sc.limit, sc.up_offset);
                }
            }
    }
    __syncthreads();
    const int half = lane >> 5, i = lane & 31, nbp = Fp / 32;
    for (int r0 = 0; r0 < kGemmBM; r0 += 2) {
        const int row = r0 + half;
        uint32_t codes = 0, scales = 0x7f7f7f7fu;
        if (live) fp8_terms_group(sAct[w][row][i], codes, scales);
        if (row < tl.n) {
            const size_t p = static_cast<size_t>(tl.p0 + row);
#pragma unroll
            for (int n = 0; n < kTerms; ++n) {
                act_q[(p * kTerms + n) * Fp + f0 + i] = static_cast<uint8_t>(codes >> (8 * n));
                if (i == 0) act_s[(p * kTerms + n) * nbp + f0 / 32] = static_cast<uint8_t>(scales >> (8 * n));
            }
        }
    }
}

// down: grid = kXcds-rounded ceil(H / 256) x max_tiles items.
__global__ __launch_bounds__(kThreads) void down_gemm_kernel(
    const uint8_t *act_q, const uint8_t *act_s, int T, int H, int F, int E, int k, int n_shared,
    ExpertPtrs ex, ExpertPtrs sh, const int32_t *offsets, const int32_t *perm, const float *wts,
    const int32_t *mprefix, int max_tiles, float *out) {
    __shared__ int s_pre[kMaxE + 2];
    __shared__ int s_brow[kGemmBM];
    __shared__ int s_tok[kGemmBM];
    __shared__ float s_wt[kGemmBM];
    __shared__ __align__(16) uint8_t sB[2 * kBBufBytes];
    __shared__ uint32_t sBs[2 * kGemmBM * kTerms];
    const int G = E + n_shared, R = T * k;
    load_pre(mprefix, G, s_pre);
    const int nrb = (H + kDownRowsWG - 1) / kDownRowsWG;
    int rb;
    Tile tl;
    if (!find_item(max_tiles, nrb, offsets, s_pre, G, rb, tl)) return;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    if (tid < kGemmBM) {
        const int p = tl.p0 + min(tid, tl.n - 1);
        s_brow[tid] = p;  // activation rows are in position order
        if (p < R) {
            const int route = perm[p];
            s_tok[tid] = route / k;
            s_wt[tid] = wts[route];
        } else {
            s_tok[tid] = p - R;
            s_wt[tid] = 1.0f;
        }
    }
    __syncthreads();
    const uint8_t *blob = tl.g < E ? ex.base + static_cast<size_t>(tl.g) * ex.stride : sh.base;
    const int h0 = rb * kDownRowsWG + 64 * w;  // this wavefront's 64 hidden rows
    const int last_tile = H / 16 - 1;
    const uint8_t *const aq[4] = {blob + ex.down_q, blob + ex.down_q, blob + ex.down_q, blob + ex.down_q};
    const uint8_t *const as[4] = {blob + ex.down_s, blob + ex.down_s, blob + ex.down_s, blob + ex.down_s};
    const int atile[4] = {min(h0 / 16, last_tile), min(h0 / 16 + 1, last_tile),
                          min(h0 / 16 + 2, last_tile), min(h0 / 16 + 3, last_tile)};
    f32x4_t acc[4][kRowGroups];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int rg = 0; rg < kRowGroups; ++rg) acc[j][rg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int Fp = pad128(F);
    gemm_mainloop<4>(aq, as, atile, F / 32, Fp / 128, act_q, act_s, Fp, s_brow, sB, sBs, acc);

    const float *db = reinterpret_cast<const float *>(blob + ex.down_b);
    const int rq = (lane & 15) >> 2;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int h = h0 + 16 * j + 4 * (lane >> 4) + v;
            const float bias = h < H ? db[h] : 0.f;
#pragma unroll
            for (int rg = 0; rg < kRowGroups; ++rg) {
                const float y = quad_sum(acc[j][rg][v]);
                const int row = 4 * rg + rq;
                if ((lane & 3) == 0 && h < H && row < tl.n)
                    unsafeAtomicAdd(out + static_cast<size_t>(s_tok[row]) * H + h, s_wt[row] * (y + bias));
            }
        }
}

int items(int nrb, int max_tiles) {
    const long long n = static_cast<long long>(nrb) * max_tiles;
    return static_cast<int>((n + kXcds - 1) / kXcds * kXcds);
}

}  // namespace

hipError_t launch_gate_up_gemm(const uint8_t *xq, const uint8_t *xs, int T, int H, int F, int E,
                               int k, int n_shared, const ExpertPtrs &ex, const ExpertPtrs &sh,
                               SwigluConsts c, const int32_t *offsets, const int32_t *perm,
                               const int32_t *mprefix, int max_tiles, uint8_t *act_q,
                               uint8_t *act_s, hipStream_t s) {
    const int grid = items(pad128(F) / kGateUpRowsWG, max_tiles);
    if (grid == 0) return hipSuccess;
    launch_kernel(gate_up_gemm_kernel, grid, kThreads, s, xq, xs, T, H, F, E, k, n_shared, ex, sh,
                  c, offsets, perm, mprefix, max_tiles, act_q, act_s);
    return hipGetLastError();
}

hipError_t launch_down_gemm(const uint8_t *act_q, const uint8_t *act_s, int T, int H, int F, int E,
                            int k, int n_shared, const ExpertPtrs &ex, const ExpertPtrs &sh,
                            const int32_t *offsets, const int32_t *perm, const float *wts,
                            const int32_t *mprefix, int max_tiles, float *out, hipStream_t s) {
    const int grid = items((H + kDownRowsWG - 1) / kDownRowsWG, max_tiles);
    if (grid == 0) return hipSuccess;
    launch_kernel(down_gemm_kernel, grid, kThreads, s, act_q, act_s, T, H, F, E, k, n_shared, ex, sh,
                  offsets, perm, wts, mprefix, max_tiles, out);
    return hipGetLastError();
}

}  // namespace moe
