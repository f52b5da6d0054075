// Prefill: grouped GEMMs over the routed rows in expert order, on the
// block-scaled matrix cores (MXFP4 weights as operand A, FP8-term activations
// as operand B).
//
// A work item is (weight-row block, tile of up to kGemmBM rows of one expert). Its
// workgroup of 4 wavefronts streams the weight rows once per tile, each
// wavefront its own rows (4 A fragments per 128-wide step, read as contiguous
// kilobytes from the tiled plane, kRing steps ahead), while the tile's rows x
// kTerms terms are staged per step through LDS (double-buffered) and shared
// by the 4 wavefronts: up to 4 B fragments, 16 matrix-core instructions per
// wavefront per step. Items are dealt so that the tiles of one expert and row block run
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
#include <type_traits>

#include "mx_mfma.hpp"

namespace moe {

namespace {

constexpr int kRowGroups = kGemmBM / 4;         // B operands per step (4 rows each)
constexpr int kBRowBytes = 128 + 16;            // one (row, term) step in LDS, padded
constexpr int kBBufBytes = kGemmBM * kTerms * kBRowBytes;
constexpr int kThreads = kGemmWaves * 64;
constexpr int kStage = kGemmBM * kTerms * 128 / 16 / kThreads;  // 16-byte B pieces per thread per step
constexpr int kRing = 3;                        // K-steps of A fragments in flight per wavefront
static_assert(kStage * kThreads * 16 == kGemmBM * kTerms * 128, "B staging covers the tile");
static_assert(kGemmBM * kTerms <= kThreads, "B scale staging: one dword per thread");
static_assert(kStage == 2, "the main loop stages B in two named registers");

struct Tile {
    int g;   // group: expert, or E for the shared expert
    int p0;  // first row position
    int n;   // rows in the tile (1..kGemmBM)
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

// Main loop: acc[j][rg] += A fragment j x B row group rg over all K-steps
// (aq[j] / as[j]: the tile bases of A fragment j),
// for the row groups that hold tile rows (n of them). A fragments stream
// through a register ring kRing steps deep (unrolled, so a slot is always the
// same registers and its refill waits on nothing); B pieces run 2 steps ahead
// and go through double-buffered LDS to be shared by the wavefronts (one
// barrier per step); every load is issued unconditionally with its step clamped into
// range.
template <int NA>
__device__ __forceinline__ void gemm_mainloop(const uint8_t *const (&aq)[NA],
                                              const uint8_t *const (&as)[NA], const ALane &al,
                                              int NS, const uint8_t *bq, const uint8_t *bs,
                                              int Kb, const int *s_brow, int n, uint8_t *sB,
                                              uint32_t *sBs, f32x4_t (&acc)[NA][kRowGroups]) {
    const int tid = threadIdx.x, lane = tid & 63;
    // staging pieces q = tid and tid + kThreads: (row, term, 16-byte chunk)
    const int q0 = tid, q1 = tid + kThreads;
    const uint8_t *src0 = bq + (static_cast<size_t>(s_brow[q0 >> 5]) * kTerms + ((q0 >> 3) & 3)) * Kb + 16 * (q0 & 7);
    const uint8_t *src1 = bq + (static_cast<size_t>(s_brow[q1 >> 5]) * kTerms + ((q1 >> 3) & 3)) * Kb + 16 * (q1 & 7);
    const int dst0 = ((q0 >> 5) * kTerms + ((q0 >> 3) & 3)) * kBRowBytes + 16 * (q0 & 7);
    const int dst1 = ((q1 >> 5) * kTerms + ((q1 >> 3) & 3)) * kBRowBytes + 16 * (q1 & 7);
    const bool sc_on = tid < kGemmBM * kTerms;
    const int srow = sc_on ? tid >> 2 : 0, sterm = tid & 3;
    const uint32_t *ssrc = reinterpret_cast<const uint32_t *>(
        bs + (static_cast<size_t>(s_brow[srow]) * kTerms + sterm) * (Kb / 32));
    const int ngroups = (n + 3) >> 2;  // row groups holding tile rows

    // Loads run ahead of use: A fragments kRing = 3 steps, B pieces 2 steps.
    // Vector loads complete in issue order, so within a step B(s+2) is issued
    // before A(s+3): waiting for B(s) then leaves A(s+1), A(s+2) in flight.
    // Slots are named (A slot s % 3, B slot and LDS buffer s % 2; the pattern
    // repeats every 6 steps) so that no slot is ever indexed at run time. All
    // loads are unconditional with their step clamped into range; the steps
    // past NS in the last round skip their matrix-core work.
    typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
    struct BSlot {
        u32x4_t b0, b1;  // this thread's two B pieces
        uint32_t bs;     // B scale dword (threads < kGemmBM * kTerms)
    };
    struct ASlot {
        AFrag a[NA];
    };
    auto fill_b = [&](BSlot &sl, int step) __attribute__((always_inline)) {
        const int sd = min(step, NS - 1);
        sl.b0 = *reinterpret_cast<const u32x4_t *>(src0 + 128 * sd);
        sl.b1 = *reinterpret_cast<const u32x4_t *>(src1 + 128 * sd);
        sl.bs = ssrc[sd];
    };
    auto fill_a = [&](ASlot &sl, int step) __attribute__((always_inline)) {
        const int sd = min(step, NS - 1);
#pragma unroll
        for (int j = 0; j < NA; ++j) sl.a[j] = load_afrag(aq[j], as[j], al, sd);
    };
    const int bn = lane & 15, bh = lane >> 4;
    const int brd = ((bn >> 2) * kTerms + (bn & 3)) * kBRowBytes + 16 * bh;
    auto step = [&](auto lbuf, BSlot &bsl, ASlot &asl, int s) __attribute__((always_inline)) {
        constexpr int L = decltype(lbuf)::value;
        uint8_t *buf = sB + L * kBBufBytes;
        uint32_t *sbuf = sBs + L * (kGemmBM * kTerms);
        *reinterpret_cast<u32x4_t *>(buf + dst0) = bsl.b0;
        *reinterpret_cast<u32x4_t *>(buf + dst1) = bsl.b1;
        if (sc_on) sbuf[tid] = bsl.bs;
        fill_b(bsl, s + 2);
        __syncthreads();
        if (s < NS) {  // uniform; no loads inside
#pragma unroll
            for (int rg = 0; rg < kRowGroups; ++rg) {
                if (rg < ngroups) {
                    const int off = brd + rg * 4 * kTerms * kBRowBytes;
                    const uint4 blo = *reinterpret_cast<const uint4 *>(buf + off);
                    const uint4 bhi = *reinterpret_cast<const uint4 *>(buf + off + 64);
                    const uint32_t bsc = (sbuf[(4 * rg + (bn >> 2)) * kTerms + (bn & 3)] >> (8 * bh)) & 0xffu;
#pragma unroll
                    for (int j = 0; j < NA; ++j) acc[j][rg] = mx_mfma(asl.a[j], blo, bhi, bsc, acc[j][rg]);
                }
            }
        }
        fill_a(asl, s + kRing);
    };
    static_assert(kRing == 3, "three named A slots");
    ASlot a0, a1, a2;
    BSlot b0, b1;
    fill_a(a0, 0);
    fill_b(b0, 0);
    fill_a(a1, 1);
    fill_b(b1, 1);
    fill_a(a2, 2);
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    for (int s0 = 0; s0 < NS; s0 += 6) {
        step(I0{}, b0, a0, s0);
        step(I1{}, b1, a1, s0 + 1);
        step(I0{}, b0, a2, s0 + 2);
        step(I1{}, b1, a0, s0 + 3);
        step(I0{}, b0, a1, s0 + 4);
        step(I1{}, b1, a2, s0 + 5);
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
    const int last_tile = F / 16 - 1, nblk = H / 32;
    const int t0 = min(f0 / 16, last_tile), t1 = min(f0 / 16 + 1, last_tile);
    const uint8_t *const aq[4] = {blob + ex.gate_q + tile_code_base(t0, nblk), blob + ex.gate_q + tile_code_base(t1, nblk),
                                  blob + ex.up_q + tile_code_base(t0, nblk), blob + ex.up_q + tile_code_base(t1, nblk)};
    const uint8_t *const as[4] = {blob + ex.gate_s + tile_scale_base(t0, nblk), blob + ex.gate_s + tile_scale_base(t1, nblk),
                                  blob + ex.up_s + tile_scale_base(t0, nblk), blob + ex.up_s + tile_scale_base(t1, nblk)};
    const ALane al(nblk, lane);
    f32x4_t acc[4][kRowGroups];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int rg = 0; rg < kRowGroups; ++rg) acc[j][rg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int Kp = pad128(H);
    gemm_mainloop<4>(aq, as, al, Kp / 128, xq, xs, Kp, s_brow, tl.n, sB, sBs, acc);

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
    for (int r0 = 0; r0 < tl.n; r0 += 2) {
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
    const int last_tile = H / 16 - 1, nblk = F / 32;
    const uint8_t *aq[4], *as[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int tj = min(h0 / 16 + j, last_tile);
        aq[j] = blob + ex.down_q + tile_code_base(tj, nblk);
        as[j] = blob + ex.down_s + tile_scale_base(tj, nblk);
    }
    const ALane al(nblk, lane);
    f32x4_t acc[4][kRowGroups];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int rg = 0; rg < kRowGroups; ++rg) acc[j][rg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int Fp = pad128(F);
    gemm_mainloop<4>(aq, as, al, Fp / 128, act_q, act_s, Fp, s_brow, tl.n, sB, sBs, acc);

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
