// Prefill: grouped GEMMs over the routed rows in expert order, on the
// block-scaled matrix cores (MXFP4 weights as operand A, FP8-term activations
// as operand B).
//
// The FP8 terms of an activation row are laid along K: for each 128-wide
// step, term n of 16 rows is one B operand (column c = row c of the group),
// and the terms' instructions accumulate into the same result. So a 16x16
// result tile holds 16 weight rows x 16 activation rows outright. gate/up
// uses all kTerms terms of a float32 input and three of a bfloat16 one; down
// uses kDownTerms of the SwiGLU output.
//
// A work item is (tile of up to 16*NG rows of one expert, weight-row block).
// Its workgroup of W wavefronts streams the block's weight rows once per tile:
// each wavefront has its own rows and NA A fragments per step, read as
// contiguous kilobytes from the tiled plane 2-3 steps ahead. The tile's rows x
// terms are staged 2 steps ahead through double-buffered LDS and shared by the
// W wavefronts. Per step a wavefront issues NA x NG x (terms used)
// matrix-core instructions, less for row groups of 16 the tile does not fill. Items are
// dealt so that the row blocks of one tile run back to back on one
// accelerator die and share its activation rows in L2.
//
// gate/up: NA/2 16-row tiles of each matrix per wavefront. The epilogue adds
// the biases, applies the clamped SwiGLU and writes the FP8 terms of each
// 32-feature block per row (the down GEMM's operand). down: NA 16-row tiles
// per wavefront. The epilogue adds the bias and writes route weight x result
// as the row's fp32 output y[p]; the combine kernel then adds each token's
// rows to its residual in a fixed order (no atomics, deterministic).
//
// Page: goosedump `gpt_oss.rs`, `mixture_of_experts` and its grouped form over
// expert-sorted rows (`mixture_of_experts_batch`); DeepSeek-V4 shared expert
// (ungated, weight 1).
#include <type_traits>

#include "mx_mfma.hpp"

namespace moe {

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Tile geometry: NG row groups of 16 per tile, W wavefronts per workgroup,
// NA A fragments (16-row weight tiles) per wavefront.
template <int NG, int W, int NA>
struct Geo {
    static constexpr int kThreads = 64 * W;
    static constexpr int kRows = 16 * NG;                  // activation rows per tile
    static constexpr int kPieces = kTerms * NG * 8 * 16;   // 16-byte B pieces per step
    static constexpr int kPerThread = kPieces / kThreads;  // pieces staged per thread
    static constexpr int kBufBytes = kPieces * 16;
    static constexpr int kScales = kRows * kTerms;         // B scale dwords per step
    static constexpr int kGURowsWave = 8 * NA;             // gate/up features per wavefront
    static constexpr int kGateUpRows = W * kGURowsWave;    // features per gate/up workgroup
    static constexpr int kDownRows = W * 16 * NA;          // hidden rows per down workgroup
    // K-steps of A fragments in flight: 3 for 32-row tiles in 8-wavefront
    // workgroups; 2 for 16-row tiles (at most 128 VGPRs: four workgroups per
    // CU, which beats three with a deeper ring), for 32-row tiles in
    // 4-wavefront workgroups (three workgroups per CU within 168 VGPRs: the
    // 24-layer stack 6.64 -> 6.36 ms per step against two per CU with a
    // third step in flight) and for 64-row tiles
    static constexpr int kASlots = (NG == 2 && W == 8) ? 3 : 2;
    // K-steps of B staged ahead in registers: 2, or 1 for 64-row tiles (a
    // step of their B is 128 bytes per thread)
    static constexpr int kBAhead = NG == 4 ? 1 : 2;
    static_assert(NG == 1 || NG == 2 || NG == 4, "16-, 32- or 64-row tiles");
    static_assert(kPieces % kThreads == 0, "B staging divides evenly");
    static_assert(kScales <= kThreads, "one scale dword per thread at most");
    static_assert(kGateUpRows % 32 == 0, "gate/up blocks hold whole 32-feature MX blocks");
};

struct Tile {
    int g;   // group: expert, or E for the shared expert
    int p0;  // first row position
    int n;   // rows in the tile (1..16*NG)
};

// Work item of this workgroup, dealt XCD-major (items i and i+1 run back to
// back on one die). Items run group by group; inside a group (an expert's
// tiles x the row blocks) row block by row block, and inside a row block tile
// by tile: all tiles of an expert that need the same weight rows run side by
// side and share them in L2, and a tile's row blocks follow each other (its
// activation rows stay in L2 too); groups with many tiles and row blocks go
// tile by tile instead (below). False when past the real tiles.
__device__ __forceinline__ bool find_item(int nrb, int bm, const int32_t *offsets,
                                          const int *s_pre, int G, int &rb, Tile &tl) {
    // the real item count splits evenly over the dies (the grid is an upper
    // bound; dealing by grid size would leave the last dies without work)
    const int total = s_pre[G] * nrb;
    const int per = (total + kXcds - 1) / kXcds;
    const int xi = blockIdx.x / kXcds;  // this workgroup's turn on its die
    if (xi >= per) return false;
    const int item = (blockIdx.x % kXcds) * per + xi;
    if (item >= total) return false;
    int lo = 0, hi = G - 1;  // last group whose first item is <= item
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_pre[mid] * nrb <= item) lo = mid;
        else hi = mid - 1;
    }
    const int nt = s_pre[lo + 1] - s_pre[lo];  // >= 1: a group with no tiles owns no items
    const int local = item - s_pre[lo] * nrb;
    // a group with many tiles and many row blocks (the shared expert at the
    // DeepSeek-V4-Pro shape) runs tile by tile, a tile's row blocks back to
    // back, so its activation rows stay in L2 while the weights stream (7%
    // faster per step there); with fewer row blocks (the Flash shape, 16) the
    // row-block order measured 1% faster, and routed experts have few tiles
    int tile;
    if (nt >= 16 && nrb >= 20) {
        tile = local / nrb;
        rb = local - tile * nrb;
    } else {
        rb = local / nt;
        tile = local - rb * nt;
    }
    tl.g = lo;
    tl.p0 = offsets[lo] + tile * bm;
    tl.n = min(bm, offsets[lo + 1] - tl.p0);
    return true;
}

// Main loop: acc[j][g] += A fragment j x (row group g, all terms) over all
// K-steps (aq[j] / as[j]: the tile bases of A fragment j; brow: per tile row,
// the FP8-term row index in bq / bs, row stride kTerms).
//
// Loads run ahead of use: A fragments kASlots (3 or 2) steps, B pieces 2
// steps. Vector loads complete in issue order, so within a step B(s+2) is
// issued before A(s+kASlots): waiting for B(s) leaves the later A fragments
// in flight. Slots are named (A slot s % kASlots, B slot and LDS buffer s % 2;
// the pattern repeats every 6 or 2 steps) so that no slot is indexed at run
// time. All loads are unconditional with their step clamped into range; the
// steps past NS in the last round skip their matrix-core work.
//
// LDS holds a step's B pieces in fragment order: piece p = ((term * NG +
// group) * 8 + chunk) * 16 + column, so the 16 lanes of one k-group read 256
// contiguous bytes; the B scale bytes sit in lane order, [term][k-group][row].
// Only the NT terms that meet the A fragments are staged (three of the four
// stored: a quarter less B traffic through L2 and LDS per step); when the
// pieces do not divide evenly over the threads, the last threads reload and
// rewrite the last piece (the same bytes to the same place).
template <int NG, int W, int NA, int NT>
__device__ __forceinline__ void gemm_mainloop(const uint8_t *const (&aq)[NA],
                                              const uint8_t *const (&as)[NA], const ALane &al,
                                              int NS, const uint8_t *bq, const uint8_t *bs, int Kb,
                                              const int *s_brow, int n, uint8_t *sB, uint8_t *sBs,
                                              f32x4_t (&acc)[NA][NG]) {
    using Gm = Geo<NG, W, NA>;
    constexpr int kThreads = Gm::kThreads;
    constexpr int kPcs = NT * NG * 8 * 16;                    // staged pieces per step
    constexpr int kPT = (kPcs + kThreads - 1) / kThreads;     // per thread
    constexpr int kScl = Gm::kRows * NT;                      // staged scale dwords per step
    static_assert(kScl <= kThreads, "one scale dword per thread at most");
    const int tid = threadIdx.x, lane = tid & 63;
    // this thread's B pieces: byte offsets from bq at step 0, and LDS slots
    uint32_t soff[kPT];
    int sdp[kPT];
#pragma unroll
    for (int i = 0; i < kPT; ++i) {
        const int p = min(tid + kThreads * i, kPcs - 1);
        const int col = p & 15, chunk = (p >> 4) & 7, grp = (p >> 7) % NG, term = (p >> 7) / NG;
        soff[i] = static_cast<uint32_t>((s_brow[16 * grp + col] * kTerms + term) * Kb + 16 * chunk);
        sdp[i] = 16 * p;
    }
    // threads < kScl stage the scale dword (blocks 4s..4s+3) of one (row, term)
    const bool sc_on = tid < kScl;
    const int stok = sc_on ? tid / NT : 0, sterm = tid % NT;
    const uint32_t *ssrc = reinterpret_cast<const uint32_t *>(
        bs + (static_cast<size_t>(s_brow[stok]) * kTerms + sterm) * (Kb / 32));
    const int sdst = sterm * 4 * Gm::kRows + stok;  // byte of k-group h at sdst + h * kRows
    const int ngroups = (n + 15) >> 4;               // row groups holding tile rows

    struct BSlot {
        u32x4_t b[kPT];
        uint32_t s;
    };
    struct ASlot {
        AFrag a[NA];
    };
    auto fill_b = [&](BSlot &sl, int step) __attribute__((always_inline)) {
        const int sd = min(step, NS - 1);
#pragma unroll
        for (int i = 0; i < kPT; ++i)
            sl.b[i] = *reinterpret_cast<const u32x4_t *>(bq + soff[i] + 128 * sd);
        sl.s = ssrc[sd];
    };
    auto fill_a = [&](ASlot &sl, int step) __attribute__((always_inline)) {
        const int sd = min(step, NS - 1);
#pragma unroll
        for (int j = 0; j < NA; ++j) sl.a[j] = load_afrag(aq[j], as[j], al, sd);
    };
    const int col = lane & 15, kh = lane >> 4;
    auto step = [&](auto lbuf, BSlot &bsl, ASlot &asl, int s) __attribute__((always_inline)) {
        constexpr int L = decltype(lbuf)::value;
        uint8_t *buf = sB + L * Gm::kBufBytes;
        uint8_t *sbuf = sBs + L * 4 * Gm::kScales;
#pragma unroll
        for (int i = 0; i < kPT; ++i) *reinterpret_cast<u32x4_t *>(buf + sdp[i]) = bsl.b[i];
        if (sc_on) {
#pragma unroll
            for (int h = 0; h < 4; ++h) sbuf[sdst + h * Gm::kRows] = static_cast<uint8_t>(bsl.s >> (8 * h));
        }
        fill_b(bsl, s + 2);
        __syncthreads();
        if (s < NS) {  // uniform; no loads inside
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                if (g < ngroups) {  // uniform: row groups the tile fills
                    // term t + 1's LDS reads are issued before term t's
                    // instructions (two B operands live), so the reads'
                    // latency hides behind the matrix core; the scheduling
                    // barriers keep the compiler from hoisting every term's
                    // reads into registers the tile needs
                    uint4 blo[2], bhi[2];
                    uint32_t bsc[2];
                    auto rd = [&](int t, int sl) __attribute__((always_inline)) {
                        const int pc = ((t * NG + g) * 8 + kh) * 16 + col;
                        blo[sl] = *reinterpret_cast<const uint4 *>(buf + 16 * pc);
                        bhi[sl] = *reinterpret_cast<const uint4 *>(buf + 16 * (pc + 64));
                        bsc[sl] = sbuf[(t * 4 + kh) * Gm::kRows + 16 * g + col];
                    };
                    rd(0, 0);
#pragma unroll
                    for (int t = 0; t < NT; ++t) {
                        if (t + 1 < NT) rd(t + 1, (t + 1) & 1);
                        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                        for (int j = 0; j < NA; ++j)
                            acc[j][g] = mx_mfma(asl.a[j], blo[t & 1], bhi[t & 1], bsc[t & 1], acc[j][g]);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            }
        }
        fill_a(asl, s + Gm::kASlots);
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    if constexpr (Gm::kBAhead == 1) {
        // one B slot, refilled for the next step right after its data is in
        // LDS; the A ring as for 16-row tiles
        auto step1 = [&](auto lbuf, BSlot &bsl, ASlot &asl, int s) __attribute__((always_inline)) {
            constexpr int L = decltype(lbuf)::value;
            uint8_t *buf = sB + L * Gm::kBufBytes;
            uint8_t *sbuf = sBs + L * 4 * Gm::kScales;
#pragma unroll
            for (int i = 0; i < kPT; ++i) *reinterpret_cast<u32x4_t *>(buf + sdp[i]) = bsl.b[i];
            if (sc_on) {
#pragma unroll
                for (int h = 0; h < 4; ++h) sbuf[sdst + h * Gm::kRows] = static_cast<uint8_t>(bsl.s >> (8 * h));
            }
            fill_b(bsl, s + 1);
            __syncthreads();
            if (s < NS) {  // uniform; no loads inside
#pragma unroll
                for (int g = 0; g < NG; ++g) {
                    if (g < ngroups) {  // uniform: row groups the tile fills
                        // one term's B at a time: the other wavefront on the
                        // SIMD covers the LDS latency, and the registers stay
                        // within two wavefronts per SIMD
#pragma unroll
                        for (int t = 0; t < NT; ++t) {
                            const int pc = ((t * NG + g) * 8 + kh) * 16 + col;
                            const uint4 blo = *reinterpret_cast<const uint4 *>(buf + 16 * pc);
                            const uint4 bhi = *reinterpret_cast<const uint4 *>(buf + 16 * (pc + 64));
                            const uint32_t bsc = sbuf[(t * 4 + kh) * Gm::kRows + 16 * g + col];
#pragma unroll
                            for (int j = 0; j < NA; ++j)
                                acc[j][g] = mx_mfma(asl.a[j], blo, bhi, bsc, acc[j][g]);
                            __builtin_amdgcn_sched_barrier(0);
                        }
                    }
                }
            }
            fill_a(asl, s + Gm::kASlots);
        };
        ASlot a0, a1;
        BSlot b0;
        fill_b(b0, 0);
        __builtin_amdgcn_sched_barrier(0);
        fill_a(a0, 0);
        __builtin_amdgcn_sched_barrier(0);
        fill_a(a1, 1);
        __builtin_amdgcn_sched_barrier(0);
        for (int s0 = 0; s0 < NS; s0 += 2) {
            step1(I0{}, b0, a0, s0);
            step1(I1{}, b0, a1, s0 + 1);
        }
    } else if constexpr (Gm::kASlots == 3) {
        ASlot a0, a1, a2;
        BSlot b0, b1;
        fill_a(a0, 0);
        fill_b(b0, 0);
        fill_a(a1, 1);
        fill_b(b1, 1);
        fill_a(a2, 2);
        for (int s0 = 0; s0 < NS; s0 += 6) {
            step(I0{}, b0, a0, s0);
            step(I1{}, b1, a1, s0 + 1);
            step(I0{}, b0, a2, s0 + 2);
            step(I1{}, b1, a0, s0 + 3);
            step(I0{}, b0, a1, s0 + 4);
            step(I1{}, b1, a2, s0 + 5);
        }
    } else {
        // the prologue issues its loads in the loop's own order (B(s), A(s),
        // B(s+1), A(s+1)), held there by scheduling barriers: the memory
        // waits at the loop head merge the prologue's order with the loop's,
        // and any other order makes every iteration wait for the next step's
        // loads as well
        ASlot a0, a1;
        BSlot b0, b1;
        fill_b(b0, 0);
        __builtin_amdgcn_sched_barrier(0);
        fill_a(a0, 0);
        __builtin_amdgcn_sched_barrier(0);
        fill_b(b1, 1);
        __builtin_amdgcn_sched_barrier(0);
        fill_a(a1, 1);
        __builtin_amdgcn_sched_barrier(0);
        for (int s0 = 0; s0 < NS; s0 += 2) {
            step(I0{}, b0, a0, s0);
            step(I1{}, b1, a1, s0 + 1);
        }
    }
}

// Main loop with an MX-FP4 expert input (the quantised expert-input mode):
// both operands FP4, one block-scaled instruction per A fragment and row
// group. A step's B is one 16-byte piece per (row, k-group): the 32 codes of
// MX block 4s + h of the row, from the packed rows bq[row][Kb / 2] with their
// scale bytes bs[row][Kb / 32]. Pieces are staged 2 steps ahead through
// double-buffered LDS (piece (group * 4 + h) * 16 + column, the scale dword of
// a row's four k-groups at its row), A fragments 2 steps ahead as in
// gemm_mainloop. All loads are unconditional (threads past the pieces reload
// one), so no branch sits between loads and matrix-core work.
template <int NG, int W, int NA>
__device__ __forceinline__ void gemm_mainloop_x4(const uint8_t *const (&aq)[NA],
                                                 const uint8_t *const (&as)[NA], const ALane &al,
                                                 int NS, const uint8_t *bq, const uint8_t *bs,
                                                 int Kb, const int *s_brow, int n, uint8_t *sB,
                                                 uint8_t *sBs, f32x4_t (&acc)[NA][NG]) {
    constexpr int kThreads = 64 * W;
    constexpr int kPieces = 64 * NG;     // per step
    constexpr int kRows = 16 * NG;
    constexpr int kBuf = 16 * kPieces;   // bytes per LDS buffer
    static_assert(kPieces <= kThreads && kRows <= kThreads, "one piece per thread");
    const int tid = threadIdx.x, lane = tid & 63;
    const int pc = tid % kPieces;
    const uint32_t soff = static_cast<uint32_t>(s_brow[16 * (pc >> 6) + (pc & 15)]) * (Kb / 2) +
                          16u * ((pc >> 4) & 3);
    const uint32_t *ssrc =
        reinterpret_cast<const uint32_t *>(bs + static_cast<size_t>(s_brow[tid % kRows]) * (Kb / 32));
    const int ngroups = (n + 15) >> 4;
    struct BSlot {
        u32x4_t b;
        uint32_t s;
    };
    struct ASlot {
        AFrag a[NA];
    };
    auto fill_b = [&](BSlot &sl, int step) __attribute__((always_inline)) {
        const int sd = min(step, NS - 1);
        sl.b = *reinterpret_cast<const u32x4_t *>(bq + soff + 64u * sd);
        sl.s = ssrc[sd];
    };
    auto fill_a = [&](ASlot &sl, int step) __attribute__((always_inline)) {
        const int sd = min(step, NS - 1);
#pragma unroll
        for (int j = 0; j < NA; ++j) sl.a[j] = load_afrag(aq[j], as[j], al, sd);
    };
    const int col = lane & 15, kh = lane >> 4;
    auto step = [&](auto lbuf, BSlot &bsl, ASlot &asl, int s) __attribute__((always_inline)) {
        constexpr int L = decltype(lbuf)::value;
        uint8_t *buf = sB + L * kBuf;
        uint32_t *sbuf = reinterpret_cast<uint32_t *>(sBs) + L * kRows;
        if (tid < kPieces) *reinterpret_cast<u32x4_t *>(buf + 16 * tid) = bsl.b;
        if (tid < kRows) sbuf[tid] = bsl.s;
        fill_b(bsl, s + 2);
        __syncthreads();
        if (s < NS) {  // uniform; no loads inside
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                if (g < ngroups) {  // uniform: row groups the tile fills
                    const uint4 blo = *reinterpret_cast<const uint4 *>(buf + 16 * ((g * 4 + kh) * 16 + col));
                    const uint32_t bsc = reinterpret_cast<const uint8_t *>(sbuf)[4 * (16 * g + col) + kh];
#pragma unroll
                    for (int j = 0; j < NA; ++j) acc[j][g] = mx_mfma_fp4(asl.a[j], blo, bsc, acc[j][g]);
                }
            }
        }
        fill_a(asl, s + 2);
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    ASlot a0, a1;
    BSlot b0, b1;
    fill_b(b0, 0);
    __builtin_amdgcn_sched_barrier(0);
    fill_a(a0, 0);
    __builtin_amdgcn_sched_barrier(0);
    fill_b(b1, 1);
    __builtin_amdgcn_sched_barrier(0);
    fill_a(a1, 1);
    __builtin_amdgcn_sched_barrier(0);
    for (int s0 = 0; s0 < NS; s0 += 2) {
        step(I0{}, b0, a0, s0);
        step(I1{}, b1, a1, s0 + 1);
    }
}

// Main loop with the bfloat16 expert input itself as operand B (a bfloat16
// input with no RMSNorm in between): the MXFP4 weights are decoded to
// bfloat16 in registers with the scaled FP4 converts (exact: an E2M1 value
// times 2^n is a bfloat16 for scale bytes 1..252) and multiplied on the
// bfloat16 matrix cores, v_mfma_f32_16x16x32_bf16, one instruction per
// 32-wide slice of K instead of one per FP8 term: two thirds of the
// matrix-core time of three terms, and two bytes per activation staged
// instead of three. The products are exact and accumulate in float32, as on
// the FP8-term path.
//
// K order: an A fragment (16 B per lane) holds the 32 codes of k-group
// h = l / 16 of its row; instruction j (0..3) of a step takes codes 8j..8j+7
// of every lane, so lane group h stands for k = 32h + 8j .. 32h + 8j + 7, and
// B lane (column c, group h) supplies the same k of its row. The result layout
// is that of the block-scaled instruction (lane l: rows 4 (l / 16) + v of
// column l % 16).
//
// LDS holds a step's B rows, 128 values (256 B) each at a 272-byte stride (the
// 16 lanes of a k-group read 16 B each from 16 rows on distinct banks); rows
// are staged 2 steps ahead through two buffers, 16-byte pieces, consecutive
// threads along a row. A piece at or past K = H loads as zeros (buffer
// bounds), so the ragged last step adds nothing; x is [T][H] bfloat16.
constexpr int kBfRow = 272;  // LDS bytes per staged bfloat16 row
template <int NG>
__host__ __device__ constexpr int bf_stage_bytes() { return 16 * NG * kBfRow; }

template <int NG, int W, int NA>
__device__ __forceinline__ void gemm_mainloop_bf(const uint8_t *const (&aq)[NA],
                                                 const uint8_t *const (&as)[NA], const ALane &al,
                                                 int NS, const uint8_t *x, int T, int H,
                                                 const int *s_brow, int n, uint8_t *sB,
                                                 f32x4_t (&acc)[NA][NG]) {
    constexpr int kThreads = 64 * W;
    constexpr int kPcs = NG * 16 * 16;                     // 16-byte pieces per step
    constexpr int kPT = (kPcs + kThreads - 1) / kThreads;  // per thread
    constexpr int kBuf = bf_stage_bytes<NG>();
    constexpr uint32_t kOob = 0x80000000u;                 // past the buffer: loads zeros
    constexpr int kRawFlags = 0x00020000;
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(x), 0, static_cast<int>(2u * static_cast<uint32_t>(T) * H), kRawFlags);
    const int tid = threadIdx.x, lane = tid & 63;
    uint32_t roff[kPT];
    int kq[kPT], sdp[kPT];
#pragma unroll
    for (int i = 0; i < kPT; ++i) {
        const int p = min(tid + kThreads * i, kPcs - 1);
        const int r = p >> 4, q = p & 15;
        roff[i] = 2u * (static_cast<uint32_t>(s_brow[r]) * H + 8u * q);
        kq[i] = 8 * q;
        sdp[i] = r * kBfRow + 16 * q;
    }
    const int ngroups = (n + 15) >> 4;
    typedef int bf_i32x4 __attribute__((ext_vector_type(4)));
    struct BSlot {
        bf_i32x4 b[kPT];
    };
    struct ASlot {
        AFrag a[NA];
    };
    auto fill_b = [&](BSlot &sl, int step) __attribute__((always_inline)) {
        const int sd = min(step, NS - 1);
#pragma unroll
        for (int i = 0; i < kPT; ++i) {
            const uint32_t o = 128 * sd + kq[i] < H ? roff[i] + 256u * sd : kOob;
            sl.b[i] = __builtin_amdgcn_raw_buffer_load_b128(xr, o, 0, 0);
        }
    };
    auto fill_a = [&](ASlot &sl, int step) __attribute__((always_inline)) {
        const int sd = min(step, NS - 1);
#pragma unroll
        for (int j = 0; j < NA; ++j) sl.a[j] = load_afrag(aq[j], as[j], al, sd);
    };
    const int col = lane & 15, kh = lane >> 4;
    auto step = [&](auto lbuf, BSlot &bsl, ASlot &asl, int s) __attribute__((always_inline)) {
        constexpr int L = decltype(lbuf)::value;
        uint8_t *buf = sB + L * kBuf;
#pragma unroll
        for (int i = 0; i < kPT; ++i) *reinterpret_cast<bf_i32x4 *>(buf + sdp[i]) = bsl.b[i];
        fill_b(bsl, s + 2);
        __syncthreads();
        if (s < NS) {  // uniform; no loads inside
            float sc[NA];
#pragma unroll
            for (int jj = 0; jj < NA; ++jj) sc[jj] = e8m0_scale(asl.a[jj].s & 0xffu);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                bf16x8_t abf[NA];
#pragma unroll
                for (int jj = 0; jj < NA; ++jj) {
                    const uint32_t d = j == 0 ? asl.a[jj].q.x
                                     : j == 1 ? asl.a[jj].q.y
                                     : j == 2 ? asl.a[jj].q.z
                                              : asl.a[jj].q.w;
                    abf[jj] = fp4x8_to_bf16(d, sc[jj]);
                }
#pragma unroll
                for (int g = 0; g < NG; ++g) {
                    if (g < ngroups) {  // uniform: row groups the tile fills
                        const bf16x8_t b = *reinterpret_cast<const bf16x8_t *>(
                            buf + (16 * g + col) * kBfRow + 64 * kh + 16 * j);
#pragma unroll
                        for (int jj = 0; jj < NA; ++jj)
                            acc[jj][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(abf[jj], b, acc[jj][g], 0, 0, 0);
                    }
                }
            }
        }
        fill_a(asl, s + 2);
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    ASlot a0, a1;
    BSlot b0, b1;
    fill_b(b0, 0);
    __builtin_amdgcn_sched_barrier(0);
    fill_a(a0, 0);
    __builtin_amdgcn_sched_barrier(0);
    fill_b(b1, 1);
    __builtin_amdgcn_sched_barrier(0);
    fill_a(a1, 1);
    __builtin_amdgcn_sched_barrier(0);
    for (int s0 = 0; s0 < NS; s0 += 2) {
        step(I0{}, b0, a0, s0);
        step(I1{}, b1, a1, s0 + 1);
    }
}

__device__ __forceinline__ void load_pre(const int32_t *mprefix, int G, int *s_pre) {
    for (int i = threadIdx.x; i <= G; i += blockDim.x) s_pre[i] = mprefix[i];
    __syncthreads();
}

// gate/up: grid = kXcds-rounded max_tiles x ceil(pad128(F) / kGateUpRows) items;
// NT (3 or 4) FP8 terms of the expert input take part, or (NT = 1) the
// bfloat16 input itself, or (NT = 0) its MX-FP4 codes.
// Q4A: the SwiGLU output leaves as MX-FP4 codes (act_q [rows][Fp / 2], one
// scale byte per 32 values in act_s [rows][Fp / 32]) instead of FP8 terms.
// 16-row tiles are held to 4 wavefronts per SIMD (128 VGPRs, no spills),
// 32-row FP8-term tiles in 4-wavefront workgroups to 3 (168 VGPRs), 64-row
// tiles with the bfloat16 or MX-FP4 operand and 2 A fragments per wavefront
// to 4 (two 8-wavefront workgroups per CU).
template <int NG, int W, int NA, int NT, bool Q4A>
__global__ __launch_bounds__(64 * W, NG == 1 ? 4 : (W == 4 ? (NG == 2 && NT >= 3 ? 3 : 2) : (NT <= 1 && NA == 2 ? 4 : 1))) void gate_up_gemm_kernel(
    const uint8_t *xq, const uint8_t *xs, int T, int H, int F, int E, int k, int n_shared,
    ExpertPtrs ex, ExpertPtrs sh, SwigluConsts sc, const int32_t *offsets, const int32_t *perm,
    const int32_t *mprefix, uint8_t *act_q, uint8_t *act_s) {
    using Gm = Geo<NG, W, NA>;
    constexpr int kTilesPerMat = NA / 2;   // 16-row tiles of gate (and of up) per wavefront
    constexpr int kActStride = Gm::kGateUpRows + 1;
    __shared__ int s_pre[kMaxE + 2];
    __shared__ int s_brow[Gm::kRows];
    // B staging buffers; after the main loop the workgroup's SwiGLU outputs
    // ([rows][kGateUpRows + 1] floats) reuse them
    constexpr int kActBytes = Gm::kRows * kActStride * 4;
    constexpr int kStageBytes = NT == 1 ? 2 * bf_stage_bytes<NG>() : 2 * Gm::kBufBytes;
    __shared__ __align__(16) uint8_t sB[kStageBytes > kActBytes ? kStageBytes : kActBytes];
    __shared__ __align__(16) uint8_t sBs[2 * 4 * Gm::kScales];  // dword-read by the FP4 main loop
    __shared__ float s_bias[2][Gm::kGateUpRows];  // gate, up biases of the workgroup's features
    const int G = E + n_shared, R = T * k;
    load_pre(mprefix, G, s_pre);
    const int Fp = pad128(F), nrb = (Fp + Gm::kGateUpRows - 1) / Gm::kGateUpRows;
    int rb;
    Tile tl;
    if (!find_item(nrb, Gm::kRows, offsets, s_pre, G, rb, tl)) return;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint8_t *blob = tl.g < E ? ex.base + static_cast<size_t>(tl.g) * ex.stride : sh.base;
    const int fw = rb * Gm::kGateUpRows;          // the workgroup's first feature
    if (tid < Gm::kRows) {
        const int p = tl.p0 + min(tid, tl.n - 1);
        s_brow[tid] = p < R ? perm[p] / k : p - R;  // the token (x row)
    }
    // the epilogue's biases, fetched now rather than after the main loop
    for (int i = tid; i < 2 * Gm::kGateUpRows; i += Gm::kThreads) {
        const int m = i / Gm::kGateUpRows, fl = i - m * Gm::kGateUpRows;
        const float *bp = reinterpret_cast<const float *>(blob + (m ? ex.up_b : ex.gate_b));
        s_bias[m][fl] = fw + fl < F ? bp[fw + fl] : 0.f;
    }
    __syncthreads();
    const int f0 = fw + Gm::kGURowsWave * w;     // this wavefront's first feature
    const int last_tile = F / 16 - 1, nblk = H / 32;
    const uint8_t *aq[NA], *as[NA];
#pragma unroll
    for (int j = 0; j < kTilesPerMat; ++j) {
        const int tj = min(f0 / 16 + j, last_tile);
        aq[j] = blob + ex.gate_q + tile_code_base(tj, nblk);
        as[j] = blob + ex.gate_s + tile_scale_base(tj, nblk);
        aq[kTilesPerMat + j] = blob + ex.up_q + tile_code_base(tj, nblk);
        as[kTilesPerMat + j] = blob + ex.up_s + tile_scale_base(tj, nblk);
    }
    const ALane al(nblk, lane);
    f32x4_t acc[NA][NG];
#pragma unroll
    for (int j = 0; j < NA; ++j)
#pragma unroll
        for (int g = 0; g < NG; ++g) acc[j][g] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int Kp = pad128(H);
    if constexpr (NT == 0)  // MX-FP4 expert input
        gemm_mainloop_x4<NG, W, NA>(aq, as, al, Kp / 128, xq, xs, Kp, s_brow, tl.n, sB, sBs, acc);
    else if constexpr (NT == 1)  // the bfloat16 expert input (xq: x [T][H])
        gemm_mainloop_bf<NG, W, NA>(aq, as, al, Kp / 128, xq, T, H, s_brow, tl.n, sB, acc);
    else
        gemm_mainloop<NG, W, NA, NT>(aq, as, al, Kp / 128, xq, xs, Kp, s_brow, tl.n, sB, sBs, acc);

    // epilogue: SwiGLU of the workgroup's features into LDS, then one
    // 32-feature block per (row, block) to FP8 terms (or MX-FP4 codes)
    __syncthreads();  // the staging buffers become the SwiGLU outputs
    float *sAct = reinterpret_cast<float *>(sB);
    const int col = lane & 15, kh = lane >> 4;
    if (f0 < F) {  // F % 16 == 0: a wavefront's features are all real or all padding
#pragma unroll
        for (int j = 0; j < kTilesPerMat; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int fl = Gm::kGURowsWave * w + 16 * j + 4 * kh + v;  // feature - fw
                const float bg = s_bias[0][fl], bu = s_bias[1][fl];
#pragma unroll
                for (int g = 0; g < NG; ++g)
                    sAct[(16 * g + col) * kActStride + fl] =
                        swiglu(acc[j][g][v] + bg, acc[kTilesPerMat + j][g][v] + bu, sc.alpha, sc.limit,
                               sc.up_offset);
            }
    }
    __syncthreads();
    // (row, block) tasks, two per half-wavefront at a time (their reduction
    // chains interleave); blocks at or past F are the K padding of the down
    // GEMM's operand (zero codes), blocks past Fp skipped
    constexpr int kBlocks = Gm::kGateUpRows / 32;
    const int half = lane >> 5, i = lane & 31, nbp = Fp / 32;
    const int ntask = tl.n * kBlocks;
    if constexpr (Q4A) {
        // one (row, block) per half-wavefront at a time; every lane takes part
        // in the block maximum, blocks at or past F are zeros (code 0)
        for (int task0 = 2 * w; task0 < ntask; task0 += 2 * W) {
            const int task = task0 + half;
            const bool on = task < ntask;
            const int row = on ? task / kBlocks : 0;
            const int blk = on ? task - row * kBlocks : 0;
            const int fb = fw + 32 * blk;
            const float v = on && fb < F ? sAct[row * kActStride + 32 * blk + i] : 0.f;
            uint32_t sbyte;
            const uint32_t pair = fp4_pack_pair(fp4_act_code(v, sbyte));
            if (on && fb < Fp) {
                const size_t p = static_cast<size_t>(tl.p0 + row);
                if ((i & 1) == 0) act_q[p * (Fp / 2) + fb / 2 + (i >> 1)] = static_cast<uint8_t>(pair);
                if (i == 0) act_s[p * nbp + fb / 32] = static_cast<uint8_t>(sbyte);
            }
        }
        return;
    }
    for (int task0 = 4 * w; task0 < ntask; task0 += 4 * W) {
        int row[2], fb[2];
        bool on[2];
        uint32_t codes[2], scales[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int task = task0 + 2 * u + half;
            on[u] = task < ntask;
            row[u] = on[u] ? task / kBlocks : 0;
            const int blk = on[u] ? task - row[u] * kBlocks : 0;
            fb[u] = fw + 32 * blk;  // first feature of the block
            const float v = fb[u] < F ? sAct[row[u] * kActStride + 32 * blk + i] : 0.f;
            fp8_terms_group(v, codes[u], scales[u]);  // every lane takes part
            if (fb[u] >= F) {
                codes[u] = 0;
                scales[u] = 0x7f7f7f7fu;
            }
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            if (on[u] && fb[u] < Fp) {
                const size_t p = static_cast<size_t>(tl.p0 + row[u]);
#pragma unroll
                for (int n = 0; n < kDownTerms; ++n) {  // the terms the down GEMM reads
                    act_q[(p * kTerms + n) * Fp + fb[u] + i] = static_cast<uint8_t>(codes[u] >> (8 * n));
                    if (i == 0)
                        act_s[(p * kTerms + n) * nbp + fb[u] / 32] = static_cast<uint8_t>(scales[u] >> (8 * n));
                }
            }
        }
    }
}

// down: grid = kXcds-rounded max_tiles x ceil(H / kDownRows) items. A4: the
// activation rows are MX-FP4 codes (FP4 x FP4 products) instead of FP8 terms.
// With MX-FP4 rows and 2 A fragments per wavefront: 4 wavefronts per SIMD.
template <int NG, int W, int NA, bool A4>
__global__ __launch_bounds__(64 * W, A4 && NA == 2 ? 4 : 1) void down_gemm_kernel(
    const uint8_t *act_q, const uint8_t *act_s, int T, int H, int F, int E, int k, int n_shared,
    ExpertPtrs ex, ExpertPtrs sh, const int32_t *offsets, const int32_t *perm, const float *wts,
    const int32_t *mprefix, float *y) {
    using Gm = Geo<NG, W, NA>;
    __shared__ int s_pre[kMaxE + 2];
    __shared__ int s_brow[Gm::kRows];
    __shared__ float s_wt[Gm::kRows];
    __shared__ __align__(16) uint8_t sB[2 * Gm::kBufBytes];
    __shared__ __align__(16) uint8_t sBs[2 * 4 * Gm::kScales];  // dword-read by the FP4 main loop
    __shared__ __align__(16) float s_bias[Gm::kDownRows];  // biases of the workgroup's hidden rows
    const int G = E + n_shared, R = T * k;
    load_pre(mprefix, G, s_pre);
    const int nrb = (H + Gm::kDownRows - 1) / Gm::kDownRows;
    int rb;
    Tile tl;
    if (!find_item(nrb, Gm::kRows, offsets, s_pre, G, rb, tl)) return;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint8_t *blob = tl.g < E ? ex.base + static_cast<size_t>(tl.g) * ex.stride : sh.base;
    if (tid < Gm::kRows) {
        const int p = tl.p0 + min(tid, tl.n - 1);
        s_brow[tid] = p;  // activation rows are in position order
        s_wt[tid] = p < R ? wts[perm[p]] : 1.0f;
    }
    // the epilogue's biases, fetched now rather than after the main loop
    for (int i = tid; i < Gm::kDownRows; i += Gm::kThreads) {
        const int h = rb * Gm::kDownRows + i;
        s_bias[i] = h < H ? reinterpret_cast<const float *>(blob + ex.down_b)[h] : 0.f;
    }
    __syncthreads();
    const int h0 = rb * Gm::kDownRows + 16 * NA * w;  // this wavefront's hidden rows
    const int last_tile = H / 16 - 1, nblk = F / 32;
    const uint8_t *aq[NA], *as[NA];
#pragma unroll
    for (int j = 0; j < NA; ++j) {
        const int tj = min(h0 / 16 + j, last_tile);
        aq[j] = blob + ex.down_q + tile_code_base(tj, nblk);
        as[j] = blob + ex.down_s + tile_scale_base(tj, nblk);
    }
    const ALane al(nblk, lane);
    f32x4_t acc[NA][NG];
#pragma unroll
    for (int j = 0; j < NA; ++j)
#pragma unroll
        for (int g = 0; g < NG; ++g) acc[j][g] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int Fp = pad128(F);
    if constexpr (A4)
        gemm_mainloop_x4<NG, W, NA>(aq, as, al, Fp / 128, act_q, act_s, Fp, s_brow, tl.n, sB, sBs, acc);
    else
        gemm_mainloop<NG, W, NA, kDownTerms>(aq, as, al, Fp / 128, act_q, act_s, Fp, s_brow, tl.n, sB,
                                             sBs, acc);

    // y[p][h] = route weight x (down + bias), four consecutive h per lane
    const int col = lane & 15, kh = lane >> 4;
#pragma unroll
    for (int j = 0; j < NA; ++j) {
        const int h = h0 + 16 * j + 4 * kh;
        if (h < H) {  // H % 16 == 0: the lane's four rows are all in or all out
            const float4 bias = *reinterpret_cast<const float4 *>(s_bias + (h - rb * Gm::kDownRows));
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                const int row = 16 * g + col;
                if (row < tl.n) {
                    const float wt = s_wt[row];
                    const float4 yv = make_float4(wt * (acc[j][g][0] + bias.x), wt * (acc[j][g][1] + bias.y),
                                                  wt * (acc[j][g][2] + bias.z), wt * (acc[j][g][3] + bias.w));
                    *reinterpret_cast<float4 *>(y + static_cast<size_t>(tl.p0 + row) * H + h) = yv;
                }
            }
        }
    }
}

// out[t] = resid[t] + sum over slots j of y[inv[t*k + j]] (+ y[T*k + t] for the
// shared expert), added in that fixed order; four hidden units per thread.
__global__ __launch_bounds__(256) void combine_kernel(const float *y, const int32_t *inv, int T,
                                                      int H, int k, int n_shared,
                                                      const void *resid, int resid_bf16,
                                                      float *out) {
    const int H4 = H / 4;
    const long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= static_cast<long long>(T) * H4) return;
    const int t = static_cast<int>(i / H4), h = 4 * static_cast<int>(i - static_cast<long long>(t) * H4);
    float4 a;
    if (resid_bf16) {
        const uint2 rb = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(resid) +
                                                          static_cast<size_t>(t) * H + h);
        a = make_float4(bf16_bits_to_f32(rb.x & 0xffffu), bf16_bits_to_f32(rb.x >> 16),
                        bf16_bits_to_f32(rb.y & 0xffffu), bf16_bits_to_f32(rb.y >> 16));
    } else {
        a = *reinterpret_cast<const float4 *>(static_cast<const float *>(resid) + static_cast<size_t>(t) * H + h);
    }
    for (int j = 0; j < k; ++j) {
        const float4 v = *reinterpret_cast<const float4 *>(y + static_cast<size_t>(inv[t * k + j]) * H + h);
        a.x += v.x; a.y += v.y; a.z += v.z; a.w += v.w;
    }
    if (n_shared) {
        const float4 v = *reinterpret_cast<const float4 *>(y + (static_cast<size_t>(T) * k + t) * H + h);
        a.x += v.x; a.y += v.y; a.z += v.z; a.w += v.w;
    }
    *reinterpret_cast<float4 *>(out + static_cast<size_t>(t) * H + h) = a;
}


int items(int nrb, int max_tiles) {
    const long long n = static_cast<long long>(nrb) * max_tiles;
    return static_cast<int>((n + kXcds - 1) / kXcds * kXcds);
}

}  // namespace

// Tile rows and input terms of the grouped GEMMs for a shape, from the
// average rows per group (an expert's routes, or the shared expert's T rows)
// and the work items a tile size makes (tiles x weight-row blocks):
//  - 64-row tiles (8 wavefronts, 256 features per gate/up workgroup) when
//    groups average at least 30 rows and the items fill the GPU about eight
//    times over: each weight fragment feeds up to 4 row groups, so an expert's
//    weights stream once (DeepSeek-V4 Flash 1.91 -> 1.58 ms per layer, Pro
//    5.54 -> 4.99 ms); with few items the last round runs mostly empty (the
//    24-layer stack: 7.46 -> 8.71 ms);
//  - 32-row tiles from 24 rows on average (the stack, 64 rows per expert:
//    7.46 -> 6.98 ms with 8 wavefronts; with FP8 terms 4 wavefronts and 128
//    features per gate/up workgroup, two workgroups per CU);
//  - 16-row tiles (4 wavefronts, four per CU) below (the T = 128 layer).
// A bfloat16 expert input with no RMSNorm in between (x_bf16_exact) is
// operand B itself on the bfloat16 matrix cores (x_terms 1). Otherwise tiles
// of 32 rows and more take three FP8 terms of the expert input (a fourth does
// not fit two wavefronts' registers per SIMD at 64 rows and was slower at
// 32); 16-row tiles take four of a float32 input. An MX-FP4 expert input
// (x_fp4) is one FP4 operand (x_terms 0).
GemmPlan gemm_plan(int T, int k, int E, int n_shared, int F, bool x_bf16_exact, bool x_fp4,
                   bool act_fp4) {
    const double rows = static_cast<double>(T) * (k + n_shared);
    const int groups = E + n_shared;
    const double avg = rows / groups;
    const double items64 = (rows / 64.0 + 0.5 * groups) * ((pad128(F) + 255) / 256);
    GemmPlan p;
    if (avg >= 30.0 && items64 >= 2048.0) p.tile_rows = 64;
    else if (avg >= 24.0) p.tile_rows = 32;
    else p.tile_rows = 16;
    p.x_terms = x_fp4 ? 0 : x_bf16_exact ? 1 : p.tile_rows >= 32 ? 3 : kTerms;
    p.act_terms = act_fp4 ? 0 : kDownTerms;
    // 128 features: 4-wavefront workgroups, or 8 wavefronts of two A
    // fragments (64-row tiles with the bfloat16 or MX-FP4 operand)
    p.gate_up_features = p.tile_rows == 16 || (p.tile_rows == 32 && p.x_terms == 3) ||
                                 (p.tile_rows == 64 && p.x_terms <= 1)
                             ? 128
                             : 256;
    p.down_rows = p.tile_rows == 64 && p.act_terms != 0 ? 512 : 256;
    return p;
}

// 16-row tiles: 4 wavefronts with 4 A fragments each (four workgroups per
// CU); 32-row tiles with FP8 terms, and the 32-row down GEMM: 4 wavefronts,
// three workgroups per CU (their barriers do not hold each other: 4% faster
// per gate/up launch than 8 wavefronts on the 24-layer stack, though each
// workgroup covers half the features); 64-row tiles with the bfloat16
// operand: 8 wavefronts with 2 A fragments each (96 VGPRs, two workgroups per
// CU: DeepSeek-V4-Flash gate/up 664 -> 593 us against 4 fragments and one
// workgroup per CU); otherwise 8 wavefronts with 4 A fragments each.
hipError_t launch_gate_up_gemm(const uint8_t *xq, const uint8_t *xs, int T, int H, int F, int E,
                               int k, int n_shared, const ExpertPtrs &ex, const ExpertPtrs &sh,
                               SwigluConsts c, const int32_t *offsets, const int32_t *perm,
                               const int32_t *mprefix, int tile_rows, int max_tiles, int x_terms,
                               bool act_fp4, uint8_t *act_q, uint8_t *act_s, hipStream_t s) {
    if (act_fp4 && x_terms != 0) return hipErrorInvalidValue;  // the FP4 output comes with the FP4 input
#define MOE_GU(NG, W, NA, NT)                                                                       \
    do {                                                                                            \
        using Gm = Geo<NG, W, NA>;                                                                  \
        const int grid = items((pad128(F) + Gm::kGateUpRows - 1) / Gm::kGateUpRows, max_tiles);    \
        if (grid == 0) return hipSuccess;                                                           \
        if constexpr ((NT) == 0) {  /* the FP4 output comes only with the FP4 input */          \
            if (act_fp4) {                                                                          \
                launch_kernel(gate_up_gemm_kernel<NG, W, NA, NT, true>, grid, 64 * (W), s, xq, xs, \
                              T, H, F, E, k, n_shared, ex, sh, c, offsets, perm, mprefix, act_q,    \
                              act_s);                                                               \
                break;                                                                              \
            }                                                                                       \
        }                                                                                           \
        launch_kernel(gate_up_gemm_kernel<NG, W, NA, NT, false>, grid, 64 * (W), s, xq, xs, T, H,  \
                      F, E, k, n_shared, ex, sh, c, offsets, perm, mprefix, act_q, act_s);          \
    } while (0)
    if (x_terms < 0 || x_terms == 2 || x_terms > kTerms) return hipErrorInvalidValue;
    switch (tile_rows * 10 + x_terms) {
    case 160: MOE_GU(1, 4, 4, 0); break;
    case 320: MOE_GU(2, 8, 4, 0); break;
    case 640: MOE_GU(4, 8, 2, 0); break;
    case 161: MOE_GU(1, 4, 4, 1); break;
    case 321: MOE_GU(2, 8, 4, 1); break;
    case 641: MOE_GU(4, 8, 2, 1); break;
    case 163: MOE_GU(1, 4, 4, 3); break;
    case 164: MOE_GU(1, 4, 4, 4); break;
    case 323: MOE_GU(2, 4, 4, 3); break;
    case 643: MOE_GU(4, 8, 4, 3); break;
    default: return hipErrorInvalidValue;
    }
#undef MOE_GU
    return hipGetLastError();
}

hipError_t launch_down_gemm(const uint8_t *act_q, const uint8_t *act_s, int T, int H, int F, int E,
                            int k, int n_shared, const ExpertPtrs &ex, const ExpertPtrs &sh,
                            const int32_t *offsets, const int32_t *perm, const float *wts,
                            const int32_t *mprefix, int tile_rows, int max_tiles, bool act_fp4,
                            float *y, hipStream_t s) {
#define MOE_DN(NG, W, NA, A4)                                                                       \
    do {                                                                                            \
        using Gm = Geo<NG, W, NA>;                                                                  \
        const int grid = items((H + Gm::kDownRows - 1) / Gm::kDownRows, max_tiles);                 \
        if (grid == 0) return hipSuccess;                                                           \
        launch_kernel(down_gemm_kernel<NG, W, NA, A4>, grid, 64 * (W), s, act_q, act_s, T, H, F, E, \
                      k, n_shared, ex, sh, offsets, perm, wts, mprefix, y);                         \
    } while (0)
    switch (tile_rows * 2 + (act_fp4 ? 1 : 0)) {
    case 32: MOE_DN(1, 4, 4, false); break;
    case 33: MOE_DN(1, 4, 4, true); break;
    case 64: MOE_DN(2, 4, 4, false); break;
    case 65: MOE_DN(2, 4, 4, true); break;
    case 128: MOE_DN(4, 8, 4, false); break;
    case 129: MOE_DN(4, 8, 2, true); break;  // 97 VGPRs: two workgroups per CU
    default: return hipErrorInvalidValue;
    }
#undef MOE_DN
    return hipGetLastError();
}

hipError_t launch_combine(const float *y, const int32_t *inv, int T, int H, int k, int n_shared,
                          const void *resid, int resid_bf16, float *out, hipStream_t s) {
    const long long n = static_cast<long long>(T) * (H / 4);
    const int grid = static_cast<int>((n + 255) / 256);
    if (grid == 0) return hipSuccess;
    launch_kernel(combine_kernel, grid, 256, s, y, inv, T, H, k, n_shared, resid, resid_bf16, out);
    return hipGetLastError();
}

}  // namespace moe
