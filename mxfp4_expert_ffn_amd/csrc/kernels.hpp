// Host-side launchers of the MoE kernels (internal to the library).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kXcds = 8;   // MI355X: 8 accelerator dies; workgroups are dealt round-robin
constexpr int kMaxK = 8;   // experts per token
constexpr int kMaxE = 512; // routed experts (DeepSeek-V4-Pro has 384)
constexpr int kMaxQ = kMaxE / 64;  // experts per lane in a wavefront's top-k
constexpr int kTerms = 4;  // FP8 terms per activation on the block-scaled matrix cores

// Grouped GEMMs: tiles of 16, 32 or 64 routed rows of one expert
// (gemm_plan), which the permutation's tile prefix also uses.
// Decode GEMVs: 8 wavefronts per workgroup; gate/up takes 32 weight rows of
// one route, K split over the wavefronts; down takes 16 output rows of one
// token over all its routes.
constexpr int kDecodeWaves = 8;

// Packed MXFP4 plane of `rows` x K weights (rows and K multiples of 32), as
// laid out in an expert blob: rows in tiles of 16, K in steps of 128 (four
// 32-value MX blocks); inside a (tile, step) the 16-byte code blocks run
// block-major then row, so the 64 lanes of a wavefront, lane = 16 * block +
// row, read one contiguous kilobyte, which is also the A operand of the
// block-scaled 16x16x128 matrix-core instruction. Scale bytes follow the same
// order, one byte per code block. A ragged last step holds only its blocks.
__host__ __device__ constexpr uint64_t mx_code_offset(uint32_t row, uint32_t blk, uint32_t nblk) {
    return static_cast<uint64_t>(row >> 4) * (256ull * nblk) + static_cast<uint64_t>(blk >> 2) * 1024ull +
           static_cast<uint64_t>(((blk & 3u) << 4) | (row & 15u)) * 16ull;
}
__host__ __device__ constexpr uint64_t mx_scale_offset(uint32_t row, uint32_t blk, uint32_t nblk) {
    return static_cast<uint64_t>(row >> 4) * (16ull * nblk) + static_cast<uint64_t>(blk >> 2) * 64ull +
           (((blk & 3u) << 4) | (row & 15u));
}

// K padded to whole 128-wide steps (the FP8-term rows of activations).
__host__ __device__ constexpr int pad128(int k) { return (k + 127) / 128 * 128; }

// Events attached to the next kernel dispatch (the library's timing hook):
// hipExtLaunchKernel stamps them with that kernel's own start and end. Null
// events make it a plain launch. Thread-local, set by the C ABI layer.
struct LaunchEvents {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};
LaunchEvents &launch_events();

template <typename Kernel, typename... Args>
inline void launch_kernel(Kernel kernel, dim3 grid, dim3 block, hipStream_t s, Args... args) {
    const LaunchEvents &ev = launch_events();
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, ev.start, ev.stop, 0, args...);
}

// Same with `shm` bytes of dynamic LDS.
template <typename Kernel, typename... Args>
inline void launch_kernel_shm(Kernel kernel, dim3 grid, dim3 block, size_t shm, hipStream_t s,
                              Args... args) {
    const LaunchEvents &ev = launch_events();
    hipExtLaunchKernelGGL(kernel, grid, block, shm, s, ev.start, ev.stop, 0, args...);
}

struct ExpertPtrs {
    const uint8_t *base;     // first packed expert
    uint64_t stride;         // bytes between experts
    uint64_t gate_q, up_q, down_q, gate_s, up_s, down_s, gate_b, up_b, down_b;
};

struct SwigluConsts {
    float alpha, limit, up_offset;
};

// routing -----------------------------------------------------------------
// Input of the router and of the expert path: x (float32, or bf16 bits) or,
// with an RMSNorm, the fp64 value (x[t][h] * inv[t]) * gamma[h], which the
// router takes as is and the expert path rounds to float32.
struct RouteIn {
    const void *x;
    int bf16;
    const double *inv;   // [T] RMSNorm scale, or NULL: no norm
    const float *gamma;  // [H] norm weight (16-byte aligned) when inv is set
    float *seed;         // [T][H]: the quantisation also writes the raw input here
                         // as float32 (decode's residual seed), or NULL
};
// RMSNorm scale inv[t] = 1 / sqrt(sum_h x[t][h]^2 / H + eps), summed in fp64.
hipError_t launch_rms_inv(const void *x, int x_bf16, int T, int H, float eps, double *inv,
                          hipStream_t s);
// Router: split-K partial logits partial[splits][T][E] (fp64, bias not added).
// GEMV form for T <= kRouterGemvMaxT (one wavefront per expert and
// 512-wide hidden slice), tiled form otherwise (slices sized for about 1024
// workgroups, four per CU, at most kRouterMaxSplits: at DeepSeek-V4-Flash's
// T = 2048 the tiled router took 98 us against 113 us with about 512).
constexpr int kRouterGemvMaxT = 16;
constexpr int kRouterMaxSplits = 64;
// 512-wide slices: 2048 and 1024 were 1-3% slower per decode token, 256 much
// slower (the gate/up kernel's gather of the partials grows)
constexpr int kRouterGemvSlice = 512;
// Most quantisation workgroups beside the tiled router (grid-stride beyond).
constexpr int kQuantizeMaxWgs = 1024;
struct RouterPlan {
    bool gemv;
    int slice;   // hidden units per split
    int splits;  // S
};
RouterPlan router_plan(int T, int H, int E);
// FP8-term quantisation of the expert input (every forward), done by extra
// workgroups of the router launch: q [T][kTerms][Kp] E4M3 codes, scales
// [T][kTerms][Kp/32] E8M0 bytes, Kp = pad128(H), zero codes past H.
// fp4: the MX-FP4 round trip of the expert input instead (the quantised
// expert-input mode): codes packed two per byte, q [T][Kp / 2], one E8M0
// scale per 32 values, scales [T][Kp / 32], zero codes past H.
struct TermsOut {
    uint8_t *q;
    uint8_t *scales;
    int fp4;
};
// The MX-FP4 expert input alone, rows of H values: q [T][H / 2],
// scales [T][H / 32] (the quantised mode's debug export).
hipError_t launch_act_fp4(const RouteIn &in, int T, int H, uint8_t *q, uint8_t *scales,
                          hipStream_t s);
// `terms` NULL: router only.
hipError_t launch_router(const RouteIn &in, const float *w, int T, int H, int E, double *partial,
                         const TermsOut *terms, hipStream_t s);
// DeepSeek-V4 routing variants (page: antirez ds4.c `ds4_layer_weights`,
// `weights_validate_layout`: exp_probs_b [n_expert]; tid2eid [n_expert_used,
// n_vocab] for the first n_hash_layer layers). Readings: the selection-only
// bias is added to the logits that top-k ranks, the weights stay the softmax
// of the selected experts' own logits; a hash-routed token takes the k
// experts of its id's table row, in row order, weighted by their logits.
struct RouteSel {
    const float *bias;     // [E] selection-only bias, or NULL
    const int32_t *table;  // [vocab][k] experts per token id, or NULL (hash routing)
    const int32_t *ids;    // [T] token ids (with table)
    int vocab;
};
// rs: the routing variant (plain top-k when both pointers are NULL).
hipError_t launch_topk(const double *partial, int S, const float *bias, const RouteSel &rs, int T,
                       int E, int k, float route_scale, int32_t *idx, float *wts, int32_t *out_idx,
                       float *out_w, hipStream_t s);
// mprefix[g] = tiles of tile_rows rows before group g (groups: E experts,
// then the shared expert's T rows when n_shared). With `terms` (and `qin`,
// the expert input) the launch's other workgroups make the FP8 terms, as
// launch_router would; the permutation itself is one workgroup per 1024
// routes, so they run on otherwise idle compute units.
constexpr int kPermuteQuantizeWgs = 512;
hipError_t launch_permute(const int32_t *idx, int T, int E, int k, int n_shared, int tile_rows,
                          int32_t *counts, int32_t *offsets, int32_t *perm, int32_t *inv,
                          int32_t *mprefix, int32_t *out_counts,
                          int32_t *out_offsets, int32_t *out_perm, int32_t *out_inv,
                          uint64_t *route_counts, const RouteIn *qin, int H,
                          const TermsOut *terms, hipStream_t s);

// decode (T <= 64) -----------------------------------------------------------
// Route r < T*k is slot r % k of token r / k; r >= T*k is the shared expert of
// token r - T*k. act_q / act_s: FP8 terms of the SwiGLU output times the
// route weight, per route, [routes][kTerms][pad128(F)] codes and
// [routes][kTerms][pad128(F)/32] scales.
// Every gate/up workgroup selects its token's experts itself (top-k of the
// router's partial logits); slot 0's first feature block writes idx / wts and
// the optional exports.
struct DecodeArgs {
    const uint8_t *xq, *xs;  // FP8 terms of the expert input
    const double *partial;   // router partial logits [S][T][E]
    int S;
    const float *router_b;
    RouteSel rs;             // routing variant
    int T, H, F, E, k, n_shared;
    float route_scale;
    ExpertPtrs ex, sh;
    SwigluConsts sc;
    int32_t *idx;
    float *wts;
    int32_t *out_idx;  // optional exports (NULL: not written)
    float *out_w;
    uint64_t *route_counts;  // optional [E] profile: += 1 per selection (NULL: off)
    float *out;
    uint8_t *act_q, *act_s;
};
// gate/up (which also selects the experts), then down, which adds every route
// of a token into out in a fixed order (one writer per element); both after
// launch_router, whose quantisation seeds out with the residual (RouteIn::seed)
// unless out already is the float32 input.
hipError_t launch_decode_gate_up(const DecodeArgs &a, hipStream_t s);
hipError_t launch_decode_down(const DecodeArgs &a, hipStream_t s);

// prefill (any T) -------------------------------------------------------------
// Rows in expert order: position p < T*k is route perm[p]; p >= T*k is the
// shared expert of token p - T*k. act_q / act_s are indexed by p. tile_rows
// (16, 32 or 64) and x_terms come from gemm_plan, max_tiles bounds the tile
// count.
struct GemmPlan {
    int tile_rows;         // activation rows per tile
    int x_terms;           // FP8 terms of the expert input that take part (3 or kTerms), or 1:
                           // the bfloat16 input itself (bfloat16 matrix cores), or 0: the
                           // MX-FP4 expert input of the quantised mode
    int act_terms;         // FP8 terms of the SwiGLU output that take part, or 0: its
                           // MX-FP4 codes (quantised mode 2)
    int gate_up_features;  // features per gate/up workgroup
    int down_rows;         // hidden rows per down workgroup
};
// x_bf16_exact: the expert input is a bfloat16 value (no RMSNorm in between),
// taken as it is by the bfloat16 matrix cores.
// x_fp4: the quantised expert-input mode; act_fp4: its mode 2 (the SwiGLU
// output quantised too).
GemmPlan gemm_plan(int T, int k, int E, int n_shared, int F, bool x_bf16_exact, bool x_fp4,
                   bool act_fp4);
// x_terms: FP8 terms of the expert input that take part, 3 or kTerms (xq /
// xs: the term rows), 1 (xq: the bfloat16 input [T][H] itself), or 0 (MX-FP4
// input); act_fp4: the SwiGLU output leaves as MX-FP4 codes (needs x_terms 0).
hipError_t launch_gate_up_gemm(const uint8_t *xq, const uint8_t *xs, int T, int H, int F, int E,
                               int k, int n_shared, const ExpertPtrs &ex, const ExpertPtrs &sh,
                               SwigluConsts c, const int32_t *offsets, const int32_t *perm,
                               const int32_t *mprefix, int tile_rows, int max_tiles, int x_terms,
                               bool act_fp4, uint8_t *act_q, uint8_t *act_s, hipStream_t s);
// FP8 terms of the SwiGLU output that take part in the grouped down GEMM:
// the fourth moves the block output by under 3e-5 of its RMS on every
// configuration (the down GEMM averages the third term's rounding away).
constexpr int kDownTerms = 3;
// y [T*k + T*n_shared][H] fp32: route weight x (down + bias) per row position;
// act_fp4: the activation rows are MX-FP4 codes (quantised mode 2)
hipError_t launch_down_gemm(const uint8_t *act_q, const uint8_t *act_s, int T, int H, int F, int E,
                            int k, int n_shared, const ExpertPtrs &ex, const ExpertPtrs &sh,
                            const int32_t *offsets, const int32_t *perm, const float *wts,
                            const int32_t *mprefix, int tile_rows, int max_tiles, bool act_fp4,
                            float *y, hipStream_t s);
// out[t] = resid[t] + sum_j y[inv[t*k + j]] (+ y[T*k + t]); out may alias a float32 resid
hipError_t launch_combine(const float *y, const int32_t *inv, int T, int H, int k, int n_shared,
                          const void *resid, int resid_bf16, float *out, hipStream_t s);

// debug -------------------------------------------------------------------
// Decoded weights of one packed plane as float32 [rows][K]: path 0 through
// the scaled FP4 converts, path 1 through the bfloat16 converts, path 2
// through the block-scaled matrix core (one-hot FP8 operand B).
hipError_t launch_dequant(const uint8_t *codes, const uint8_t *scales, int rows, int K, int path,
                          float *out, hipStream_t s);

}  // namespace moe
