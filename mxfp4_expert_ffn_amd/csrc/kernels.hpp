// Host-side launchers of the MoE kernels (internal to the library).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kXcds = 8;   // MI355X: 8 accelerator dies; workgroups are dealt round-robin
constexpr int kMaxK = 8;   // experts per token
constexpr int kMaxE = 256; // routed experts
constexpr int kTerms = 4;  // FP8 terms per activation on the block-scaled matrix cores

// Tile geometry of the grouped GEMMs (rows of one expert per tile, weight rows
// per workgroup), shared by the permutation's tile prefix and the launches.
constexpr int kGemmBM = 32;
constexpr int kGateUpBN = 256;   // features per gate/up workgroup (4 waves x 2 x 32)
constexpr int kDownBN = 512;     // hidden rows per down workgroup (4 waves x 4 x 32)
constexpr int kDecodeRowsGU = 16; // expert rows per decode gate/up workgroup
constexpr int kDecodeRowsDn = 16; // hidden rows per decode down workgroup

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

struct ExpertPtrs {
    const uint8_t *base;     // first packed expert
    uint64_t stride;         // bytes between experts
    uint64_t gate_q, up_q, down_q, gate_s, up_s, down_s, gate_b, up_b, down_b;
};

struct SwigluConsts {
    float alpha, limit, up_offset;
};

// routing -----------------------------------------------------------------
hipError_t launch_rmsnorm(const void *x, int x_bf16, const float *gamma, int T, int H, float eps,
                          double *xn64, float *xn32, hipStream_t s);
// Router: split-K partial logits partial[splits][T][E] (fp64, bias not added).
// GEMV form for T <= kRouterGemvMaxT (one wavefront per expert and
// 2048-wide hidden slice), tiled form otherwise (slices sized for enough
// workgroups, at most 16).
constexpr int kRouterGemvMaxT = 16;
constexpr int kRouterGemvSlice = 2048;
struct RouterPlan {
    bool gemv;
    int slice;   // hidden units per split
    int splits;  // S
};
RouterPlan router_plan(int T, int H, int E);
// FP8-term quantisation of the expert input riding with the GEMV router:
// q [T][kTerms][Kp] codes, scales [T][kTerms][Kp/32], Kp = H rounded up to 128.
struct TermsOut {
    const void *in;
    int in_bf16;
    uint8_t *q;
    uint8_t *scales;
};
// in_kind: 0 float32, 1 bf16 bits, 2 float64
hipError_t launch_router(const void *x, int in_kind, const float *w, int T, int H, int E,
                         double *partial, const TermsOut *terms, hipStream_t s);
hipError_t launch_topk(const double *partial, int S, const float *bias, int T, int E, int k,
                       float route_scale, int32_t *idx, float *wts, int32_t *out_idx, float *out_w,
                       const void *resid, int resid_bf16, int H, float *out, hipStream_t s);
hipError_t launch_permute(const int32_t *idx, int T, int E, int k, int n_shared,
                          int32_t *counts, int32_t *offsets, int32_t *perm, int32_t *inv,
                          int32_t *rank, int32_t *mprefix, int32_t *out_counts,
                          int32_t *out_offsets, int32_t *out_perm, int32_t *out_inv,
                          hipStream_t s);

// decode ------------------------------------------------------------------
hipError_t launch_decode_gate_up(const void *x, int x_bf16, const double *partial, int S,
                                 const float *router_b, int T, int H, int F, int E, int k,
                                 int n_shared, float route_scale, const ExpertPtrs &ex,
                                 const ExpertPtrs &sh, SwigluConsts c, int32_t *idx, float *wts,
                                 int32_t *out_idx, float *out_w, const void *resid,
                                 int resid_bf16, float *out, float *act, hipStream_t s);
hipError_t launch_decode_down(int T, int H, int F, int k, int n_shared, const ExpertPtrs &ex,
                              const ExpertPtrs &sh, const int32_t *idx, const float *wts,
                              const float *act, float *out, hipStream_t s);

// decode on the block-scaled matrix cores: K-steps per wavefront for a
// K-wide GEMV (0 when K is too large for this form)
int mx_steps_per_wave(int K);
hipError_t launch_decode_gate_up_mx(const uint8_t *xq, const uint8_t *xs, const double *partial,
                                    int S, const float *router_b, int T, int H, int F, int E, int k,
                                    int n_shared, float route_scale, const ExpertPtrs &ex,
                                    const ExpertPtrs &sh, SwigluConsts c, int act_e0,
                                    int32_t *idx, float *wts, int32_t *out_idx, float *out_w,
                                    const void *resid, int resid_bf16, float *out, uint8_t *act_q,
                                    hipStream_t s);
hipError_t launch_decode_down_mx(const uint8_t *act_q, int act_e0, int T, int H, int F, int k,
                                 int n_shared, const ExpertPtrs &ex, const ExpertPtrs &sh,
                                 const int32_t *idx, const float *wts, float *out, hipStream_t s);

// prefill -----------------------------------------------------------------
hipError_t launch_gate_up_gemm(const void *x, int x_bf16, int T, int H, int F, int E, int k,
                               int n_shared, const ExpertPtrs &ex, const ExpertPtrs &sh,
                               SwigluConsts c, const int32_t *offsets, const int32_t *perm,
                               const int32_t *mprefix, int max_mtiles, float *act,
                               hipStream_t s);
hipError_t launch_down_gemm(int T, int H, int F, int E, int k, int n_shared, const ExpertPtrs &ex,
                            const ExpertPtrs &sh, const int32_t *offsets, const int32_t *perm,
                            const float *wts, const int32_t *mprefix, int max_mtiles,
                            const float *act, float *out, hipStream_t s);

// debug -------------------------------------------------------------------
hipError_t launch_dequant(const uint8_t *codes, const uint8_t *scales, int rows, int K, int path,
                          float *out, hipStream_t s);

}  // namespace moe
