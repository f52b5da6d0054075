// C ABI of the routed MXFP4 MoE block: host-side validation, workspace
// carving and the launch sequences. Declarations and contracts are in
// include/moe_mxfp4.h.
#include "moe_mxfp4.h"

#include <cmath>
#include <cstdint>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "host_status.hpp"
#include "kernels.hpp"

namespace {

thread_local std::string g_last_error;

#define MOE_TRY(expr)                  \
    do {                               \
        const int rc_ = (expr);        \
        if (rc_ != MOE_OK) return rc_; \
    } while (0)

#define MOE_TRY_HIP(expr, what)                                                           \
    do {                                                                                  \
        const hipError_t e_ = (expr);                                                     \
        if (e_ != hipSuccess) return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e_)); \
    } while (0)

int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int ok() {
    g_last_error.clear();
    return MOE_OK;
}

}  // namespace

int moe::host_fail(int code, const char *msg) { return fail(code, "%s", msg); }
int moe::host_ok() { return ok(); }

namespace {

constexpr uint64_t align_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_shape(const moe_shape *s) {
    if (!s) return fail(MOE_ERR_INVALID_ARG, "shape is NULL");
    if (s->T < 0 || s->T > (1 << 20)) return fail(MOE_ERR_INVALID_ARG, "T=%d outside [0, 2^20]", s->T);
    if (s->E < 1 || s->E > moe::kMaxE) return fail(MOE_ERR_INVALID_ARG, "E=%d outside [1, 512]", s->E);
    if (s->k < 1 || s->k > moe::kMaxK || s->k > s->E)
        return fail(MOE_ERR_INVALID_ARG, "k=%d outside [1, min(E, 8)]", s->k);
    if (s->H < 32 || s->H > 16384 || s->H % 32)
        return fail(MOE_ERR_INVALID_ARG, "H=%d must be a multiple of 32 in [32, 16384]", s->H);
    if (s->F < 32 || s->F > 16384 || s->F % 32)
        return fail(MOE_ERR_INVALID_ARG, "F=%d must be a multiple of 32 in [32, 16384]", s->F);
    if (s->act_dtype != MOE_F32 && s->act_dtype != MOE_BF16)
        return fail(MOE_ERR_INVALID_ARG, "act_dtype=%d is neither MOE_F32 nor MOE_BF16", s->act_dtype);
    if (s->n_shared != 0 && s->n_shared != 1)
        return fail(MOE_ERR_INVALID_ARG, "n_shared=%d must be 0 or 1", s->n_shared);
    if (!std::isfinite(s->swiglu_alpha)) return fail(MOE_ERR_INVALID_ARG, "swiglu_alpha is not finite");
    if (!(s->swiglu_limit > 0.f)) return fail(MOE_ERR_INVALID_ARG, "swiglu_limit must be > 0");
    if (!std::isfinite(s->swiglu_up_offset)) return fail(MOE_ERR_INVALID_ARG, "swiglu_up_offset is not finite");
    if (!std::isfinite(s->route_scale) || !(s->route_scale > 0.f))
        return fail(MOE_ERR_INVALID_ARG, "route_scale must be finite and > 0");
    if (s->act_quant < 0 || s->act_quant > 2)
        return fail(MOE_ERR_INVALID_ARG, "act_quant=%d must be 0, 1 or 2", s->act_quant);
    return MOE_OK;
}

void layout_of(const moe_shape *s, moe_blob_layout *L) {
    const uint64_t H = s->H, F = s->F;
    uint64_t o = 0;
    auto take = [&](uint64_t bytes) {
        const uint64_t at = o;
        o = align_up(o + bytes, 256);
        return at;
    };
    L->gate_q = take(F * H / 2);
    L->up_q = take(F * H / 2);
    L->down_q = take(H * F / 2);
    L->gate_s = take(F * H / 32);
    L->up_s = take(F * H / 32);
    L->down_s = take(H * F / 32);
    L->gate_b = take(F * 4);
    L->up_b = take(F * 4);
    const uint64_t db = o;
    L->down_b = db;
    L->bytes = db + H * 4;
    L->stride = align_up(L->bytes, 4096);
}

struct Workspace {
    double *rinv;     // RMSNorm scale per token [T]
    double *partial;  // router split-K partial logits [splits][T][E]
    int splits;
    int32_t *idx;
    float *wts;
    int32_t *counts, *offsets, *mprefix, *perm, *inv;
    // FP8 terms (codes, E8M0 scales) of the expert input [T] and of the
    // SwiGLU output [T*k + T*n_shared] (route order in decode, position
    // order in prefill)
    uint8_t *xq, *xs, *act_q, *act_s;
    float *y;  // prefill: weighted down output per row position [T*k + T*n_shared][H]
    uint64_t bytes;
};

Workspace carve(const moe_shape *s, uint8_t *base) {
    const uint64_t T = s->T, H = s->H, E = s->E, k = s->k, ns = s->n_shared;
    const uint64_t R = T * k;
    const uint64_t Hp = moe::pad128(s->H), Fp = moe::pad128(s->F);
    Workspace w{};
    uint64_t o = 0;
    auto take = [&](uint64_t bytes) {
        uint8_t *p = base ? base + o : nullptr;
        o = align_up(o + bytes, 256);
        return p;
    };
    w.rinv = reinterpret_cast<double *>(take(T * 8));
    const moe::RouterPlan rp = moe::router_plan(s->T, s->H, s->E);
    w.splits = rp.splits;
    w.partial = reinterpret_cast<double *>(take(static_cast<uint64_t>(rp.splits) * T * E * 8));
    w.idx = reinterpret_cast<int32_t *>(take(R * 4));
    w.wts = reinterpret_cast<float *>(take(R * 4));
    w.counts = reinterpret_cast<int32_t *>(take((E + 1) * 4));
    w.offsets = reinterpret_cast<int32_t *>(take((E + 2) * 4));
    w.mprefix = reinterpret_cast<int32_t *>(take((E + 2) * 4));
    w.perm = reinterpret_cast<int32_t *>(take(R * 4));
    w.inv = reinterpret_cast<int32_t *>(take(R * 4));
    w.xq = take(T * moe::kTerms * Hp);
    w.xs = take(T * moe::kTerms * Hp / 32);
    w.act_q = take((R + T * ns) * moe::kTerms * Fp);
    w.act_s = take((R + T * ns) * moe::kTerms * Fp / 32);
    w.y = reinterpret_cast<float *>(take((R + T * ns) * H * 4));
    w.bytes = o;
    return w;
}

int check_ws(const moe_shape *s, void *ws, size_t ws_bytes) {
    const uint64_t need = carve(s, nullptr).bytes;
    if (!ws) return fail(MOE_ERR_WORKSPACE, "workspace is NULL");
    if (!aligned(ws, 256)) return fail(MOE_ERR_WORKSPACE, "workspace is not 256-byte aligned");
    if (ws_bytes < need)
        return fail(MOE_ERR_WORKSPACE, "workspace has %zu bytes, needs %llu", ws_bytes,
                    static_cast<unsigned long long>(need));
    return MOE_OK;
}

moe::ExpertPtrs expert_ptrs(const moe_shape *s, const uint8_t *base) {
    moe_blob_layout L;
    layout_of(s, &L);
    moe::ExpertPtrs p;
    p.base = base;
    p.stride = L.stride;
    p.gate_q = L.gate_q;
    p.up_q = L.up_q;
    p.down_q = L.down_q;
    p.gate_s = L.gate_s;
    p.up_s = L.up_s;
    p.down_s = L.down_s;
    p.gate_b = L.gate_b;
    p.up_b = L.up_b;
    p.down_b = L.down_b;
    return p;
}

int hip_check(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return MOE_OK;
}

// One-shot timing hook armed by moe_profile_next_launch.
struct ProfileHook {
    int kernel = -1;
    hipEvent_t start = nullptr, stop = nullptr;
};
thread_local ProfileHook g_hook;
constexpr int kUnprofiled = -2;  // id of launches the hook never times

// Launch through `fn` (one kernel, returning hipError_t). When the hook is
// armed for kernel `id`, its events ride on that dispatch (hipExtLaunchKernel
// stamps the kernel's own start and end into them).
template <typename Fn>
int launch(int id, const char *what, hipStream_t st, Fn &&fn) {
    (void)st;
    const bool armed = g_hook.kernel == id;
    if (armed) moe::launch_events() = moe::LaunchEvents{g_hook.start, g_hook.stop};
    // the check after the launch reads the thread's last HIP error: drop one
    // left by an earlier, unrelated call so it is not taken for this launch's
    (void)hipGetLastError();
    const int rc = hip_check(fn(), what);
    if (armed) {
        moe::launch_events() = moe::LaunchEvents{};
        g_hook.kernel = -1;
    }
    return rc;
}

// The routing variant as the kernels take it (NULL: plain top-k).
int route_sel_of(const moe_routing *r, moe::RouteSel *rs) {
    *rs = moe::RouteSel{nullptr, nullptr, nullptr, 0};
    if (!r) return MOE_OK;
    if (r->tid2eid) {
        if (!r->token_ids) return fail(MOE_ERR_INVALID_ARG, "hash routing (tid2eid) needs token_ids");
        if (r->vocab < 1) return fail(MOE_ERR_INVALID_ARG, "hash routing needs vocab >= 1 (vocab=%d)", r->vocab);
        if (!aligned(r->tid2eid, 4) || !aligned(r->token_ids, 4))
            return fail(MOE_ERR_INVALID_ARG, "tid2eid and token_ids must be 4-byte aligned");
        *rs = moe::RouteSel{nullptr, r->tid2eid, r->token_ids, r->vocab};
        return MOE_OK;
    }
    if (r->sel_bias && !aligned(r->sel_bias, 4))
        return fail(MOE_ERR_INVALID_ARG, "sel_bias must be 4-byte aligned");
    rs->bias = r->sel_bias;
    return MOE_OK;
}

// Shared argument checks of the two forward entry points.
int check_forward(const moe_shape *s, const void *hidden, const float *norm_w,
                  const float *router_w, const float *router_b, const uint8_t *experts,
                  const uint8_t *shared, const float *out, void *ws, size_t ws_bytes) {
    MOE_TRY(check_shape(s));
    if (s->T == 0) return MOE_OK;  // nothing is read or written
    if (!hidden || !router_w || !router_b || !experts || !out)
        return fail(MOE_ERR_INVALID_ARG, "hidden, router_w, router_b, experts and out must be non-NULL");
    if (s->n_shared && !shared) return fail(MOE_ERR_INVALID_ARG, "n_shared=1 needs a shared expert blob");
    if (!s->n_shared && shared) return fail(MOE_ERR_INVALID_ARG, "shared blob given with n_shared=0");
    if (!aligned(hidden, 16) || !aligned(out, 16) || !aligned(router_w, 16) ||
        (norm_w && !aligned(norm_w, 16)))
        return fail(MOE_ERR_INVALID_ARG, "hidden, out, router_w and norm_w must be 16-byte aligned");
    if (!aligned(experts, 256) || (shared && !aligned(shared, 256)))
        return fail(MOE_ERR_INVALID_ARG, "expert blobs must be 256-byte aligned");
    if (norm_w && !(s->rms_eps >= 0.f)) return fail(MOE_ERR_INVALID_ARG, "rms_eps must be >= 0");
    if (s->act_dtype == MOE_BF16 && static_cast<const void *>(out) == hidden)
        return fail(MOE_ERR_INVALID_ARG, "out may not alias a bfloat16 hidden");
    return check_ws(s, ws, ws_bytes);
}

// RMSNorm (optional), the router's partial logits and, with `terms`, the FP8
// terms of the expert input (in the router's grid for small T, else their own
// kernel).
// RMSNorm scale (with a norm) and router. `terms`: the router launch also
// makes the FP8 terms of the expert input. Returns the expert input in `in`.
int route_front(const moe_shape *s, const void *x, const float *norm_w, const float *router_w,
                const Workspace &w, bool terms, float *seed, moe::RouteIn *in, hipStream_t st) {
    const int bf16 = s->act_dtype == MOE_BF16;
    *in = moe::RouteIn{x, bf16, nullptr, nullptr, seed};
    if (norm_w) {
        MOE_TRY(launch(MOE_KERNEL_RMSNORM, "rmsnorm", st, [&] {
            return moe::launch_rms_inv(x, bf16, s->T, s->H, s->rms_eps, w.rinv, st);
        }));
        in->inv = w.rinv;
        in->gamma = norm_w;
    }
    const moe::TermsOut tq{w.xq, w.xs, s->act_quant};
    MOE_TRY(launch(MOE_KERNEL_ROUTER, "router", st, [&] {
        return moe::launch_router(*in, router_w, s->T, s->H, s->E, w.partial, terms ? &tq : nullptr,
                                  st);
    }));
    return MOE_OK;
}

// The grouped GEMMs' tiling and term counts for this call.
moe::GemmPlan gemm_plan_of(const moe_shape *s, bool norm) {
    return moe::gemm_plan(s->T, s->k, s->E, s->n_shared, s->F, s->act_dtype == MOE_BF16 && !norm,
                          s->act_quant != 0, s->act_quant == 2);
}

// Upper bound on the grouped GEMMs' row tiles (the grid is sized by it).
int max_tiles(const moe_shape *s, int bm) {
    const long long R = static_cast<long long>(s->T) * s->k;
    long long m = (R + bm - 1) / bm + (s->E < R ? s->E : R);
    if (s->n_shared) m += (s->T + bm - 1) / bm;
    return static_cast<int>(m);
}

}  // namespace

namespace moe {
LaunchEvents &launch_events() {
    thread_local LaunchEvents ev;
    return ev;
}
}  // namespace moe

extern "C" {

int moe_blob_layout_get(const moe_shape *shape, moe_blob_layout *layout) {
    if (!shape || !layout) return fail(MOE_ERR_INVALID_ARG, "shape and layout must be non-NULL");
    if (shape->H < 32 || shape->H > 16384 || shape->H % 32 || shape->F < 32 ||
        shape->F > 16384 || shape->F % 32)
        return fail(MOE_ERR_INVALID_ARG, "H and F must be multiples of 32 in [32, 16384]");
    layout_of(shape, layout);
    return ok();
}

int moe_pack_experts(const moe_shape *shape, int32_t n, const moe_expert_planes *p, uint8_t *dst) {
    moe_blob_layout L;
    MOE_TRY(moe_blob_layout_get(shape, &L));
    if (n < 0 || !p || !dst) return fail(MOE_ERR_INVALID_ARG, "n >= 0, planes and dst required");
    if (n > 0 && (!p->gate_q || !p->up_q || !p->down_q || !p->gate_s || !p->up_s || !p->down_s ||
                  !p->gate_b || !p->up_b || !p->down_b))
        return fail(MOE_ERR_INVALID_ARG, "every plane pointer must be non-NULL");
    const uint32_t H = shape->H, F = shape->F;
    // one row-major code/scale plane (rows x K) into the tiled order
    auto tile_plane = [](uint8_t *q_dst, uint8_t *s_dst, const uint8_t *q_src, const uint8_t *s_src,
                         uint32_t rows, uint32_t K) {
        const uint32_t nb = K / 32;
        for (uint32_t r = 0; r < rows; ++r)
            for (uint32_t c = 0; c < nb; ++c) {
                std::memcpy(q_dst + moe::mx_code_offset(r, c, nb),
                            q_src + static_cast<uint64_t>(r) * (K / 2) + 16ull * c, 16);
                s_dst[moe::mx_scale_offset(r, c, nb)] = s_src[static_cast<uint64_t>(r) * nb + c];
            }
    };
    const uint64_t fh = static_cast<uint64_t>(F) * H;
    for (int32_t i = 0; i < n; ++i) {
        uint8_t *b = dst + static_cast<uint64_t>(i) * L.stride;
        std::memset(b, 0, L.stride);
        tile_plane(b + L.gate_q, b + L.gate_s, p->gate_q + i * fh / 2, p->gate_s + i * fh / 32, F, H);
        tile_plane(b + L.up_q, b + L.up_s, p->up_q + i * fh / 2, p->up_s + i * fh / 32, F, H);
        tile_plane(b + L.down_q, b + L.down_s, p->down_q + i * fh / 2, p->down_s + i * fh / 32, H, F);
        std::memcpy(b + L.gate_b, p->gate_b + static_cast<uint64_t>(i) * F, F * 4ull);
        std::memcpy(b + L.up_b, p->up_b + static_cast<uint64_t>(i) * F, F * 4ull);
        std::memcpy(b + L.down_b, p->down_b + static_cast<uint64_t>(i) * H, H * 4ull);
    }
    return ok();
}

size_t moe_workspace_bytes(const moe_shape *shape) {
    if (check_shape(shape) != MOE_OK) return 0;
    return carve(shape, nullptr).bytes;
}

int moe_route_profile_summary(const uint64_t *counts, int32_t layers, int32_t E,
                              uint64_t *selections, uint64_t *unique_layer_experts,
                              int32_t *layer_unique) {
    if (!counts || !selections || !unique_layer_experts)
        return fail(MOE_ERR_INVALID_ARG, "counts, selections and unique_layer_experts must be non-NULL");
    if (layers < 0 || E < 1) return fail(MOE_ERR_INVALID_ARG, "need layers >= 0 and E >= 1");
    uint64_t total = 0, unique = 0;
    for (int32_t l = 0; l < layers; ++l) {
        int32_t nz = 0;
        for (int32_t e = 0; e < E; ++e) {
            const uint64_t c = counts[static_cast<size_t>(l) * E + e];
            total = c > UINT64_MAX - total ? UINT64_MAX : total + c;  // saturating, as the page's fold
            nz += c != 0;
        }
        unique += static_cast<uint64_t>(nz);
        if (layer_unique) layer_unique[l] = nz;
    }
    *selections = total;
    *unique_layer_experts = unique;
    return ok();
}

int moe_route(const moe_shape *s, const void *x, const float *norm_w, const float *router_w,
              const float *router_b, const moe_routing *routing, const moe_route_out *out, void *ws,
              size_t ws_bytes, hipStream_t st) {
    MOE_TRY(check_shape(s));
    if (s->T == 0) return ok();
    if (!x || !router_w || !router_b || !out)
        return fail(MOE_ERR_INVALID_ARG, "x, router_w, router_b and out must be non-NULL");
    if (!aligned(x, 16) || !aligned(router_w, 16) || (norm_w && !aligned(norm_w, 16)))
        return fail(MOE_ERR_INVALID_ARG, "x, router_w and norm_w must be 16-byte aligned");
    if (norm_w && !(s->rms_eps >= 0.f)) return fail(MOE_ERR_INVALID_ARG, "rms_eps must be >= 0");
    moe::RouteSel rs;
    MOE_TRY(route_sel_of(routing, &rs));
    MOE_TRY(check_ws(s, ws, ws_bytes));
    const Workspace w = carve(s, static_cast<uint8_t *>(ws));
    moe::RouteIn in;
    MOE_TRY(route_front(s, x, norm_w, router_w, w, false, nullptr, &in, st));
    MOE_TRY(launch(MOE_KERNEL_TOPK, "topk", st, [&] {
        return moe::launch_topk(w.partial, w.splits, router_b, rs, s->T, s->E, s->k,
                                s->route_scale, w.idx, w.wts, out->topk_idx, out->topk_w, st);
    }));
    MOE_TRY(launch(MOE_KERNEL_PERMUTE, "permute", st, [&] { return moe::launch_permute(w.idx, s->T, s->E, s->k, 0, 16, w.counts, w.offsets, w.perm,
                                          w.inv, w.mprefix, out->counts, out->offsets,
                                          out->perm, out->inv, out->route_counts, nullptr, s->H,
                                          nullptr, st); }));
    return ok();
}

int moe_act_quant_debug(const moe_shape *s, const void *x, const float *norm_w, uint8_t *codes,
                        uint8_t *scales, void *ws, size_t ws_bytes, hipStream_t st) {
    MOE_TRY(check_shape(s));
    if (s->T == 0) return ok();
    if (!x || !codes || !scales) return fail(MOE_ERR_INVALID_ARG, "x, codes and scales must be non-NULL");
    if (!aligned(x, 16) || (norm_w && !aligned(norm_w, 16)))
        return fail(MOE_ERR_INVALID_ARG, "x and norm_w must be 16-byte aligned");
    if (norm_w && !(s->rms_eps >= 0.f)) return fail(MOE_ERR_INVALID_ARG, "rms_eps must be >= 0");
    MOE_TRY(check_ws(s, ws, ws_bytes));
    const Workspace w = carve(s, static_cast<uint8_t *>(ws));
    const int bf16 = s->act_dtype == MOE_BF16;
    moe::RouteIn in{x, bf16, nullptr, nullptr, nullptr};
    if (norm_w) {
        MOE_TRY(launch(MOE_KERNEL_RMSNORM, "rmsnorm", st, [&] {
            return moe::launch_rms_inv(x, bf16, s->T, s->H, s->rms_eps, w.rinv, st);
        }));
        in.inv = w.rinv;
        in.gamma = norm_w;
    }
    MOE_TRY(launch(kUnprofiled, "act_fp4", st, [&] { return moe::launch_act_fp4(in, s->T, s->H, codes, scales, st); }));
    return ok();
}

int moe_forward_decode(const moe_shape *s, const void *hidden, const float *norm_w,
                       const float *router_w, const float *router_b, const moe_routing *routing,
                       const uint8_t *experts, const uint8_t *shared, float *out,
                       const moe_route_out *ro, void *ws, size_t ws_bytes, hipStream_t st) {
    MOE_TRY(check_forward(s, hidden, norm_w, router_w, router_b, experts, shared, out, ws, ws_bytes));
    moe::RouteSel rs;
    MOE_TRY(route_sel_of(routing, &rs));
    if (s->T > 64) return fail(MOE_ERR_UNSUPPORTED, "decode takes T <= 64 (T=%d); use prefill", s->T);
    if (s->act_quant)
        return fail(MOE_ERR_UNSUPPORTED, "the quantised expert-input mode is a prefill mode");
    if (s->H > 8192 || s->F > 8192)
        return fail(MOE_ERR_UNSUPPORTED, "decode takes H, F <= 8192");
    if (s->T == 0) return ok();
    const Workspace w = carve(s, static_cast<uint8_t *>(ws));
    moe::RouteIn in;
    // the router launch's quantisation seeds out with the residual, unless out
    // already is the float32 input (in place)
    const bool in_place = s->act_dtype == MOE_F32 && static_cast<const void *>(out) == hidden;
    MOE_TRY(route_front(s, hidden, norm_w, router_w, w, true, in_place ? nullptr : out, &in, st));
    moe::DecodeArgs a{};
    a.xq = w.xq;
    a.xs = w.xs;
    a.partial = w.partial;
    a.S = w.splits;
    a.router_b = router_b;
    a.rs = rs;
    a.T = s->T;
    a.H = s->H;
    a.F = s->F;
    a.E = s->E;
    a.k = s->k;
    a.n_shared = s->n_shared;
    a.route_scale = s->route_scale;
    a.ex = expert_ptrs(s, experts);
    a.sh = expert_ptrs(s, shared);
    a.sc = moe::SwigluConsts{s->swiglu_alpha, s->swiglu_limit, s->swiglu_up_offset};
    a.idx = w.idx;
    a.wts = w.wts;
    a.out_idx = ro ? ro->topk_idx : nullptr;
    a.out_w = ro ? ro->topk_w : nullptr;
    a.route_counts = ro ? ro->route_counts : nullptr;  // added where the experts are published
    a.out = out;
    a.act_q = w.act_q;
    a.act_s = w.act_s;
    MOE_TRY(launch(MOE_KERNEL_DECODE_GATE_UP, "decode_gate_up", st,
                   [&] { return moe::launch_decode_gate_up(a, st); }));
    MOE_TRY(launch(MOE_KERNEL_DECODE_DOWN, "decode_down", st,
                   [&] { return moe::launch_decode_down(a, st); }));
    if (ro && (ro->counts || ro->offsets || ro->perm || ro->inv))
        MOE_TRY(launch(MOE_KERNEL_PERMUTE, "permute", st, [&] {
            return moe::launch_permute(w.idx, s->T, s->E, s->k, 0, 16, w.counts, w.offsets, w.perm,
                                       w.inv, w.mprefix, ro->counts, ro->offsets,
                                       ro->perm, ro->inv, nullptr, nullptr, s->H, nullptr, st);
        }));
    return ok();
}

int moe_forward_prefill(const moe_shape *s, const void *hidden, const float *norm_w,
                        const float *router_w, const float *router_b, const moe_routing *routing,
                        const uint8_t *experts, const uint8_t *shared, float *out,
                        const moe_route_out *ro, void *ws, size_t ws_bytes, hipStream_t st) {
    MOE_TRY(check_forward(s, hidden, norm_w, router_w, router_b, experts, shared, out, ws, ws_bytes));
    moe::RouteSel rs;
    MOE_TRY(route_sel_of(routing, &rs));
    if (s->T == 0) return ok();
    {  // the grouped GEMMs address FP8-term rows with 32-bit byte offsets
        const uint64_t rows = static_cast<uint64_t>(s->T) * (s->k + s->n_shared);
        if (static_cast<uint64_t>(s->T) * moe::kTerms * moe::pad128(s->H) >= (1ull << 32) ||
            rows * moe::kTerms * moe::pad128(s->F) >= (1ull << 32))
            return fail(MOE_ERR_UNSUPPORTED, "prefill needs T*(k+n_shared)*4*pad128(F) and T*4*pad128(H) below 2^32");
    }
    const Workspace w = carve(s, static_cast<uint8_t *>(ws));
    const moe::GemmPlan plan = gemm_plan_of(s, norm_w != nullptr);
    // the FP8 terms (or MX-FP4 codes) of the expert input ride in the router
    // launch in its GEMV form, else beside the permutation's workgroups; a
    // bfloat16 input taken as it is (x_terms 1) needs neither
    const bool need_terms = plan.x_terms != 1;
    moe::RouteIn in;
    const bool router_terms = need_terms && moe::router_plan(s->T, s->H, s->E).gemv;
    MOE_TRY(route_front(s, hidden, norm_w, router_w, w, router_terms, nullptr, &in, st));
    MOE_TRY(launch(MOE_KERNEL_TOPK, "topk", st, [&] {
        return moe::launch_topk(w.partial, w.splits, router_b, rs, s->T, s->E, s->k,
                                s->route_scale, w.idx, w.wts, ro ? ro->topk_idx : nullptr,
                                ro ? ro->topk_w : nullptr, st);
    }));
    const int bm = plan.tile_rows;
    const moe::TermsOut tq{w.xq, w.xs, s->act_quant};
    MOE_TRY(launch(MOE_KERNEL_PERMUTE, "permute", st, [&] {
        return moe::launch_permute(w.idx, s->T, s->E, s->k, s->n_shared, bm, w.counts, w.offsets,
                                   w.perm, w.inv, w.mprefix, ro ? ro->counts : nullptr,
                                   ro ? ro->offsets : nullptr, ro ? ro->perm : nullptr,
                                   ro ? ro->inv : nullptr, ro ? ro->route_counts : nullptr, &in,
                                   s->H, need_terms && !router_terms ? &tq : nullptr, st);
    }));
    const moe::ExpertPtrs ex = expert_ptrs(s, experts);
    const moe::ExpertPtrs sh = expert_ptrs(s, shared);
    const moe::SwigluConsts c{s->swiglu_alpha, s->swiglu_limit, s->swiglu_up_offset};
    const int mt = max_tiles(s, bm);
    MOE_TRY(launch(MOE_KERNEL_GATE_UP_GEMM, "gate_up_gemm", st, [&] {
        const uint8_t *xb = plan.x_terms == 1 ? static_cast<const uint8_t *>(hidden) : w.xq;
        return moe::launch_gate_up_gemm(xb, w.xs, s->T, s->H, s->F, s->E, s->k, s->n_shared, ex,
                                        sh, c, w.offsets, w.perm, w.mprefix, bm, mt, plan.x_terms,
                                        plan.act_terms == 0, w.act_q, w.act_s, st);
    }));
    MOE_TRY(launch(MOE_KERNEL_DOWN_GEMM, "down_gemm", st, [&] {
        return moe::launch_down_gemm(w.act_q, w.act_s, s->T, s->H, s->F, s->E, s->k, s->n_shared,
                                     ex, sh, w.offsets, w.perm, w.wts, w.mprefix, bm, mt,
                                     plan.act_terms == 0, w.y, st);
    }));
    MOE_TRY(launch(MOE_KERNEL_COMBINE, "combine", st, [&] {
        return moe::launch_combine(w.y, w.inv, s->T, s->H, s->k, s->n_shared, hidden,
                                   s->act_dtype == MOE_BF16, out, st);
    }));
    return ok();
}

int moe_prefill_plan(const moe_shape *s, int32_t with_norm, moe_prefill_plan_t *plan) {
    MOE_TRY(check_shape(s));
    if (!plan) return fail(MOE_ERR_INVALID_ARG, "plan must be non-NULL");
    const moe::GemmPlan p = gemm_plan_of(s, with_norm != 0);
    plan->tile_rows = p.tile_rows;
    plan->x_terms = p.x_terms;
    plan->act_terms = p.act_terms;
    plan->gate_up_features = p.gate_up_features;
    plan->down_rows = p.down_rows;
    return ok();
}

int moe_dequant_debug(const moe_shape *s, const uint8_t *blob, int32_t which, int32_t path,
                      float *out, hipStream_t st) {
    moe_blob_layout L;
    MOE_TRY(moe_blob_layout_get(s, &L));
    if (!blob || !out) return fail(MOE_ERR_INVALID_ARG, "blob and out must be non-NULL");
    if (!aligned(blob, 256)) return fail(MOE_ERR_INVALID_ARG, "blob must be 256-byte aligned");
    if (which < 0 || which > 2) return fail(MOE_ERR_INVALID_ARG, "which must be 0, 1 or 2");
    if (path < 0 || path > 2) return fail(MOE_ERR_INVALID_ARG, "path must be 0, 1 or 2");
    const int rows = which == 2 ? s->H : s->F;
    const int K = which == 2 ? s->F : s->H;
    const uint8_t *q = blob + (which == 0 ? L.gate_q : which == 1 ? L.up_q : L.down_q);
    const uint8_t *sc = blob + (which == 0 ? L.gate_s : which == 1 ? L.up_s : L.down_s);
    MOE_TRY(hip_check(moe::launch_dequant(q, sc, rows, K, path, out, st), "dequant"));
    return ok();
}

int moe_profile_next_launch(int32_t kernel, hipEvent_t start, hipEvent_t stop) {
    if (kernel < 0) {
        g_hook = ProfileHook{};
        return ok();
    }
    if (kernel > MOE_KERNEL_COMBINE || !start || !stop)
        return fail(MOE_ERR_INVALID_ARG, "unknown kernel id %d or NULL event", kernel);
    g_hook.kernel = kernel;
    g_hook.start = start;
    g_hook.stop = stop;
    return ok();
}

const char *moe_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
