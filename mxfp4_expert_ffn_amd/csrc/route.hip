// Routing kernels: RMSNorm scale, router logits (fp64), top-k + route weights,
// per-expert histogram / exclusive scan / stable permutation.
//
// Pages: goosedump `gpt_oss.rs` `mixture_of_experts_batch` (router matmul,
// add_bias_batch, top_experts, softmax, routes_by_expert in token order),
// `top_experts` (descending value, lower index on ties); antirez `ds4.c`
// `rms_norm_weight` (sum of squares accumulated in double).
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

// x[i] widened exactly to fp64; KIND 0 float32, 1 bf16 bits.
template <int KIND>
__device__ __forceinline__ double load_in(const void *x, size_t i) {
    if constexpr (KIND == 0) return static_cast<double>(static_cast<const float *>(x)[i]);
    else return static_cast<double>(bf16_bits_to_f32(static_cast<const uint16_t *>(x)[i]));
}

// Four consecutive inputs x[i..i+3] (i a multiple of 4) widened to fp64.
template <int KIND>
__device__ __forceinline__ void load4(const void *x, size_t i, double (&v)[4]) {
    if constexpr (KIND == 0) {
        const float4 f = *reinterpret_cast<const float4 *>(static_cast<const float *>(x) + i);
        v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
    } else {
        const uint2 u = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(x) + i);
        v[0] = __uint_as_float(u.x << 16); v[1] = __uint_as_float(u.x & 0xffff0000u);
        v[2] = __uint_as_float(u.y << 16); v[3] = __uint_as_float(u.y & 0xffff0000u);
    }
}

// ---------------------------------------------------------------- RMSNorm
// One workgroup per token: fp64 sum of squares, inv[t] = 1/sqrt(ss/H + eps).
// Each thread takes groups of 4 consecutive values (H is a multiple of 32),
// loading up to 4 groups before it adds them. The normalised input
// (x * inv[t]) * gamma[h] is formed in fp64, in that order, where it is read
// (router, FP8-term quantisation), so it never goes through memory.
template <int KIND>
__global__ __launch_bounds__(256) void rms_inv_kernel(const void *x, int H, float eps,
                                                      double *inv) {
    constexpr int kU = 4;
    const int t = blockIdx.x;
    const size_t row = static_cast<size_t>(t) * H;
    const int groups = H / 4;
    double ss = 0.0;
    for (int g0 = threadIdx.x; g0 < groups; g0 += kU * 256) {
        double v[kU][4];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int g = g0 + 256 * u;
            load4<KIND>(x, row + 4 * static_cast<size_t>(g < groups ? g : 0), v[u]);
        }
#pragma unroll
        for (int u = 0; u < kU; ++u)
            if (g0 + 256 * u < groups)
#pragma unroll
                for (int j = 0; j < 4; ++j) ss = fma(v[u][j], v[u][j], ss);
    }
    __shared__ double part[4];
    ss = wave_sum_f64(ss);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
    __syncthreads();
    if (threadIdx.x == 0) {
        const double total = part[0] + part[1] + part[2] + part[3];
        inv[t] = 1.0 / sqrt(total / H + static_cast<double>(eps));
    }
}

// ---------------------------------------------------------------- four values per lane
// The block splits of fp8_terms_group and fp4_act_code for a block of 32
// values held four per lane by a group of 8 consecutive lanes (lane j of the
// group: values 4j .. 4j + 3): the same arithmetic value by value, with the
// block maximum taken over the group. The 8 lanes of a group take part
// together.

// Maximum over each group of 8 consecutive lanes of a value that is >= 0,
// returned to all 8: DPP swaps inside each quad, then the mirror inside the
// group of 8 (lane i and lane 7 - i sit in different quads).
__device__ __forceinline__ float group8_max(float v) {
    v = fmaxf(v, __builtin_amdgcn_update_dpp(0.0f, v, 0xB1, 0xf, 0xf, false));    // quad_perm [1,0,3,2]
    v = fmaxf(v, __builtin_amdgcn_update_dpp(0.0f, v, 0x4E, 0xf, 0xf, false));    // quad_perm [2,3,0,1]
    return fmaxf(v, __builtin_amdgcn_update_dpp(0.0f, v, 0x141, 0xf, 0xf, false));  // row_half_mirror
}

__device__ __forceinline__ float abs_max4(const float (&v)[4]) {
    return fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
}

// codes[n]: term n of the lane's four values (value m in byte m); scales:
// the scale byte of term n in byte n.
__device__ __forceinline__ void fp8_terms_group4(const float (&v)[4], uint32_t (&codes)[kTerms],
                                                 uint32_t &scales) {
    const float amax = group8_max(abs_max4(v));
    const int e0 = static_cast<int>((__float_as_uint(amax) >> 23) & 0xffu) - 127 - 7;
    float r[4] = {v[0], v[1], v[2], v[3]};
    scales = 0;
#pragma unroll
    for (int n = 0; n < kTerms; ++n) {
        int e = e0 - 4 * n;
        e = e < -126 ? -126 : (e > 127 ? 127 : e);
        uint32_t c = 0;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const uint32_t q = e4m3_encode(r[m] * pow2f(-e));
            r[m] -= e4m3_decode(q) * pow2f(e);
            c |= q << (8 * m);
        }
        codes[n] = c;
        scales |= static_cast<uint32_t>(e + 127) << (8 * n);
    }
}

// The lane's four E2M1 codes packed in 16 bits (value m in bits 4m .. 4m + 3,
// so the low nibble of each byte is the even element) and the block's scale
// byte.
__device__ __forceinline__ uint32_t fp4_act_codes4(const float (&v)[4], uint32_t &scale_byte) {
    const float amax = fmaxf(group8_max(abs_max4(v)), 7.052966104933725e-38f);  // 6 * 2^-126
    const uint32_t bits = __float_as_uint(amax);
    const int E = static_cast<int>((bits >> 23) & 0xffu) - 127;
    const int e = (bits & 0x7fffffu) <= 0x400000u ? E - 2 : E - 1;  // amax <= 1.5 * 2^E: 6 * 2^(E-2) fits
    scale_byte = static_cast<uint32_t>(e + 127);
    uint32_t c = 0;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const float a = fminf(fabsf(v[m]) * pow2f(-e), 6.0f);
        // nearest of {0, .5, 1, 1.5, 2, 3, 4, 6}; a midpoint goes to the even index
        const uint32_t idx = static_cast<uint32_t>(a > 0.25f) + static_cast<uint32_t>(a >= 0.75f) +
                             static_cast<uint32_t>(a > 1.25f) + static_cast<uint32_t>(a >= 1.75f) +
                             static_cast<uint32_t>(a > 2.5f) + static_cast<uint32_t>(a >= 3.5f) +
                             static_cast<uint32_t>(a > 5.0f);
        c |= (idx | (v[m] < 0.0f ? 8u : 0u)) << (4 * m);
    }
    return c;
}

// ---------------------------------------------------------------- FP8 terms
// Quantisation of the expert input into FP8 terms for the block-scaled
// matrix-core kernels, done by the workgroups past a router launch's or the
// permutation launch's own. A 32-value block of k (the unit an E8M0 scale of
// the instruction's operand covers) belongs to a group of lanes: 32 lanes of
// one value each (VPL 1: the few blocks of a small batch, where the chain of
// one lane is the launch's latency), or 8 lanes of four consecutive values
// each (VPL 4: a quarter of the instructions, 16-byte loads and 4-byte stores
// for a large batch; the stack's and DeepSeek-V4's quantisation 2x faster).
// Codes go to xq[t][n][k] (zero past H), scales to xs[t][n][k / 32]. With a
// norm the value is float32((x * inv[t]) * gamma[k]). With a seed buffer the
// raw input value is also stored there as float32 (decode's residual: the
// store rides on the load the quantisation makes anyway, ahead of every
// expert launch). H is a multiple of 32, so a block is all in or all out.

// The lane's VPL values of block gidx (zeros past the last block or past H).
template <int VPL>
__device__ __forceinline__ void quantize_input(const RouteIn &in, int T, int H, int nb, int gidx,
                                               float (&v)[VPL]) {
#pragma unroll
    for (int m = 0; m < VPL; ++m) v[m] = 0.f;
    if (gidx >= T * nb) return;
    const int t = gidx / nb, kk = 32 * (gidx - t * nb) + VPL * (threadIdx.x & (32 / VPL - 1));
    if (kk >= H) return;
    const size_t at = static_cast<size_t>(t) * H + kk;
    double x[VPL];
    if constexpr (VPL == 1) {
        x[0] = in.bf16 ? load_in<1>(in.x, at) : load_in<0>(in.x, at);
        if (in.seed) in.seed[at] = static_cast<float>(x[0]);  // exact: the input is f32 or bf16
    } else {
        if (in.bf16) load4<1>(in.x, at, x);
        else load4<0>(in.x, at, x);
        if (in.seed)
            *reinterpret_cast<float4 *>(in.seed + at) =
                make_float4(static_cast<float>(x[0]), static_cast<float>(x[1]), static_cast<float>(x[2]),
                            static_cast<float>(x[3]));
    }
    if (in.inv) {
        const double iv = in.inv[t];
        float g[VPL];
        if constexpr (VPL == 1) {
            g[0] = in.gamma[kk];
        } else {
            const float4 g4 = *reinterpret_cast<const float4 *>(in.gamma + kk);
            g[0] = g4.x; g[1] = g4.y; g[2] = g4.z; g[3] = g4.w;
        }
#pragma unroll
        for (int m = 0; m < VPL; ++m) v[m] = static_cast<float>(x[m] * iv * static_cast<double>(g[m]));
    } else {
#pragma unroll
        for (int m = 0; m < VPL; ++m) v[m] = static_cast<float>(x[m]);
    }
}

// Terms of block gidx from the group's values; the group's lanes take part
// together (VPL 1: the whole wavefront, one half-wavefront maximum). fp4: the
// MX-FP4 round trip instead, codes packed two per byte in xq[t][Kp / 2] and
// the block's scale byte in xs[t][Kp / 32].
template <int VPL>
__device__ __forceinline__ void quantize_store(const float (&v)[VPL], int T, int nb, int Kp, uint8_t *xq,
                                               uint8_t *xs, int gidx, int fp4) {
    const int j = threadIdx.x & (32 / VPL - 1);  // the lane in its group
    const bool real = VPL == 1 ? gidx < T * nb : true;
    const int t = gidx / nb, blk = gidx - t * nb;
    if (fp4) {
        uint32_t sbyte;
        if constexpr (VPL == 1) {
            const uint32_t pair = fp4_pack_pair(fp4_act_code(v[0], sbyte));
            if (real && (j & 1) == 0)
                xq[static_cast<size_t>(t) * (Kp / 2) + 16 * blk + (j >> 1)] = static_cast<uint8_t>(pair);
        } else {
            const uint32_t c = fp4_act_codes4(v, sbyte);
            *reinterpret_cast<uint16_t *>(xq + static_cast<size_t>(t) * (Kp / 2) + 16 * blk + 2 * j) =
                static_cast<uint16_t>(c);
        }
        if (real && j == 0) xs[static_cast<size_t>(t) * nb + blk] = static_cast<uint8_t>(sbyte);
        return;
    }
    uint32_t codes[kTerms], scales;
    if constexpr (VPL == 1) {
        uint32_t packed;
        fp8_terms_group(v[0], packed, scales);
#pragma unroll
        for (int n = 0; n < kTerms; ++n) codes[n] = (packed >> (8 * n)) & 0xffu;
    } else {
        fp8_terms_group4(v, codes, scales);
    }
    if (!real) return;
    const int kk = 32 * blk + VPL * j;
#pragma unroll
    for (int n = 0; n < kTerms; ++n) {
        uint8_t *dst = xq + (static_cast<size_t>(t) * kTerms + n) * Kp + kk;
        if constexpr (VPL == 1) *dst = static_cast<uint8_t>(codes[n]);
        else *reinterpret_cast<uint32_t *>(dst) = codes[n];
        if (j == 0) xs[(static_cast<size_t>(t) * kTerms + n) * nb + blk] = static_cast<uint8_t>(scales >> (8 * n));
    }
}

// Workgroups [first, gridDim.x) of a launch: blockDim.x * VPL / 32 blocks of
// 32 values per workgroup and round, in a grid-stride loop that loads kU
// rounds before it quantises them. The loop and its guards are per group of
// lanes (VPL 1: per wavefront, both halves together, as the half-wavefront
// maximum needs).
template <int VPL>
__device__ __forceinline__ void quantize_terms_wgs(const RouteIn &in, int T, int H, int Kp,
                                                   uint8_t *xq, uint8_t *xs, int first, int fp4) {
    static_assert(VPL == 1 || VPL == 4, "one or four values per lane");
    constexpr int kU = 4;
    constexpr int kLanes = 32 / VPL;  // lanes per block
    const int nb = Kp / 32;
    const int total = T * nb;
    const int per_wg = static_cast<int>(blockDim.x) / kLanes;
    const int stride = (static_cast<int>(gridDim.x) - first) * per_wg;
    // VPL 1: the wavefront's two blocks are g0 (lanes 0..31) and g0 + 1
    const int lead = VPL == 1 ? 2 * (static_cast<int>(threadIdx.x) >> 6) : static_cast<int>(threadIdx.x) / kLanes;
    const int half = VPL == 1 ? (static_cast<int>(threadIdx.x) >> 5) & 1 : 0;
    for (int g0 = (static_cast<int>(blockIdx.x) - first) * per_wg + lead; g0 < total; g0 += kU * stride) {
        float v[kU][VPL];
#pragma unroll
        for (int u = 0; u < kU; ++u) quantize_input<VPL>(in, T, H, nb, g0 + u * stride + half, v[u]);
#pragma unroll
        for (int u = 0; u < kU; ++u)
            if (g0 + u * stride < total) quantize_store<VPL>(v[u], T, nb, Kp, xq, xs, g0 + u * stride + half, fp4);
    }
}

// ---------------------------------------------------------------- router logits
// Both router kernels write split-K partial sums partial[s][t][e] (fp64) over
// hidden-dimension slices; top-k adds the S partials in a fixed order and
// then the bias, so the logits are deterministic. fp32 x fp32 products are
// exact in fp64.

// Few tokens: one wavefront per (expert, hidden slice of kRouterGemvSlice
// units); lane l holds the router weights (and norm weights) of units
// 4(l + 64i) .. +3 of the slice in registers (all loads issued at once), then
// each token's activations are loaded the same way and reduced with a wave
// sum. Workgroups past router_wgs quantise the expert input.
template <int KIND, bool NORM>
__global__ __launch_bounds__(256) void router_gemv_kernel(RouteIn in, const float *w, int T,
                                                          int H, int E, double *partial,
                                                          int router_wgs, int Kp, uint8_t *xq,
                                                          uint8_t *xs, int fp4) {
    constexpr int NV = kRouterGemvSlice / 256;  // float4 per lane
    const int lane = threadIdx.x & 63;
    if (static_cast<int>(blockIdx.x) >= router_wgs) {
        quantize_terms_wgs<1>(in, T, H, Kp, xq, xs, router_wgs, fp4);
        return;
    }
    const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int S = (H + kRouterGemvSlice - 1) / kRouterGemvSlice;
    if (item >= E * S) return;  // whole wavefront; no workgroup barrier below
    const int e = item / S, s = item - e * S;
    const int hbase = s * kRouterGemvSlice;
    float4 wr[NV], gm[NV];
    bool on[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int h = hbase + 4 * (lane + 64 * i);
        on[i] = h < H;
        wr[i] = *reinterpret_cast<const float4 *>(w + static_cast<size_t>(e) * H + (on[i] ? h : 0));
        if constexpr (NORM) gm[i] = *reinterpret_cast<const float4 *>(in.gamma + (on[i] ? h : 0));
    }
    for (int t = 0; t < T; ++t) {
        double xv[NV][4];
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int h = hbase + 4 * (lane + 64 * i);
            load4<KIND>(in.x, static_cast<size_t>(t) * H + (on[i] ? h : 0), xv[i]);
        }
        if constexpr (NORM) {
            const double r = in.inv[t];
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                xv[i][0] = xv[i][0] * r * static_cast<double>(gm[i].x);
                xv[i][1] = xv[i][1] * r * static_cast<double>(gm[i].y);
                xv[i][2] = xv[i][2] * r * static_cast<double>(gm[i].z);
                xv[i][3] = xv[i][3] * r * static_cast<double>(gm[i].w);
            }
        }
        double acc = 0.0;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            if (on[i]) {
                acc = fma(static_cast<double>(wr[i].x), xv[i][0], acc);
                acc = fma(static_cast<double>(wr[i].y), xv[i][1], acc);
                acc = fma(static_cast<double>(wr[i].z), xv[i][2], acc);
                acc = fma(static_cast<double>(wr[i].w), xv[i][3], acc);
            }
        }
        acc = wave_sum_f64(acc);
        if (lane == 0) partial[(static_cast<size_t>(s) * T + t) * E + e] = acc;
    }
}

// Tiled router for larger batches: a workgroup computes the fp64 partial
// logits of 64 tokens x 64 experts over one K slice on the fp64 matrix cores
// (v_mfma_f64_16x16x4_f64): each of its 4 wavefronts holds 32 tokens x 32
// experts as 2 x 2 tiles of 16 x 16. K advances in chunks of 32 through
// double-buffered LDS tiles (float32, or fp64 once normalised; widened
// exactly to fp64 when read), 4 per instruction; the next chunk's loads are
// in flight during the current chunk's instructions. Tokens and experts past
// T and E are clamped on load and not written. Workgroup b < router_wgs takes
// token tile b % tiles_t, expert tile (b / tiles_t) % tiles_e and split
// b / (tiles_t * tiles_e); the rest quantise the expert input.
//
// Instruction lanes (measured on gfx950): operand A lane l = A[l % 16][l / 16]
// (token, k), operand B lane l = B[l / 16][l % 16] (k, expert); result lane l
// holds D[4v + l / 16][l % 16], v = 0..3.
typedef double f64x4_t __attribute__((ext_vector_type(4)));

template <int KIND, bool NORM>
__global__ __launch_bounds__(256) void router_tiled_kernel(RouteIn in, const float *w, int T,
                                                           int H, int E, int slice, int tiles_t,
                                                           int tiles_e, int router_wgs,
                                                           double *partial, int Kp, uint8_t *xq,
                                                           uint8_t *xs, int fp4) {
    typedef typename std::conditional<NORM, double, float>::type XT;
    constexpr int kPad = 4;
    __shared__ __align__(16) XT xsm[2][32][64 + kPad];    // [k][token]
    __shared__ __align__(16) float wsm[2][32][64 + kPad];  // [k][expert]
    const int b = blockIdx.x;
    if (b >= router_wgs) {
        quantize_terms_wgs<4>(in, T, H, Kp, xq, xs, router_wgs, fp4);
        return;
    }
    const int tid = threadIdx.x;
    const int t0 = (b % tiles_t) * 64, e0 = ((b / tiles_t) % tiles_e) * 64;
    const int s = b / (tiles_t * tiles_e);
    const int hbeg = s * slice, hend = min(H, hbeg + slice);
    // loads: thread -> (row tid / 4, k part 8 * (tid % 4)) of the 64 x 32 chunk
    const int lr = tid >> 2, lk = 8 * (tid & 3);
    const int trow = min(t0 + lr, T - 1);
    const size_t xrow = static_cast<size_t>(trow) * H;
    const float *wrow = w + static_cast<size_t>(min(e0 + lr, E - 1)) * H;
    double rinv = 0.0;
    if constexpr (NORM) rinv = in.inv[trow];
    XT xv[8];
    float wv[8];
    auto load = [&](int h0) {
        const int h = h0 + lk;
        if constexpr (NORM) {
            const float4 g0 = *reinterpret_cast<const float4 *>(in.gamma + h);
            const float4 g1 = *reinterpret_cast<const float4 *>(in.gamma + h + 4);
            const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
            for (int i = 0; i < 8; ++i)
                xv[i] = load_in<KIND>(in.x, xrow + h + i) * rinv * static_cast<double>(g[i]);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) xv[i] = static_cast<float>(load_in<KIND>(in.x, xrow + h + i));
        }
        const float4 a = *reinterpret_cast<const float4 *>(wrow + h);
        const float4 c = *reinterpret_cast<const float4 *>(wrow + h + 4);
        wv[0] = a.x; wv[1] = a.y; wv[2] = a.z; wv[3] = a.w;
        wv[4] = c.x; wv[5] = c.y; wv[6] = c.z; wv[7] = c.w;
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            xsm[buf][lk + i][lr] = xv[i];
            wsm[buf][lk + i][lr] = wv[i];
        }
    };
    const int lane = tid & 63, wave = tid >> 6;
    const int tb = (wave & 1) * 32, eb = (wave >> 1) * 32;  // the wavefront's tokens, experts
    const int col = lane & 15, kq = lane >> 4;
    f64x4_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f64x4_t{0.0, 0.0, 0.0, 0.0};
    load(hbeg);
    int buf = 0;
    for (int h0 = hbeg; h0 < hend; h0 += 32) {
        store(buf);
        __syncthreads();
        if (h0 + 32 < hend) load(h0 + 32);
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const int kk = 4 * ks + kq;
            double a[2], bb[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) a[i] = static_cast<double>(xsm[buf][kk][tb + 16 * i + col]);
#pragma unroll
            for (int j = 0; j < 2; ++j) bb[j] = static_cast<double>(wsm[buf][kk][eb + 16 * j + col]);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], bb[j], acc[i][j], 0, 0, 0);
        }
        buf ^= 1;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int t = t0 + tb + 16 * i + 4 * v + kq;
                const int e = e0 + eb + 16 * j + col;
                if (t < T && e < E) partial[(static_cast<size_t>(s) * T + t) * E + e] = acc[i][j][v];
            }
}

// ---------------------------------------------------------------- top-k
// One workgroup per token. Wavefront w adds the router partials of splits
// w, w + 4, w + 8, ... for the lane's experts e = lane + 64q (q < NQ, so
// E <= 64 NQ), issuing the loads of up to 16 / NQ splits at once (indices
// clamped, extra values masked): with at most 64 splits and E <= 64 the whole
// gather is one memory round trip. The four sums are added in wavefront
// order through LDS, then the bias; experts >= E get -inf. Wavefront 0 then
// takes top-k and the route weights.
template <int NQ>
__device__ __forceinline__ void gather_logits_wg(const double *partial, int S, int T, int t,
                                                 int E, const float *bias, double *red,
                                                 double (&v)[kMaxQ]) {
    constexpr int kU = NQ <= 16 ? 16 / NQ : 1;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    double acc[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) acc[q] = 0.0;
    for (int s0 = wave; s0 < S; s0 += 4 * kU) {
        double part[kU][NQ];
#pragma unroll
        for (int i = 0; i < kU; ++i) {
            const double *row = partial + (static_cast<size_t>(min(s0 + 4 * i, S - 1)) * T + t) * E;
#pragma unroll
            for (int q = 0; q < NQ; ++q) part[i][q] = row[min(lane + 64 * q, E - 1)];
        }
#pragma unroll
        for (int i = 0; i < kU; ++i)
#pragma unroll
            for (int q = 0; q < NQ; ++q)
                if (s0 + 4 * i < S) acc[q] += part[i][q];
    }
#pragma unroll
    for (int q = 0; q < NQ; ++q) red[wave * kMaxE + lane + 64 * q] = acc[q];
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kMaxQ; ++q) {
        const int e = lane + 64 * q;
        if (q < NQ && e < E) {
            const double sum =
                ((red[e] + red[kMaxE + e]) + red[2 * kMaxE + e]) + red[3 * kMaxE + e];
            v[q] = sum + static_cast<double>(bias[e]);
        } else {
            v[q] = -INFINITY;
        }
    }
}

__global__ __launch_bounds__(256) void topk_kernel(const double *partial, int S, const float *bias,
                                                   RouteSel rs, int T, int E, int k,
                                                   float route_scale, int32_t *idx, float *wts,
                                                   int32_t *out_idx, float *out_w) {
    __shared__ double red[4 * kMaxE];
    const int t = blockIdx.x;
    const int lane = threadIdx.x & 63;
    double v[kMaxQ];
    if (E <= 64) gather_logits_wg<1>(partial, S, T, t, E, bias, red, v);
    else if (E <= 128) gather_logits_wg<2>(partial, S, T, t, E, bias, red, v);
    else if (E <= 256) gather_logits_wg<4>(partial, S, T, t, E, bias, red, v);
    else gather_logits_wg<8>(partial, S, T, t, E, bias, red, v);
    if (threadIdx.x >= 64) return;  // after the workgroup barrier
    int sel[kMaxK];
    double val[kMaxK];
    if (E <= 64) select_routes<1>(v, rs, t, E, k, sel, val);
    else if (E <= 128) select_routes<2>(v, rs, t, E, k, sel, val);
    else if (E <= 256) select_routes<4>(v, rs, t, E, k, sel, val);
    else select_routes<8>(v, rs, t, E, k, sel, val);
    // lane j takes slot j's logit and expert; one exponential per lane
    double vj = val[0];
    int e = sel[0];
#pragma unroll
    for (int j = 1; j < kMaxK; ++j) {
        if (lane == j) {
            vj = val[j];
            e = sel[j];
        }
    }
    const float wl = route_weight_lanes(vj, k, route_scale);
    if (lane < k) {
        idx[t * k + lane] = e;
        wts[t * k + lane] = wl;
        if (out_idx) out_idx[t * k + lane] = e;
        if (out_w) out_w[t * k + lane] = wl;
    }
}

// ---------------------------------------------------------------- permutation
// Workgroups of 1024 threads, one per chunk of 1024 routes r = t*k + j (the
// workgroups past them quantise the expert input). Every chunk workgroup
// counts all routes per expert (LDS atomics), and apart the routes before its
// chunk; a workgroup scan of the counts gives the groups' offsets and the
// M-tile prefix for the grouped GEMMs (one group per thread; workgroup 0
// writes them). Its chunk's routes then start at offset + earlier routes of
// their expert: inside a wavefront the lanes holding the same expert are found
// with nine bit-plane ballots and ranked by lane, and per-wave counts are
// prefix-summed per expert in wave order, so a route's position counts exactly
// the earlier routes of its expert: the permutation is stable (ascending
// token), the same from every chunk in parallel as in one pass. Each route
// writes perm and inv at once.
// Group E (when n_shared) is the shared expert: T rows, identity order.
__global__ __launch_bounds__(1024) void permute_kernel(
    const int32_t *__restrict__ idx, int T, int E, int k, int n_shared, int bm, int nchunks,
    int32_t *counts, int32_t *offsets, int32_t *perm, int32_t *inv, int32_t *mprefix,
    int32_t *out_counts, int32_t *out_offsets, int32_t *out_perm, int32_t *out_inv,
    uint64_t *route_counts, RouteIn qin, int H, int Kp, uint8_t *xq, uint8_t *xs, int fp4) {
    __shared__ int wcnt[16][kMaxE];
    __shared__ int base[kMaxE + 1];
    __shared__ int before[kMaxE];
    const int chunk = static_cast<int>(blockIdx.x);
    if (chunk >= nchunks) {
        quantize_terms_wgs<4>(qin, T, H, Kp, xq, xs, nchunks, fp4);
        return;
    }
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int R = T * k, c0 = chunk * 1024;
    const bool writer = chunk == 0;  // workgroup 0 writes the counts, offsets and prefix
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int e = tid; e < E; e += 1024) {
        base[e] = 0;
        before[e] = 0;
    }
    // this chunk's route (its expert loads during the counting)
    const int r = c0 + tid;
    const bool valid = r < R;
    const int e = valid ? idx[r] : 0;
    __syncthreads();
    // lanes of a wavefront holding the same expert as this one: the
    // intersection of the bit-plane ballots of the expert index (9 planes:
    // E <= 512)
    static_assert(kMaxE <= 512, "expert indices fit 9 bit planes");
    auto same_expert = [&](int ex, bool on) __attribute__((always_inline)) {
        uint64_t eq = __ballot(on);
#pragma unroll
        for (int bt = 0; bt < 9; ++bt) {
            const bool bit = (ex >> bt) & 1;
            const uint64_t plane = __ballot(bit);
            eq &= bit ? plane : ~plane;
        }
        return eq;
    };
    // the experts' route counts, and those of the routes before this chunk
    // (LDS atomics; loads four rounds at a time)
    for (int r0 = tid; r0 < R; r0 += 4 * 1024) {
        int ev[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int rr = r0 + u * 1024;
            ev[u] = rr < R ? idx[rr] : -1;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (ev[u] >= 0) {
                atomicAdd(&base[ev[u]], 1);
                if (r0 + u * 1024 < c0) atomicAdd(&before[ev[u]], 1);
            }
        }
    }
    __syncthreads();
    // counts, their exclusive scan and the tile prefix: one group per thread
    // (G <= kMaxE + 1 <= 1024), wavefront scans, then the totals of the
    // wavefronts before; base[g] becomes the first position of group g's
    // routes in this chunk
    const int G = E + n_shared;
    __shared__ int wsum_c[16], wsum_t[16];
    {
        const int g = tid;
        const int c = g < G ? (g < E ? base[g] : T) : 0;
        const int nt = (c + bm - 1) / bm;
        int sc = c, st = nt;  // inclusive scans within the wavefront
        for (int d = 1; d < 64; d <<= 1) {
            const int oc = __shfl_up(sc, d), ot = __shfl_up(st, d);
            if (lane >= d) {
                sc += oc;
                st += ot;
            }
        }
        if (lane == 63) {
            wsum_c[w] = sc;
            wsum_t[w] = st;
        }
        __syncthreads();
        int pc = 0, pt = 0;
        for (int ww = 0; ww < w; ++ww) {
            pc += wsum_c[ww];
            pt += wsum_t[ww];
        }
        const int off = pc + sc - c, mt = pt + st - nt;
        __syncthreads();  // every count is read before base[] turns into positions
        if (g < E) base[g] = off + before[g];
        if (writer) {
            if (g < G) {
                offsets[g] = off;
                mprefix[g] = mt;
                counts[g] = c;
                if (out_counts && g < E) out_counts[g] = c;
                // route profile: this call's selections of expert g (one atomic per expert)
                if (route_counts && g < E && c > 0)
                    atomicAdd(reinterpret_cast<unsigned long long *>(route_counts + g),
                              static_cast<unsigned long long>(c));
                if (out_offsets && g < E) out_offsets[g] = off;
            }
            if (g == G - 1) {
                offsets[G] = off + c;
                mprefix[G] = mt + nt;
            }
            if (out_offsets && g == 0) out_offsets[E] = R;
        }
    }
    // positions of this chunk's routes
    for (int i = tid; i < 16 * kMaxE; i += 1024) wcnt[i / kMaxE][i % kMaxE] = 0;
    __syncthreads();
    const uint64_t eq = same_expert(e, valid);
    const int myrank = __popcll(eq & lt_mask);
    if (valid && myrank == 0) wcnt[w][e] = __popcll(eq);  // the first lane of its expert
    __syncthreads();
    for (int ee = tid; ee < E; ee += 1024) {
        int run = base[ee];
        for (int ww = 0; ww < 16; ++ww) {
            const int c = wcnt[ww][ee];
            wcnt[ww][ee] = run;
            run += c;
        }
    }
    __syncthreads();
    if (valid) {
        const int pos = wcnt[w][e] + myrank;
        perm[pos] = r;
        inv[r] = pos;
        if (out_perm) out_perm[pos] = r;
        if (out_inv) out_inv[r] = pos;
    }
}

}  // namespace

hipError_t launch_rms_inv(const void *x, int x_bf16, int T, int H, float eps, double *inv,
                          hipStream_t s) {
    if (x_bf16) launch_kernel(rms_inv_kernel<1>, T, 256, s, x, H, eps, inv);
    else launch_kernel(rms_inv_kernel<0>, T, 256, s, x, H, eps, inv);
    return hipGetLastError();
}

RouterPlan router_plan(int T, int H, int E) {
    RouterPlan p;
    if (T <= kRouterGemvMaxT) {
        p.gemv = true;
        p.slice = kRouterGemvSlice;
        p.splits = (H + kRouterGemvSlice - 1) / kRouterGemvSlice;
        return p;
    }
    const int tiles = ((T + 63) / 64) * ((E + 63) / 64);
    int want = (1024 + tiles - 1) / tiles;
    want = want < 1 ? 1 : (want > kRouterMaxSplits ? kRouterMaxSplits : want);
    const int units = H / 32;
    if (want > units) want = units;
    p.gemv = false;
    p.slice = 32 * ((units + want - 1) / want);
    p.splits = (H + p.slice - 1) / p.slice;
    return p;
}

namespace {
template <int KIND, bool NORM>
void router_launch(const RouterPlan &p, const RouteIn &in, const float *w, int T, int H, int E,
                   double *partial, int qwant, uint8_t *xq, uint8_t *xs, int fp4, hipStream_t s) {
    const int Kp = pad128(H);
    if (p.gemv) {
        const int rwgs = (E * p.splits + 3) / 4;
        launch_kernel(router_gemv_kernel<KIND, NORM>, rwgs + qwant, 256, s, in, w, T, H, E,
                      partial, rwgs, Kp, xq, xs, fp4);
    } else {
        const int tt = (T + 63) / 64, te = (E + 63) / 64;
        const int rwgs = tt * te * p.splits;
        const int qwgs = qwant < kQuantizeMaxWgs ? qwant : kQuantizeMaxWgs;
        launch_kernel(router_tiled_kernel<KIND, NORM>, rwgs + qwgs, 256, s, in, w, T, H, E,
                      p.slice, tt, te, rwgs, partial, Kp, xq, xs, fp4);
    }
}
}  // namespace

hipError_t launch_router(const RouteIn &in, const float *w, int T, int H, int E, double *partial,
                         const TermsOut *terms, hipStream_t s) {
    const RouterPlan p = router_plan(T, H, E);
    // quantisation workgroups, one round each: 8 blocks of 32 values beside the
    // GEMV (one value per lane), 32 beside the tiled router (four per lane)
    const int per_wg = p.gemv ? 8 : 32;
    const int qwant = terms ? (T * (pad128(H) / 32) + per_wg - 1) / per_wg : 0;
    uint8_t *xq = terms ? terms->q : nullptr;
    uint8_t *xs = terms ? terms->scales : nullptr;
    const int fp4 = terms ? terms->fp4 : 0;
    if (in.inv) {
        if (in.bf16) router_launch<1, true>(p, in, w, T, H, E, partial, qwant, xq, xs, fp4, s);
        else router_launch<0, true>(p, in, w, T, H, E, partial, qwant, xq, xs, fp4, s);
    } else {
        if (in.bf16) router_launch<1, false>(p, in, w, T, H, E, partial, qwant, xq, xs, fp4, s);
        else router_launch<0, false>(p, in, w, T, H, E, partial, qwant, xq, xs, fp4, s);
    }
    return hipGetLastError();
}

namespace {
// Rows of H values (the block count per row H / 32 in place of pad128(H) / 32,
// so that rows are packed without padding).
__global__ __launch_bounds__(256) void act_fp4_kernel(RouteIn in, int T, int H, uint8_t *q,
                                                      uint8_t *scales) {
    quantize_terms_wgs<4>(in, T, H, H, q, scales, 0, 1);
}
}  // namespace

hipError_t launch_act_fp4(const RouteIn &in, int T, int H, uint8_t *q, uint8_t *scales,
                          hipStream_t s) {
    const int want = (T * (H / 32) + 31) / 32;  // one round of 32 blocks per workgroup
    launch_kernel(act_fp4_kernel, want < kQuantizeMaxWgs ? want : kQuantizeMaxWgs, 256, s, in, T, H,
                  q, scales);
    return hipGetLastError();
}

hipError_t launch_topk(const double *partial, int S, const float *bias, const RouteSel &rs, int T,
                       int E, int k, float route_scale, int32_t *idx, float *wts, int32_t *out_idx,
                       float *out_w, hipStream_t s) {
    launch_kernel(topk_kernel, T, 256, s, partial, S, bias, rs, T, E, k, route_scale, idx, wts,
                  out_idx, out_w);
    return hipGetLastError();
}

hipError_t launch_permute(const int32_t *idx, int T, int E, int k, int n_shared, int tile_rows,
                          int32_t *counts,
                          int32_t *offsets, int32_t *perm, int32_t *inv,
                          int32_t *mprefix, int32_t *out_counts, int32_t *out_offsets,
                          int32_t *out_perm, int32_t *out_inv, uint64_t *route_counts,
                          const RouteIn *qin, int H, const TermsOut *terms, hipStream_t s) {
    const int Kp = pad128(H);
    int qwgs = 0;
    if (terms) {
        const int want = (T * (Kp / 32) + 127) / 128;  // one round of 128 blocks each
        qwgs = want < kPermuteQuantizeWgs ? want : kPermuteQuantizeWgs;
    }
    const RouteIn none{nullptr, 0, nullptr, nullptr, nullptr};
    const int nchunks = (T * k + 1023) / 1024;
    launch_kernel(permute_kernel, nchunks + qwgs, 1024, s, idx, T, E, k, n_shared, tile_rows, nchunks, counts,
                  offsets, perm, inv, mprefix, out_counts, out_offsets, out_perm, out_inv,
                  route_counts, terms ? *qin : none, H, Kp, terms ? terms->q : nullptr,
                  terms ? terms->scales : nullptr, terms ? terms->fp4 : 0);
    return hipGetLastError();
}

}  // namespace moe
