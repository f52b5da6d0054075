// Device-side building blocks shared by the MoE kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.hpp"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- MXFP4
// An E8M0 scale byte b stands for 2^(b-127); as float32 bits that is b << 23
// (exact for b in 1..254).
__device__ __forceinline__ float e8m0_scale(uint32_t b) { return __uint_as_float(b << 23); }

// Eight E2M1 codes packed in one dword (element 2i in the low nibble of byte i)
// decoded and scaled to bfloat16 with the gfx950 scaled FP4 converts; any
// E2M1 value times 2^n is exact in bfloat16.
__device__ __forceinline__ bf16x8_t fp4x8_to_bf16(uint32_t q, float s) {
    bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, s, 0);
    bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, s, 1);
    bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, s, 2);
    bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, s, 3);
    return bf16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// Same eight codes decoded to float32 (exact), times s.
__device__ __forceinline__ void fp4x8_to_f32(uint32_t q, float s, float (&w)[8]) {
    f32x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, s, 0);
    f32x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, s, 1);
    f32x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, s, 2);
    f32x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, s, 3);
    w[0] = p0[0]; w[1] = p0[1]; w[2] = p1[0]; w[3] = p1[1];
    w[4] = p2[0]; w[5] = p2[1]; w[6] = p3[0]; w[7] = p3[1];
}

// Dot product of one 32-element MX block (16 code bytes, scale s) with 32
// float32 activations held in registers.
__device__ __forceinline__ float mx_block_dot(uint4 q, float s, const float (&x)[32]) {
    float acc = 0.f;
    const uint32_t d[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float w[8];
        fp4x8_to_f32(d[i], s, w);
#pragma unroll
        for (int j = 0; j < 8; ++j) acc = fmaf(w[j], x[8 * i + j], acc);
    }
    return acc;
}

// ---------------------------------------------------------------- bfloat16
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// x = hi + lo with hi = bf16(x) and lo = bf16(x - hi): 16 significant bits,
// enough that the two-term bf16 products keep float32-level accuracy.
__device__ __forceinline__ void split_bf16(float x, __bf16 &hi, __bf16 &lo) {
    hi = static_cast<__bf16>(x);
    lo = static_cast<__bf16>(x - static_cast<float>(hi));
}

// ---------------------------------------------------------------- wave sums
// Sum over the 64 lanes with DPP row operations; the total lands in lane 63
// and is broadcast with readlane. All lanes must be active.
__device__ __forceinline__ float wave_sum(float v) {
    v += __builtin_amdgcn_update_dpp(0.0f, v, 0xB1, 0xf, 0xf, false);   // quad_perm [1,0,3,2]
    v += __builtin_amdgcn_update_dpp(0.0f, v, 0x4E, 0xf, 0xf, false);   // quad_perm [2,3,0,1]
    v += __builtin_amdgcn_update_dpp(0.0f, v, 0x141, 0xf, 0xf, false);  // row_half_mirror
    v += __builtin_amdgcn_update_dpp(0.0f, v, 0x140, 0xf, 0xf, false);  // row_mirror
    v += __builtin_amdgcn_update_dpp(0.0f, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
    v += __builtin_amdgcn_update_dpp(0.0f, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// float64 through the 32-bit DPP / readlane paths, one half at a time.
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
    const uint64_t b = static_cast<uint64_t>(__double_as_longlong(v));
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(b), CTRL, 0xf, 0xf, false));
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(b >> 32), CTRL, 0xf, 0xf, false));
    return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}

__device__ __forceinline__ double readlane_f64(double v, int lane) {
    const uint64_t b = static_cast<uint64_t>(__double_as_longlong(v));
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(b), lane));
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(b >> 32), lane));
    return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}

// Sum over the 64 lanes in a fixed order (rows of 16 by DPP, then the four
// row sums), the same in every lane. All lanes must be active.
__device__ __forceinline__ double wave_sum_f64(double v) {
    v += dpp_f64<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp_f64<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp_f64<0x141>(v);  // row_half_mirror
    v += dpp_f64<0x140>(v);  // row_mirror
    return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}

__device__ __forceinline__ double wave_max_f64(double v) {
    v = fmax(v, dpp_f64<0xB1>(v));
    v = fmax(v, dpp_f64<0x4E>(v));
    v = fmax(v, dpp_f64<0x141>(v));
    v = fmax(v, dpp_f64<0x140>(v));
    return fmax(fmax(readlane_f64(v, 0), readlane_f64(v, 16)), fmax(readlane_f64(v, 32), readlane_f64(v, 48)));
}

// ---------------------------------------------------------------- SwiGLU
// Clamped SwiGLU: gate clamped above at `limit`, up clamped to [-limit, limit],
// a = g * sigmoid(alpha * g) * (u + up_offset).
__device__ __forceinline__ float swiglu(float g, float u, float alpha, float limit, float up_off) {
    g = fminf(g, limit);
    u = fminf(fmaxf(u, -limit), limit);
    return g * __frcp_rn(1.0f + __expf(-alpha * g)) * (u + up_off);
}

// ---------------------------------------------------------------- top-k
// Logits of one token for the lane's experts e = lane + 64q (q < NQ, so
// E <= 64 NQ): the router's split-K partial sums (partial[s][t][e], fp64)
// plus the bias; experts >= E get -inf. The partials are added in the one
// order every top-k of the library uses: four running sums over the splits
// s = c, c + 4, c + 8, ... (c = 0..3), each in increasing s, combined as
// ((sum0 + sum1) + sum2) + sum3, then the bias (the workgroup top-k has
// wavefront c make sum c). The loads of each group of kGatherUnroll splits
// are issued together (indices clamped, extra values masked) so the gather
// costs one memory round trip per group; the biases load with the first
// group, and `between` (loads of the caller's own, issued behind the first
// group so that the sums wait only for the partials) runs right after it
// (up to 128 experts; past that, before it).
constexpr int kGatherUnroll = 8;
static_assert(kGatherUnroll % 4 == 0, "a group keeps each split in its residue class");
struct NoLoads {
    __device__ void operator()() const {}
};
template <int NQ, typename Between = NoLoads>
__device__ __forceinline__ void gather_logits(const double *partial, int S, int T, int t, int E,
                                              const float *bias, double (&v)[kMaxQ],
                                              Between &&between = Between{}) {
    const int lane = threadIdx.x & (kWave - 1);
    double acc[4][NQ];
    float bq[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) bq[q] = bias[min(lane + kWave * q, E - 1)];
    // with more than 128 experts a group's partials take too many registers to
    // hold the caller's loads as well: those go out first
    if constexpr (NQ > 2) between();
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int q = 0; q < NQ; ++q) acc[c][q] = 0.0;
    for (int s0 = 0; s0 < S; s0 += kGatherUnroll) {
        double part[kGatherUnroll][NQ];
#pragma unroll
        for (int i = 0; i < kGatherUnroll; ++i) {
            const double *row = partial + (static_cast<size_t>(min(s0 + i, S - 1)) * T + t) * E;
#pragma unroll
            for (int q = 0; q < NQ; ++q) part[i][q] = row[min(lane + kWave * q, E - 1)];
        }
        if constexpr (NQ <= 2)
            if (s0 == 0) between();
#pragma unroll
        for (int i = 0; i < kGatherUnroll; ++i)
#pragma unroll
            for (int q = 0; q < NQ; ++q)
                if (s0 + i < S) acc[i & 3][q] += part[i][q];
    }
#pragma unroll
    for (int q = 0; q < kMaxQ; ++q) {
        const int e = lane + kWave * q;
        const int qq = q < NQ ? q : 0;
        v[q] = (q < NQ && e < E)
                   ? ((acc[0][qq] + acc[1][qq]) + acc[2][qq]) + acc[3][qq] + static_cast<double>(bq[qq])
                   : -INFINITY;
    }
}

// Top-k of one token's fp64 logits (E <= 64 NQ <= kMaxE) by one wavefront;
// vin[q] holds the lane's expert l + 64q. Each round takes the wave maximum
// over the experts still in play, then the lowest expert index holding it
// (ballot per group of 64: lanes are in index order inside a group, groups in
// index order), and retires it; so the result is by descending value with
// equal values in ascending index order. A NaN logit counts as -inf, so every
// returned index is a distinct valid expert whatever the input.
// sel[j] and val[j] are uniform across the wave on return.
template <int NQ>
__device__ __forceinline__ void wave_topk(const double (&vin)[kMaxQ], int E, int k, int *sel,
                                          double *val) {
    const int lane = threadIdx.x & (kWave - 1);
    double v[NQ];
    bool alive[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        alive[q] = lane + kWave * q < E;
        v[q] = vin[q] == vin[q] ? vin[q] : -INFINITY;
    }
    // rounds unrolled to kMaxK with a guard: constant indices keep sel / val
    // in registers
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
        if (j >= k) break;
        double m = -INFINITY;
#pragma unroll
        for (int q = 0; q < NQ; ++q)
            if (alive[q]) m = fmax(m, v[q]);
        m = wave_max_f64(m);
        int chosen = -1;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const uint64_t hit = __ballot(alive[q] && v[q] == m);
            if (chosen < 0 && hit) chosen = kWave * q + (__ffsll(static_cast<long long>(hit)) - 1);
        }
        sel[j] = chosen;
        val[j] = m;
#pragma unroll
        for (int q = 0; q < NQ; ++q)
            if (lane + kWave * q == chosen) alive[q] = false;
    }
}

// Route weight of slot `lane` (lanes < k; the others get 0): route_scale *
// softmax over the k selected logits, in fp64, shifted by their maximum. The
// lanes take one exponential each and the sum adds the slots in order (every
// top-k of the library makes its weights here). v: the lane's slot logit.
__device__ __forceinline__ float route_weight_lanes(double v, int k, float scale) {
    const int lane = threadIdx.x & (kWave - 1);
    double m = -INFINITY;
    double vs[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
        vs[j] = __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), j),
                                 __builtin_amdgcn_readlane(__double2loint(v), j));
        if (j == 0) m = vs[0];
        else if (j < k) m = fmax(m, vs[j]);
    }
    const double z = exp(v - m);
    double s = 0.0;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j)
        if (j < k)
            s += __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(z), j),
                                  __builtin_amdgcn_readlane(__double2loint(z), j));
    return lane < k ? static_cast<float>(scale * z / s) : 0.0f;
}

// Logit of expert e (wave-uniform) from the lanes' values v[q] (expert l + 64q).
// Every group's value is read from lane e % 64 and the group e / 64 picked
// among the read values (a pick among v[q] itself would become an indexed
// access that puts v in scratch).
template <int NQ>
__device__ __forceinline__ double wave_logit(const double (&v)[kMaxQ], int e) {
    const int l = e & (kWave - 1), g = e >> 6;
    double x = 0.0;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int lo = __builtin_amdgcn_readlane(__double2loint(v[q]), l);
        const int hi = __builtin_amdgcn_readlane(__double2hiint(v[q]), l);
        if (g == q) x = __hiloint2double(hi, lo);
    }
    return x;
}

// The k experts of token t and their (unbiased) logits, by one wavefront:
// plain top-k of v, top-k of v + bias, or the table row of the token's id.
// Ids and table entries outside their ranges are clamped into them (every
// access stays in bounds). sel / val are wave-uniform on return.
template <int NQ>
__device__ __forceinline__ void select_routes(const double (&v)[kMaxQ], const RouteSel &rs, int t,
                                              int E, int k, int *sel, double *val) {
    // slot loops run over kMaxK with a guard, so every array index is a
    // compile-time constant (a runtime index would put sel / val in scratch)
    if (rs.table) {
        const int id = min(max(rs.ids[t], 0), rs.vocab - 1);
#pragma unroll
        for (int j = 0; j < kMaxK; ++j) {
            if (j < k) {
                const int e = min(max(rs.table[static_cast<size_t>(id) * k + j], 0), E - 1);
                sel[j] = e;
                val[j] = wave_logit<NQ>(v, e);
            }
        }
        return;
    }
    if (rs.bias) {
        const int lane = threadIdx.x & (kWave - 1);
        double vb[kMaxQ];
#pragma unroll
        for (int q = 0; q < kMaxQ; ++q) {
            const int e = lane + kWave * q;
            vb[q] = (q < NQ && e < E) ? v[q] + static_cast<double>(rs.bias[e]) : -INFINITY;
        }
        wave_topk<NQ>(vb, E, k, sel, val);
#pragma unroll
        for (int j = 0; j < kMaxK; ++j)
            if (j < k) val[j] = wave_logit<NQ>(v, sel[j]);
        return;
    }
    wave_topk<NQ>(v, E, k, sel, val);
}

// ---------------------------------------------------------------- XCD tiles
// Logical tile of workgroup `bid` when tiles are dealt so that each XCD (one
// L2) sweeps a contiguous range of the tile list. Returns false for spare
// workgroups of an over-sized grid.
__device__ __forceinline__ bool xcd_tile(int bid, int ntiles, int &tile) {
    const int xcd = bid % kXcds, slot = bid / kXcds;
    const int per = (ntiles + kXcds - 1) / kXcds;
    tile = xcd * per + slot;
    return slot < per && tile < ntiles;
}

}  // namespace moe

namespace moe {

// ---------------------------------------------------------------- FP8 terms
// Activations meet MXFP4 weights on the block-scaled matrix cores as a sum of
// kTerms FP8 (OCP E4M3) vectors, each with its own E8M0 scales: term n holds
// what terms 0..n-1 left over, so every extra term adds about four
// significant bits (kTerms = 4: ~16 bits, float32-level products).

// OCP E4M3 code of x, |x| < 448, rounded to nearest (ties to even), and its
// value: the gfx950 conversion instructions, which round to nearest even with
// subnormals (measured bit for bit against a software encoder of the format on
// 2^20 values, ties and subnormals included: no differences). No branches, so
// the term loops below stay straight-line code.
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
    return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(x, 0.0f, 0, false)) & 0xffu;
}

__device__ __forceinline__ float e4m3_decode(uint32_t c) {
    return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(c), 0);
}

// 2^e as float32 for e in [-126, 127].
__device__ __forceinline__ float pow2f(int e) { return __uint_as_float(static_cast<uint32_t>(e + 127) << 23); }

// Maximum over each half-wavefront (lanes 0..31 and 32..63) of a value that
// is >= 0, returned to every lane of that half: DPP within rows of 16 lanes,
// then the two rows of a half combined through readlanes.
__device__ __forceinline__ float half_wave_max(float v) {
    v = fmaxf(v, __builtin_amdgcn_update_dpp(0.0f, v, 0xB1, 0xf, 0xf, false));   // quad_perm [1,0,3,2]
    v = fmaxf(v, __builtin_amdgcn_update_dpp(0.0f, v, 0x4E, 0xf, 0xf, false));   // quad_perm [2,3,0,1]
    v = fmaxf(v, __builtin_amdgcn_update_dpp(0.0f, v, 0x141, 0xf, 0xf, false));  // row_half_mirror
    v = fmaxf(v, __builtin_amdgcn_update_dpp(0.0f, v, 0x140, 0xf, 0xf, false));  // row_mirror
    const int b = __float_as_int(v);
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(b, 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(b, 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(b, 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(b, 48));
    return (threadIdx.x & 32) ? fmaxf(r2, r3) : fmaxf(r0, r1);
}

// Split the 32 values held by the 32 lanes of a half-wavefront into kTerms
// E4M3 codes, term n with the E8M0 scale 2^(e0 - 4n), e0 = floor(log2 amax) - 7
// (so the first term's codes lie in [128, 256) x 2^e0 at the block maximum).
// After term n every value is within half an E4M3 step of that term, at most
// 8 x 2^(e0 - 4n), so term n + 1 sees at most 128 x its own scale and never
// saturates; after kTerms terms the error is at most 2^(e0 - 4 kTerms + 7),
// i.e. about 2^-4kTerms of the block maximum. Returns the codes packed in one
// dword (term n in byte n) and the scale bytes likewise. Every lane of the
// wavefront must take part (one half-wavefront maximum).
__device__ __forceinline__ void fp8_terms_group(float v, uint32_t &codes, uint32_t &scales) {
    const float amax = half_wave_max(fabsf(v));
    const int e0 = static_cast<int>((__float_as_uint(amax) >> 23) & 0xffu) - 127 - 7;
    codes = 0;
    scales = 0;
    float r = v;
#pragma unroll
    for (int n = 0; n < kTerms; ++n) {
        int e = e0 - 4 * n;
        e = e < -126 ? -126 : (e > 127 ? 127 : e);
        const uint32_t q = e4m3_encode(r * pow2f(-e));
        r -= e4m3_decode(q) * pow2f(e);
        codes |= q << (8 * n);
        scales |= static_cast<uint32_t>(e + 127) << (8 * n);
    }
}

// ---------------------------------------------------------------- MX-FP4 activations
// The MX-FP4 round trip of 32 activations held by the 32 lanes of a
// half-wavefront (the quantised expert-input mode): one shared power-of-two
// scale 2^e, the smallest with amax <= 6 * 2^e (amax held at no less than
// 6 * 2^-126), and per value the E2M1 code of the nearest magnitude of
// x / 2^e clamped to [-6, 6], ties to the even code, with the sign of x (a
// value not below zero, -0 included, is positive). x / 2^e is exact, so the
// thresholds decide exactly as a software quantiser on the same float32 x.
// Returns the lane's code (0..15) and the block's E8M0 scale byte e + 127.
// Every lane of the wavefront must take part (one half-wavefront maximum).
__device__ __forceinline__ uint32_t fp4_act_code(float v, uint32_t &scale_byte) {
    const float amax = fmaxf(half_wave_max(fabsf(v)), 7.052966104933725e-38f);  // 6 * 2^-126
    const uint32_t bits = __float_as_uint(amax);
    const int E = static_cast<int>((bits >> 23) & 0xffu) - 127;
    const int e = (bits & 0x7fffffu) <= 0x400000u ? E - 2 : E - 1;  // amax <= 1.5 * 2^E: 6 * 2^(E-2) fits
    scale_byte = static_cast<uint32_t>(e + 127);
    const float a = fminf(fabsf(v) * pow2f(-e), 6.0f);
    // nearest of {0, .5, 1, 1.5, 2, 3, 4, 6}; a midpoint goes to the even index
    const uint32_t idx = static_cast<uint32_t>(a > 0.25f) + static_cast<uint32_t>(a >= 0.75f) +
                         static_cast<uint32_t>(a > 1.25f) + static_cast<uint32_t>(a >= 1.75f) +
                         static_cast<uint32_t>(a > 2.5f) + static_cast<uint32_t>(a >= 3.5f) +
                         static_cast<uint32_t>(a > 5.0f);
    return idx | (v < 0.0f ? 8u : 0u);
}

// The byte holding the codes of this lane and the next (even lanes: element
// 2i in the low nibble); the value in odd lanes is meaningless.
__device__ __forceinline__ uint32_t fp4_pack_pair(uint32_t code) {
    const uint32_t next = static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(0, static_cast<int>(code), 0x39, 0xf, 0xf, false));  // quad_perm [1,2,3,0]
    return (code & 0xfu) | ((next & 0xfu) << 4);
}

}  // namespace moe
