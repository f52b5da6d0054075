// Operands of the gfx950 block-scaled matrix-core instruction
// v_mfma_scale_f32_16x16x128_f8f6f4 as the MoE kernels use it: MXFP4 weights
// (E2M1 codes + E8M0 block scales, exactly the packed blob's bytes) as
// operand A, activations as FP8 (E4M3) terms with E8M0 block scales as
// operand B. The hardware multiplies each 32-value block by its two scales.
//
// Lane roles, measured on gfx950 with FP4 A and FP8 B:
//  - A: lane l holds the 16 code bytes of MX block g = l / 16 (k = 32g..32g+31
//    of the 128-wide step) of tile row l % 16, and that block's scale byte.
//  - B: lane l is column n = l % 16 with k-group h = l / 16; its 32 bytes are
//    k = 16h..16h+15 (bytes 0..15) and k = 64+16h..64+16h+15 (bytes 16..31)
//    of the step, and its scale byte applies to the 32-value block k = 32h..
//    32h+31 of the step (natural k order, as for A).
//  - D: lane l holds rows 4 * (l / 16) + v, v = 0..3, of column l % 16.
//
// Columns carry (row, term) pairs, 4 rows x kTerms terms per instruction;
// after the instruction, a sum over each lane quad (the terms of one row)
// gives that row's dot product.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

static_assert(kTerms == 4, "four FP8 terms fill a lane quad of the B operand");

struct AFrag {
    uint4 q;
    uint32_t s;
};

struct BFrag {
    uint4 lo, hi;
    uint32_t s;
};

// A operand: 16-row tile `tile` of a packed plane, 128-wide step `step`. On a
// ragged last step the lanes past the plane's blocks re-read its last block;
// the B operand is zero there, so they add nothing.
__device__ __forceinline__ AFrag load_afrag(const uint8_t *codes, const uint8_t *scales, int tile,
                                            int step, int nblk, int lane) {
    const uint32_t blk = static_cast<uint32_t>(min(4 * step + (lane >> 4), nblk - 1));
    const uint32_t row = static_cast<uint32_t>(16 * tile + (lane & 15));
    AFrag a;
    a.q = *reinterpret_cast<const uint4 *>(codes + mx_code_offset(row, blk, nblk));
    a.s = scales[mx_scale_offset(row, blk, nblk)];
    return a;
}

// Per-lane byte offsets of A fragments inside a 16-row tile: step s of a
// tile starting at (uniform) code base cb and scale base sb reads cb +
// code(s) and sb + scale(s). Only the last step can be ragged; there the lanes
// past the plane's blocks re-read its last block (their B operand is zero).
struct ALane {
    uint32_t q, sc;          // step 0
    uint32_t q_last, s_last;  // step ns - 1
    int ns;
    __device__ __forceinline__ ALane(int nblk, int lane) {
        ns = (nblk + 3) >> 2;
        const int g = lane >> 4, r = lane & 15;
        q = static_cast<uint32_t>((16 * g + r) * 16);
        sc = static_cast<uint32_t>(16 * g + r);
        const int gl = min(g, nblk - 1 - 4 * (ns - 1));
        q_last = static_cast<uint32_t>((ns - 1) * 1024 + (16 * gl + r) * 16);
        s_last = static_cast<uint32_t>((ns - 1) * 64 + 16 * gl + r);
    }
    __device__ __forceinline__ uint32_t code(int s) const { return s >= ns - 1 ? q_last : q + 1024u * s; }
    __device__ __forceinline__ uint32_t scale(int s) const { return s >= ns - 1 ? s_last : sc + 64u * s; }
};

// Byte offset of 16-row tile `tile` in a code / scale plane with nblk blocks per row.
__device__ __forceinline__ uint64_t tile_code_base(int tile, int nblk) { return static_cast<uint64_t>(tile) * 256u * nblk; }
__device__ __forceinline__ uint64_t tile_scale_base(int tile, int nblk) { return static_cast<uint64_t>(tile) * 16u * nblk; }

// A fragment of step s (clamped to the last step) of the tile at cb / sb.
__device__ __forceinline__ AFrag load_afrag(const uint8_t *cb, const uint8_t *sb, const ALane &al, int s) {
    AFrag a;
    a.q = *reinterpret_cast<const uint4 *>(cb + al.code(s));
    a.s = sb[al.scale(s)];
    return a;
}

// B operand from one FP8-term row (codes `q`, scales `sc`, natural k order,
// zero past the true K) for lane k-group h.
__device__ __forceinline__ BFrag load_bfrag(const uint8_t *q, const uint8_t *sc, int step, int h) {
    BFrag b;
    b.lo = *reinterpret_cast<const uint4 *>(q + 128 * step + 16 * h);
    b.hi = *reinterpret_cast<const uint4 *>(q + 128 * step + 64 + 16 * h);
    b.s = sc[4 * step + h];
    return b;
}

__device__ __forceinline__ f32x4_t mx_mfma(const AFrag &a, const uint4 &blo, const uint4 &bhi,
                                           uint32_t bs, f32x4_t acc) {
    const i32x8_t A = {static_cast<int>(a.q.x), static_cast<int>(a.q.y), static_cast<int>(a.q.z),
                       static_cast<int>(a.q.w), 0, 0, 0, 0};
    const i32x8_t B = {static_cast<int>(blo.x), static_cast<int>(blo.y), static_cast<int>(blo.z),
                       static_cast<int>(blo.w), static_cast<int>(bhi.x), static_cast<int>(bhi.y),
                       static_cast<int>(bhi.z), static_cast<int>(bhi.w)};
    // cbsz 4: A is FP4 (E2M1); blgp 0: B is FP8 (E4M3); byte 0 of each scale operand is E8M0
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, acc, 4, 0, 0, static_cast<int>(a.s),
                                                             0, static_cast<int>(bs));
}

__device__ __forceinline__ f32x4_t mx_mfma(const AFrag &a, const BFrag &b, f32x4_t acc) {
    return mx_mfma(a, b.lo, b.hi, b.s, acc);
}

// Both operands FP4 (the quantised expert-input mode): B lane l is column
// l % 16 with the 32 codes of MX block h = l / 16 of the step (k = 32h ..
// 32h + 31, as for A), 16 bytes, and that block's scale byte.
__device__ __forceinline__ f32x4_t mx_mfma_fp4(const AFrag &a, const uint4 &b, uint32_t bs,
                                               f32x4_t acc) {
    const i32x8_t A = {static_cast<int>(a.q.x), static_cast<int>(a.q.y), static_cast<int>(a.q.z),
                       static_cast<int>(a.q.w), 0, 0, 0, 0};
    const i32x8_t B = {static_cast<int>(b.x), static_cast<int>(b.y), static_cast<int>(b.z),
                       static_cast<int>(b.w), 0, 0, 0, 0};
    // cbsz 4 and blgp 4: both operands FP4 (E2M1)
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, acc, 4, 4, 0, static_cast<int>(a.s),
                                                             0, static_cast<int>(bs));
}

// Sum over the lane quad (the kTerms columns of one row).
__device__ __forceinline__ float quad_sum(float v) {
    v += __builtin_amdgcn_update_dpp(0.0f, v, 0xB1, 0xf, 0xf, false);  // quad_perm [1,0,3,2]
    v += __builtin_amdgcn_update_dpp(0.0f, v, 0x4E, 0xf, 0xf, false);  // quad_perm [2,3,0,1]
    return v;
}

}  // namespace moe
