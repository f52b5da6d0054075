// Export of decoded MXFP4 weights from a packed (tiled) plane, for bit-exact
// checks: through the scaled FP4 converts (float32 or bfloat16), or through
// the block-scaled matrix core itself, the route every forward kernel takes.
#include "mx_mfma.hpp"

namespace moe {

namespace {

// One thread per 32-element MX block (row-major block order).
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t *codes, const uint8_t *scales,
                                                      int rows, int K, int path, float *out) {
    const int nblk = K / 32;
    const long long b = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (b >= static_cast<long long>(rows) * nblk) return;
    const int row = static_cast<int>(b / nblk), kb = static_cast<int>(b % nblk);
    const uint4 q = *reinterpret_cast<const uint4 *>(codes + mx_code_offset(row, kb, nblk));
    const float s = e8m0_scale(scales[mx_scale_offset(row, kb, nblk)]);
    const uint32_t d[4] = {q.x, q.y, q.z, q.w};
    float *o = out + static_cast<size_t>(row) * K + 32 * kb;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (path == 0) {
            float w[8];
            fp4x8_to_f32(d[i], s, w);
#pragma unroll
            for (int j = 0; j < 8; ++j) o[8 * i + j] = w[j];
        } else {
            const bf16x8_t v = fp4x8_to_bf16(d[i], s);
#pragma unroll
            for (int j = 0; j < 8; ++j) o[8 * i + j] = static_cast<float>(v[j]);
        }
    }
}

// One wavefront per (16-row tile, 128-wide step): eight instructions, each
// with B = 1.0 (E4M3 0x38, scale 2^0) at k = 16j + n of column n, so column n
// of D is weight column 16j + n exactly as the matrix core decodes it.
__global__ __launch_bounds__(64) void dequant_mfma_kernel(const uint8_t *codes,
                                                          const uint8_t *scales, int K,
                                                          float *out) {
    const int lane = threadIdx.x, tile = blockIdx.x, s = blockIdx.y;
    const int nblk = K / 32;
    const AFrag a = load_afrag(codes, scales, tile, s, nblk, lane);
    const int n = lane & 15, h = lane >> 4;
    const uint32_t one = 0x38u << (8 * (n & 3));
    for (int j = 0; j < 8; ++j) {
        uint32_t lo[4] = {0u, 0u, 0u, 0u}, hi[4] = {0u, 0u, 0u, 0u};
        if (j < 4 && h == j) lo[n >> 2] = one;
        if (j >= 4 && h == j - 4) hi[n >> 2] = one;
        const f32x4_t d = mx_mfma(a, make_uint4(lo[0], lo[1], lo[2], lo[3]),
                                  make_uint4(hi[0], hi[1], hi[2], hi[3]), 127u,
                                  f32x4_t{0.f, 0.f, 0.f, 0.f});
        const int col = 128 * s + 16 * j + n;
        if (col < K) {
#pragma unroll
            for (int v = 0; v < 4; ++v)
                out[static_cast<size_t>(16 * tile + 4 * h + v) * K + col] = d[v];
        }
    }
}

}  // namespace

hipError_t launch_dequant(const uint8_t *codes, const uint8_t *scales, int rows, int K, int path,
                          float *out, hipStream_t s) {
    if (path == 2) {
        const dim3 grid(rows / 16, pad128(K) / 128);
        if (grid.x == 0) return hipSuccess;
        launch_kernel(dequant_mfma_kernel, grid, 64, s, codes, scales, K, out);
        return hipGetLastError();
    }
    const long long blocks = static_cast<long long>(rows) * (K / 32);
    const int grid = static_cast<int>((blocks + 255) / 256);
    if (grid == 0) return hipSuccess;
    launch_kernel(dequant_kernel, grid, 256, s, codes, scales, rows, K, path, out);
    return hipGetLastError();
}

}  // namespace moe
