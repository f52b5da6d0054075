// Export of decoded MXFP4 weights, through exactly the conversions the GEMV
// (float32) and matrix-core (bfloat16) kernels use, for bit-exact checks.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

// One thread per 32-element MX block.
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t *codes, const uint8_t *scales,
                                                      int rows, int K, int path, float *out) {
    const int nblk = K / 32;
    const long long b = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (b >= static_cast<long long>(rows) * nblk) return;
    const int row = static_cast<int>(b / nblk), kb = static_cast<int>(b % nblk);
    const uint4 q = *reinterpret_cast<const uint4 *>(codes + static_cast<size_t>(row) * (K / 2) + 16 * kb);
    const float s = e8m0_scale(scales[static_cast<size_t>(row) * nblk + kb]);
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

}  // namespace

hipError_t launch_dequant(const uint8_t *codes, const uint8_t *scales, int rows, int K, int path,
                          float *out, hipStream_t s) {
    const long long blocks = static_cast<long long>(rows) * (K / 32);
    const int grid = static_cast<int>((blocks + 255) / 256);
    if (grid == 0) return hipSuccess;
    launch_kernel(dequant_kernel, grid, 256, s, codes, scales, rows, K, path, out);
    return hipGetLastError();
}

}  // namespace moe
