// Weighted combine of the routed expert outputs onto the shared expert's
// output, as a pass of its own (used where the shared expert's GEMM does not
// fuse it): y[t] += sum_j w[t, j] * y_perm[row_of[t*k + j]], j ascending, in
// fp32 on top of the shared expert's unrounded fp32 output.
//
// Scaling Efficiency: A Deep Dive into the DeepSeek-V3 Architecture,
// "Implementation: A Modular Look": the layer output is the shared output plus
// the routed outputs scaled by their gate weights.
//
// One wave per token: the token's k row indices and weights are wave-uniform
// (scalar loads); each gathered routed row is read as contiguous 1 KB runs
// (64 lanes x 8 bf16), the y row as 2 KB runs, two runs in flight per lane.
#include "device.h"
#include "kernels.h"

namespace moe {

namespace {

template <int kK>
__global__ __launch_bounds__(256) void k_combine_add(int T, int d, const uint16_t *__restrict__ y_perm,
                                                    const int32_t *__restrict__ row_of,
                                                    const float *__restrict__ cw, float *__restrict__ y) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (t >= T) return;
    int rof[kK];
    float w[kK];
#pragma unroll
    for (int j = 0; j < kK; ++j) {
        rof[j] = row_of[(size_t)t * kK + j];
        w[j] = cw[(size_t)t * kK + j];
    }
    float *yr = y + (size_t)t * d;
#pragma unroll 2
    for (int c = 8 * lane; c < d; c += 512) {
        const f32x4 s0 = *reinterpret_cast<const f32x4 *>(yr + c);
        const f32x4 s1 = *reinterpret_cast<const f32x4 *>(yr + c + 4);
        float v[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
        i32x4 g[kK];
#pragma unroll
        for (int j = 0; j < kK; ++j) g[j] = *reinterpret_cast<const i32x4 *>(y_perm + (size_t)rof[j] * d + c);
#pragma unroll
        for (int j = 0; j < kK; ++j)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                v[2 * u] += w[j] * bf16_to_f32((uint32_t)g[j][u] & 0xffffu);
                v[2 * u + 1] += w[j] * bf16_to_f32((uint32_t)g[j][u] >> 16);
            }
        *reinterpret_cast<f32x4 *>(yr + c) = f32x4{v[0], v[1], v[2], v[3]};
        *reinterpret_cast<f32x4 *>(yr + c + 4) = f32x4{v[4], v[5], v[6], v[7]};
    }
}

}  // namespace

hipError_t launch_combine_add(int T, int d, int k, const uint16_t *y_perm, const int32_t *row_of, const float *cw,
                              float *y, hipStream_t s) {
    if (k != 8 || d % 8 != 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_combine_add<8>), dim3((T + 3) / 4), dim3(256), 0, s, T, d, y_perm, row_of, cw, y);
    return hipGetLastError();
}

}  // namespace moe
