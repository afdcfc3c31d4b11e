// Sign-step bias update (DeepSeek V3 From Scratch, "In code": update_bias;
// kbwen.com DeepSeek feed, "A bias term for each expert"): once per step,
// from the whole batch's load, every expert's bias moves by the same fixed
// amount towards balance.  With load c/T and target k/E the sign of
// (target - load) is the sign of k*T - E*c, evaluated exactly in 64-bit
// integers; an expert exactly on target keeps its bias.
#include "device.h"
#include "kernels.h"

namespace moe {

namespace {

__global__ __launch_bounds__(256) void k_bias_update(int E, int k, int T, const int32_t *__restrict__ counts,
                                                     float gamma, float *__restrict__ bias) {
    const int e = blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= E) return;
    const long long diff = (long long)k * T - (long long)E * counts[e];
    const float sg = diff > 0 ? 1.0f : (diff < 0 ? -1.0f : 0.0f);
    bias[e] = bias[e] + gamma * sg;  // gamma * sg is exact: one fp32 rounding
}

}  // namespace

hipError_t launch_bias_update(int E, int k, int T, const int32_t *counts, float gamma, float *bias,
                              hipStream_t s) {
    hipLaunchKernelGGL(k_bias_update, dim3((E + 255) / 256), dim3(256), 0, s, E, k, T, counts, gamma, bias);
    return hipGetLastError();
}

}  // namespace moe
