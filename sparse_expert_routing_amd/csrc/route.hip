// Router: fp32 logits x . w_router[e], sigmoid affinities, biased top-k choice
// and renormalised unbiased weights, fused in one kernel.
//
// DeepSeek V3 From Scratch, "In code" (route) and "Worked example": the
// affinity is the sigmoid of the router logit; the bias is added for the
// choice of the top 8 only; the weights are the chosen unbiased affinities
// over their sum.  kbwen.com DeepSeek feed, "A bias term for each expert":
// the gating value comes from the original score.
//
// Layout: one workgroup of 4 waves owns a tile of 64 tokens and all 256
// experts.  The x tile is staged in LDS (shared by the 4 waves) as fp32; wave
// w reads its 64 router rows straight from global memory (no other wave uses
// them) in the fp32 MFMA operand layout.  The K loop runs
// v_mfma_f32_16x16x4_f32 on 4x4 16x16 tiles per wave.  The epilogue writes the
// 64x256 affinity tile to LDS; each wave then selects the top-k of 16 tokens
// with 64-bit (score, id) keys reduced across the wavefront, so equal scores
// resolve to the lower expert id deterministically.
//
// Accuracy: the fp32 accumulators are flushed into a second set of totals
// every 512 of K, which keeps the rounding error of the d-long dot product
// near that of a 512-long one plus d/512 additions (fewer flips of
// near-tied choices against an fp64 reference).
#include "device.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kTok = 64;   // tokens per workgroup
constexpr int kBK = 32;    // K per LDS stage
constexpr int kE = 256;    // experts (4 waves x 64)
constexpr int kXPad = 4;
constexpr int kSPad = 4;
constexpr int kChunk = 512;  // K between flushes of the partial accumulators

template <bool kXBf16, int kK>
__global__ __launch_bounds__(256) void k_route(int T, int d, const void *__restrict__ x,
                                               const float *__restrict__ wr,
                                               const float *__restrict__ bias,
                                               int32_t *__restrict__ idx, float *__restrict__ wts,
                                               float *__restrict__ gap) {
    // x tile during the K loop, affinity tile afterwards.
    __shared__ float lds[kTok * (kE + kSPad)];
    float(*xs)[kBK + kXPad] = reinterpret_cast<float(*)[kBK + kXPad]>(lds);
    float(*ss)[kE + kSPad] = reinterpret_cast<float(*)[kE + kSPad]>(lds);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int t0 = blockIdx.x * kTok;
    const int n0 = wave * 64;

    f32x4 acc[4][4], tot[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = tot[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // staging assignment: thread -> (row, 8 consecutive columns)
    const int ld_row = tid >> 2, ld_col = (tid & 3) * 8;
    const bool ld_ok = (t0 + ld_row) < T;
    const float *wrow[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) wrow[j] = wr + (size_t)(n0 + 16 * j + (lane & 15)) * d + 4 * (lane >> 4);

    for (int k0 = 0; k0 < d; k0 += kBK) {
        float v[8];
        if (kXBf16) {
            uint4 raw = make_uint4(0, 0, 0, 0);
            if (ld_ok)
                raw = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(x) +
                                                       (size_t)(t0 + ld_row) * d + k0 + ld_col);
            v[0] = bf16_to_f32(raw.x & 0xffffu); v[1] = bf16_to_f32(raw.x >> 16);
            v[2] = bf16_to_f32(raw.y & 0xffffu); v[3] = bf16_to_f32(raw.y >> 16);
            v[4] = bf16_to_f32(raw.z & 0xffffu); v[5] = bf16_to_f32(raw.z >> 16);
            v[6] = bf16_to_f32(raw.w & 0xffffu); v[7] = bf16_to_f32(raw.w >> 16);
        } else {
            float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
            if (ld_ok) {
                const float *p = static_cast<const float *>(x) + (size_t)(t0 + ld_row) * d + k0 + ld_col;
                a = *reinterpret_cast<const float4 *>(p);
                b = *reinterpret_cast<const float4 *>(p + 4);
            }
            v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
            v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
        }
        __syncthreads();  // previous stage fully consumed
        *reinterpret_cast<float4 *>(&xs[ld_row][ld_col]) = make_float4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<float4 *>(&xs[ld_row][ld_col + 4]) = make_float4(v[4], v[5], v[6], v[7]);
        __syncthreads();

#pragma unroll
        for (int kk = 0; kk < kBK; kk += 16) {
            float4 wv[4], xv[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) wv[j] = *reinterpret_cast<const float4 *>(wrow[j] + k0 + kk);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                xv[i] = *reinterpret_cast<const float4 *>(&xs[16 * i + (lane & 15)][kk + 4 * (lane >> 4)]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(xv[i].x, wv[j].x, acc[i][j], 0, 0, 0);
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(xv[i].y, wv[j].y, acc[i][j], 0, 0, 0);
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(xv[i].z, wv[j].z, acc[i][j], 0, 0, 0);
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(xv[i].w, wv[j].w, acc[i][j], 0, 0, 0);
                }
        }
        if ((k0 + kBK) % kChunk == 0 || k0 + kBK >= d) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    tot[i][j] += acc[i][j];
                    acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
        }
    }
    __syncthreads();  // x tile dead; reuse LDS for the affinities

    // C layout of a 16x16 MFMA tile: lane holds column (lane & 15) and rows
    // 4 * (lane >> 4) + r.
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float l = tot[i][j][r];
                ss[16 * i + 4 * (lane >> 4) + r][n0 + 16 * j + (lane & 15)] = 1.0f / (1.0f + expf(-l));
            }
    __syncthreads();

    float b[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) b[q] = bias[lane + 64 * q];

    constexpr int kRounds = kK + 1;  // one extra round gives the gap
    for (int tt = 0; tt < kTok / 4; ++tt) {
        const int tl = wave * (kTok / 4) + tt;
        const int t = t0 + tl;
        if (t >= T) break;
        uint64_t key[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int e = lane + 64 * q;
            const float v = ss[tl][e] + b[q];  // fp32 biased score
            key[q] = ((uint64_t)f32_order_key(v) << 32) | (uint32_t)(kE - 1 - e);
        }
        int sel[kK];
        uint64_t kth = 0, k1th = 0;
#pragma unroll
        for (int r = 0; r < kRounds; ++r) {
            if (r == kK && gap == nullptr) break;
            uint64_t m = key[0];
#pragma unroll
            for (int q = 1; q < 4; ++q) m = key[q] > m ? key[q] : m;
            m = wave_max_u64(m);
            const int e = kE - 1 - (int)(uint32_t)m;
            if (r < kK) sel[r] = e;
            if (r == kK - 1) kth = m;
            if (r == kK) k1th = m;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (e == lane + 64 * q) key[q] = 0;
        }
        // ascending id order
#pragma unroll
        for (int a = 1; a < kK; ++a)
#pragma unroll
            for (int c = a; c > 0; --c) {
                const int lo = sel[c - 1] < sel[c] ? sel[c - 1] : sel[c];
                const int hi = sel[c - 1] < sel[c] ? sel[c] : sel[c - 1];
                sel[c - 1] = lo;
                sel[c] = hi;
            }
        float sum = 0.f;
#pragma unroll
        for (int j = 0; j < kK; ++j) sum += ss[tl][sel[j]];
#pragma unroll
        for (int j = 0; j < kK; ++j)
            if (lane == j) {
                idx[(size_t)t * kK + j] = sel[j];
                wts[(size_t)t * kK + j] = ss[tl][sel[j]] / sum;
            }
        if (gap != nullptr && lane == 0)
            gap[t] = f32_from_order_key((uint32_t)(kth >> 32)) - f32_from_order_key((uint32_t)(k1th >> 32));
    }
}

}  // namespace

hipError_t launch_route(const RouteArgs &a, hipStream_t s) {
    const dim3 grid((a.T + kTok - 1) / kTok), block(256);
    if (a.x_bf16)
        hipLaunchKernelGGL((k_route<true, 8>), grid, block, 0, s, a.T, a.d, a.x, a.wr, a.bias, a.idx, a.w, a.gap);
    else
        hipLaunchKernelGGL((k_route<false, 8>), grid, block, 0, s, a.T, a.d, a.x, a.wr, a.bias, a.idx, a.w, a.gap);
    return hipGetLastError();
}

}  // namespace moe
