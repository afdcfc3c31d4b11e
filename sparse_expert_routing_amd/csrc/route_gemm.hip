// Router for bf16 activations, in three kernels: an exact three-way bf16
// split of the fp32 router weights, the fp32 logits x . w_router[e] by bf16
// MFMA, and the biased top-k choice with renormalised unbiased weights.
//
// DeepSeek V3 From Scratch, "In code" (route) and "Worked example": the
// affinity is the sigmoid of the router logit; the bias is added for the
// choice of the top 8 only; the weights are the chosen unbiased affinities
// over their sum.  kbwen.com DeepSeek feed, "A bias term for each expert":
// the gating value comes from the original score.
//
// Why the split is exact: an fp32 w is hi + mid + lo with each term a bf16
// (hi = rne(w), mid = rne(w - hi), lo = w - hi - mid: 24 mantissa bits in
// three 8-bit pieces; both remainders are exact fp32 subtractions).  A bf16 x
// times a bf16 term is exact in fp32 (8 x 8 mantissa bits), so the logit is
// the fp32 accumulation of exact products -- the arithmetic of an fp32 dot
// product, on the bf16 matrix cores (16x the fp32 MFMA rate, 3 MFMAs per
// product block).
//
// Logits kernel: one workgroup per 128 tokens x 128 experts, 4 waves (2x2)
// of 64x64, v_mfma_f32_32x32x16_bf16 with the operands swapped so a lane
// ends up owning one token and runs of 4 consecutive experts (16-byte fp32
// stores).  Both operands go global -> LDS with global_load_lds_dwordx4
// (A: 128 x 64 bf16, B: 3 x 128 x 64 bf16 per stage, two stages), rows of
// 128 bytes with XOR-swizzled 16-byte pieces; the next stage's loads are
// spread over the current stage's MFMAs.  As in the fused fp32 router, the
// accumulators are folded into running totals every 512 of K.  For small T
// the K range is split over blockIdx.z so about 256 workgroups run; the
// top-k kernel adds the partial logits in split order.
#include "device.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kE = 256;
constexpr int RM = 128;        // tokens per tile
constexpr int RN = 128;        // experts per tile
constexpr int RK = 64;         // K per stage (128-byte rows)
constexpr int kRegion = RM * RK;  // bf16 elements of one 128 x 64 operand region
constexpr int kStage = 4 * kRegion;  // A + 3 B splits (64 KB)
constexpr int kFlush = 512;

typedef __attribute__((address_space(3))) void lds_void_t;

__global__ __launch_bounds__(256) void k_router_split(int n, const float *__restrict__ w, uint16_t *__restrict__ hi,
                                                     uint16_t *__restrict__ mid, uint16_t *__restrict__ lo) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const float v = w[i];
    const uint32_t h = f32_to_bf16(v);
    const float r1 = v - bf16_to_f32(h);
    const uint32_t m = f32_to_bf16(r1);
    const float r2 = r1 - bf16_to_f32(m);
    hi[i] = (uint16_t)h;
    mid[i] = (uint16_t)m;
    lo[i] = (uint16_t)f32_to_bf16(r2);
}

__device__ __forceinline__ int piece(int row, int c) {
    return row * RK + ((c ^ (row & 7) ^ ((row >> 3) & 1)) * 8);
}

// blockIdx.z: K range [z*nk/S, (z+1)*nk/S) of the S = gridDim.z splits; its
// partial logits go to logits + z*T*E (the top-k kernel sums them in order).
__global__ __launch_bounds__(256, 1) void k_router_logits(int T, int d, const uint16_t *__restrict__ x,
                                                         const uint16_t *__restrict__ wsplit,
                                                         float *__restrict__ logits) {
    __shared__ __attribute__((aligned(1024))) uint16_t smem[2 * kStage];  // 128 KB
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1, g = lane >> 5;
    const int m0 = blockIdx.x * RM, n0 = blockIdx.y * RN;
    const int nk_all = d / RK, S = gridDim.z, z = blockIdx.z;
    const int kb0 = (int)((long long)nk_all * z / S), nk = (int)((long long)nk_all * (z + 1) / S) - kb0;
    logits += (size_t)z * T * kE;

    // DMA geometry: each region is 16 blocks of 8 rows x 128 B; wave w moves
    // blocks w, w+4, w+8, w+12 of every region (16 loads per stage).
    const uint16_t *src[16];
    int dst[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int region = i >> 2, rb = wave + 4 * (i & 3);
        const int row = 8 * rb + (lane >> 3);
        const int col = ((lane & 7) ^ (row & 7) ^ ((row >> 3) & 1)) * 8;
        if (region == 0) {
            const int t = min(m0 + row, T - 1);
            src[i] = x + (size_t)t * d + (size_t)kb0 * RK + col;
        } else {
            src[i] = wsplit + ((size_t)(region - 1) * kE + n0 + row) * d + (size_t)kb0 * RK + col;
        }
        dst[i] = region * kRegion + rb * 512;
    }

    f32x16 acc[2][2], tot[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = tot[i][j][r] = 0.f;

#define ISSUE(i_, stage_, slot_)                                                               \
    __builtin_amdgcn_global_load_lds(static_cast<const void *>(src[i_] + (size_t)(stage_) * RK), \
                                     (lds_void_t *)(smem + (slot_) * kStage + dst[i_]), 16, 0, 0)

#pragma unroll
    for (int i = 0; i < 16; ++i) ISSUE(i, 0, 0);

    for (int kt = 0; kt < nk; ++kt) {
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt((7 << 4));  // vmcnt(0), lgkmcnt(0): stage kt landed for this wave
        __builtin_amdgcn_s_barrier();          // ... for all waves; stage kt-1 no longer read
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        const uint16_t *sA = smem + (kt & 1) * kStage;
        // stage kt+1 into the idle slot; past the end the last stage is
        // reloaded there (never read), which keeps the loads unconditional
        const int kn = min(kt + 1, nk - 1), nslot = (kt + 1) & 1;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int c = 2 * kk + g;
            bf16x8 af[2], bfr[3][2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                af[i] = *reinterpret_cast<const bf16x8 *>(sA + piece(wm * 64 + 32 * i + (lane & 31), c));
#pragma unroll
            for (int s = 0; s < 3; ++s)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    bfr[s][j] = *reinterpret_cast<const bf16x8 *>(sA + (1 + s) * kRegion +
                                                                    piece(wn * 64 + 32 * j + (lane & 31), c));
#pragma unroll
            for (int s = 0; s < 3; ++s)
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[s][j], af[i], acc[i][j], 0, 0, 0);
                        // the next stage's loads, 4 per K step, between the MFMAs
                        if (i == 1 && j == 1) ISSUE(4 * kk + s, kn, nslot);
                        if (s == 2 && i == 1 && j == 1) ISSUE(4 * kk + 3, kn, nslot);
                    }
        }
        if ((kb0 + kt + 1) * RK % kFlush == 0 || kt + 1 == nk) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    tot[i][j] += acc[i][j];
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
                }
        }
    }
#undef ISSUE
    __builtin_amdgcn_s_waitcnt((7 << 4));  // the last (redundant) loads landed before the workgroup ends

    // lane: token wm*64 + 32i + (lane & 31); experts wn*64 + 32j + 8q + 4g + 0..3
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int t = m0 + wm * 64 + 32 * i + (lane & 31);
        if (t < T) {
            float *lrow = logits + (size_t)t * kE + n0 + wn * 64;
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    *reinterpret_cast<f32x4 *>(lrow + 32 * j + 8 * q + 4 * g) =
                        f32x4{tot[i][j][4 * q], tot[i][j][4 * q + 1], tot[i][j][4 * q + 2], tot[i][j][4 * q + 3]};
        }
    }
}

// One wave per token: sigmoid affinities of its 256 logits, biased top-k by
// 64-bit (ordered score, 255 - id) keys (equal scores resolve to the lower
// id), ids ascending, weights = chosen affinities over their sum, and the
// k-th minus (k+1)-th biased score when asked.
template <int kK>
__global__ __launch_bounds__(256) void k_route_topk(int T, int S, const float *__restrict__ logits,
                                                   const float *__restrict__ bias, int32_t *__restrict__ idx,
                                                   float *__restrict__ wts, float *__restrict__ gap) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    float sv[4], l[4];
    uint64_t key[4];
    const float *lt = logits + (size_t)t * kE + lane;
#pragma unroll
    for (int q = 0; q < 4; ++q) l[q] = lt[64 * q];
    // K splits, added in split order; unrolled so several loads are in flight
#pragma unroll 4
    for (int z = 1; z < S; ++z) {
        const float *lz = lt + (size_t)z * T * kE;
#pragma unroll
        for (int q = 0; q < 4; ++q) l[q] += lz[64 * q];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int e = lane + 64 * q;
        sv[q] = 1.0f / (1.0f + expf(-l[q]));
        key[q] = ((uint64_t)f32_order_key(sv[q] + bias[e]) << 32) | (uint32_t)(kE - 1 - e);
    }
    constexpr int kRounds = kK + 1;  // one extra round gives the gap
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
#pragma unroll
    for (int a = 1; a < kK; ++a)
#pragma unroll
        for (int c = a; c > 0; --c) {
            const int lo = sel[c - 1] < sel[c] ? sel[c - 1] : sel[c];
            const int hi = sel[c - 1] < sel[c] ? sel[c] : sel[c - 1];
            sel[c - 1] = lo;
            sel[c] = hi;
        }
    float s_sel[kK];
    float sum = 0.f;
#pragma unroll
    for (int j = 0; j < kK; ++j) {
        const int q = sel[j] >> 6;  // wave-uniform
        const float mine = q == 0 ? sv[0] : q == 1 ? sv[1] : q == 2 ? sv[2] : sv[3];
        s_sel[j] = __shfl(mine, sel[j] & 63, kWave);
        sum += s_sel[j];
    }
#pragma unroll
    for (int j = 0; j < kK; ++j)
        if (lane == j) {
            idx[(size_t)t * kK + j] = sel[j];
            wts[(size_t)t * kK + j] = s_sel[j] / sum;
        }
    if (gap != nullptr && lane == 0)
        gap[t] = f32_from_order_key((uint32_t)(kth >> 32)) - f32_from_order_key((uint32_t)(k1th >> 32));
}

}  // namespace

// K splits of the logits GEMM: up to about 256 workgroups for small T, each
// split keeping at least 4 K steps so its prologue and epilogue stay small.
static int route_ksplit(int T, int d) {
    const int tiles = (T + RM - 1) / RM * (kE / RN);
    const int cap = d / RK / 4;
    const int S = 256 / tiles;
    return S > cap ? (cap < 1 ? 1 : cap) : (S < 1 ? 1 : S);
}

size_t route_bf16_ws_bytes(int T, int d) {
    const size_t split = ((size_t)3 * kE * d * sizeof(uint16_t) + 255) / 256 * 256;
    return split + (size_t)route_ksplit(T, d) * T * kE * sizeof(float);
}

bool route_bf16_ok(int d) { return d % RK == 0; }

hipError_t launch_route_bf16(const RouteArgs &a, void *ws, hipStream_t s) {
    uint16_t *wsplit = static_cast<uint16_t *>(ws);
    const size_t split = ((size_t)3 * kE * a.d * sizeof(uint16_t) + 255) / 256 * 256;
    float *logits = reinterpret_cast<float *>(static_cast<char *>(ws) + split);
    const int n = kE * a.d;
    hipLaunchKernelGGL(k_router_split, dim3((n + 255) / 256), dim3(256), 0, s, n, a.wr, wsplit, wsplit + n,
                       wsplit + 2 * (size_t)n);
    const int S = route_ksplit(a.T, a.d);
    hipLaunchKernelGGL(k_router_logits, dim3((a.T + RM - 1) / RM, kE / RN, S), dim3(256), 0, s, a.T, a.d,
                       static_cast<const uint16_t *>(a.x), wsplit, logits);
    hipLaunchKernelGGL((k_route_topk<8>), dim3((a.T + 3) / 4), dim3(256), 0, s, a.T, S, logits, a.bias, a.idx,
                       a.w, a.gap);
    return hipGetLastError();
}

}  // namespace moe
