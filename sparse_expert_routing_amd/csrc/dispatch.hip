// Dispatch: per-expert load (histogram), exclusive scan, stable permutation of
// the T*k assignments by expert, and the row gather into x_perm (with the
// 1x128-tile e4m3 quantisation when the expert GEMMs run in fp8).
//
// Load per expert: DeepSeek V3 From Scratch, "In code" (update_bias: the load
// is the fraction of tokens per expert).  Grouping tokens by expert: Scaling
// Efficiency: A Deep Dive into the DeepSeek-V3 Architecture, "Implementation:
// A Modular Look" (each expert runs on the tokens that chose it, in token
// order).  No capacity and no drops: kbwen.com DeepSeek feed, "A bias term for
// each expert".  FP8 with a scale per tile: crackai.dev DeepSeek-V3 summary, "How
// It Works".
//
// Determinism: no atomic return value ever decides a position.  Within a
// block of 256 tokens each wave builds, in LDS, one 64-bit token mask per
// expert (bit = lane); the rank of an assignment inside its expert is the
// popcount of the earlier tokens' bits plus the counts of earlier waves and
// earlier blocks, so the permutation is the stable counting sort.
#include "device.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kE = 256;
constexpr int kK = 8;
constexpr int kWaves = kDispatchBlock / 64;

// Build mask[w][e] for the block's tokens.  Each token's k ids are distinct.
// An id outside [0, E) is not dispatched (no mask bit; k_disp_rank gives it
// row -1), so it can neither write out of bounds nor take a row.
__device__ __forceinline__ void build_masks(uint64_t (*mask)[kE], int T, const int32_t *__restrict__ idx,
                                            int t, int lane, int wave, int32_t (&ids)[kK]) {
    for (int e = threadIdx.x; e < kWaves * kE; e += blockDim.x) (&mask[0][0])[e] = 0ull;
    __syncthreads();
    if (t < T) {
        const int4 *p = reinterpret_cast<const int4 *>(idx + (size_t)t * kK);
        int4 a = p[0], b = p[1];
        ids[0] = a.x; ids[1] = a.y; ids[2] = a.z; ids[3] = a.w;
        ids[4] = b.x; ids[5] = b.y; ids[6] = b.z; ids[7] = b.w;
#pragma unroll
        for (int j = 0; j < kK; ++j)
            if ((unsigned)ids[j] < (unsigned)kE)
                atomicOr(reinterpret_cast<unsigned long long *>(&mask[wave][ids[j]]), 1ull << lane);
    }
    __syncthreads();
}

__global__ __launch_bounds__(kDispatchBlock) void k_disp_count(int T, const int32_t *__restrict__ idx,
                                                             int32_t *__restrict__ block_cnt) {
    __shared__ uint64_t mask[kWaves][kE];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t = blockIdx.x * kDispatchBlock + threadIdx.x;
    int32_t ids[kK];
    build_masks(mask, T, idx, t, lane, wave, ids);
    const int e = threadIdx.x;  // blockDim == E
    int c = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) c += __popcll(mask[w][e]);
    block_cnt[(size_t)blockIdx.x * kE + e] = c;
}

// One workgroup: per expert, exclusive scan of the block counts (in place ->
// block base), total count, then the exclusive scan over experts.
__global__ __launch_bounds__(kE) void k_disp_scan(int nblk, int32_t *__restrict__ block_cnt,
                                                  int32_t *__restrict__ counts, int32_t *__restrict__ offsets) {
    __shared__ int part[kE / 64];
    const int e = threadIdx.x, lane = e & 63, wave = e >> 6;
    int run = 0;
    int b = 0;
    for (; b + 8 <= nblk; b += 8) {
        int v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = block_cnt[(size_t)(b + u) * kE + e];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            block_cnt[(size_t)(b + u) * kE + e] = run;
            run += v[u];
        }
    }
    for (; b < nblk; ++b) {
        int v = block_cnt[(size_t)b * kE + e];
        block_cnt[(size_t)b * kE + e] = run;
        run += v;
    }
    counts[e] = run;
    int incl = wave_incl_scan(run);
    if (lane == 63) part[wave] = incl;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave; ++w) base += part[w];
    const int excl = base + incl - run;
    offsets[e] = excl;
    if (e == kE - 1) offsets[kE] = excl + run;
    for (b = 0; b < nblk; ++b) block_cnt[(size_t)b * kE + e] += excl;
}

__global__ __launch_bounds__(kDispatchBlock) void k_disp_rank(int T, const int32_t *__restrict__ idx,
                                                            const int32_t *__restrict__ block_base,
                                                            int32_t *__restrict__ row_src,
                                                            int32_t *__restrict__ row_of) {
    __shared__ uint64_t mask[kWaves][kE];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t = blockIdx.x * kDispatchBlock + threadIdx.x;
    int32_t ids[kK];
    build_masks(mask, T, idx, t, lane, wave, ids);
    if (t >= T) return;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
    for (int j = 0; j < kK; ++j) {
        const int e = ids[j];
        const int f = t * kK + j;
        if ((unsigned)e >= (unsigned)kE) {  // not dispatched
            row_of[f] = -1;
            continue;
        }
        int r = block_base[(size_t)blockIdx.x * kE + e] + __popcll(mask[wave][e] & below);
        for (int w = 0; w < wave; ++w) r += __popcll(mask[w][e]);
        row_src[r] = f;
        row_of[f] = r;
    }
}

// Copy each token row to its k permuted rows: one wave per token, the row is
// read once and written k times in 16-byte pieces.
__global__ __launch_bounds__(256) void k_disp_gather_copy(int T, int row_bytes, const uint8_t *__restrict__ x,
                                                          const int32_t *__restrict__ row_of,
                                                          uint8_t *__restrict__ x_perm) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    int32_t dst[kK];
#pragma unroll
    for (int j = 0; j < kK; ++j) dst[j] = row_of[(size_t)t * kK + j];
    const int nchunk = row_bytes / 16;
    const uint4 *src = reinterpret_cast<const uint4 *>(x + (size_t)t * row_bytes);
    for (int c = lane; c < nchunk; c += 64) {
        const uint4 v = src[c];
#pragma unroll
        for (int j = 0; j < kK; ++j)
            if (dst[j] >= 0) reinterpret_cast<uint4 *>(x_perm + (size_t)dst[j] * row_bytes)[c] = v;
    }
}

// Quantise one bf16 row piece: lane holds 8 values of a 128-wide tile that 16
// consecutive lanes share.  Returns the 8 codes packed in a uint2 and the
// tile scale's E8M0 byte.
__device__ __forceinline__ uint2 quant8(uint4 raw, uint8_t &scale) {
    float v[8];
    v[0] = bf16_to_f32(raw.x & 0xffffu); v[1] = bf16_to_f32(raw.x >> 16);
    v[2] = bf16_to_f32(raw.y & 0xffffu); v[3] = bf16_to_f32(raw.y >> 16);
    v[4] = bf16_to_f32(raw.z & 0xffffu); v[5] = bf16_to_f32(raw.z >> 16);
    v[6] = bf16_to_f32(raw.w & 0xffffu); v[7] = bf16_to_f32(raw.w >> 16);
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = wave_max_f32(amax, 16);
    const float s = e4m3_tile_scale(amax);
    scale = (uint8_t)e8m0_of(s);
    const float inv = 1.0f / s;  // a power of two: v * inv == v / s exactly
    const uint32_t lo = e4m3x4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
    const uint32_t hi = e4m3x4(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
    return make_uint2(lo, hi);
}

__global__ __launch_bounds__(256) void k_disp_gather_e4m3(int T, int d, const uint16_t *__restrict__ x,
                                                          const int32_t *__restrict__ row_of,
                                                          uint8_t *__restrict__ xq, uint8_t *__restrict__ xs) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    int32_t dst[kK];
#pragma unroll
    for (int j = 0; j < kK; ++j) dst[j] = row_of[(size_t)t * kK + j];
    const int ntile = d / 128;
    const uint4 *src = reinterpret_cast<const uint4 *>(x + (size_t)t * d);
    for (int c = lane; c < d / 8; c += 64) {  // d % 128 == 0: a tile's 16 lanes are all in or all out
        uint8_t s;
        const uint2 q = quant8(src[c], s);
#pragma unroll
        for (int j = 0; j < kK; ++j) {
            if (dst[j] < 0) continue;
            reinterpret_cast<uint2 *>(xq + (size_t)dst[j] * d)[c] = q;
            if ((lane & 15) == 0) xs[(size_t)dst[j] * ntile + c / 16] = s;
        }
    }
}

__global__ __launch_bounds__(256) void k_quant_rows_e4m3(int rows, int d, const uint16_t *__restrict__ x,
                                                         uint8_t *__restrict__ xq, uint8_t *__restrict__ xs) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= rows) return;
    const int ntile = d / 128;
    const uint4 *src = reinterpret_cast<const uint4 *>(x + (size_t)t * d);
    for (int c = lane; c < d / 8; c += 64) {
        uint8_t s;
        const uint2 q = quant8(src[c], s);
        reinterpret_cast<uint2 *>(xq + (size_t)t * d)[c] = q;
        if ((lane & 15) == 0) xs[(size_t)t * ntile + c / 16] = s;
    }
}

// Static scratch of the allocation-free dispatch: the per-block count
// table [ceil(T/256), E] int32 for up to kDispatchScratchTokens tokens
// (4 MiB), one copy per GPU, held until the process ends.  Every entry a
// call reads is written by that call's k_disp_count first, so nothing needs
// clearing between calls; calls that overlap on one GPU share it and race.
constexpr size_t kScratchInts = (size_t)(kDispatchScratchTokens / kDispatchBlock) * kE;
__device__ __align__(256) int32_t scratch[kScratchInts];

constexpr int kMaxDevices = 64;
// Device address of `scratch` on each GPU, looked up once per device with
// that device current (host code never passes the array's own name).
int32_t *g_scratch[kMaxDevices];

hipError_t scratch_ptr(int32_t **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    int32_t *p = __atomic_load_n(&g_scratch[dev], __ATOMIC_ACQUIRE);
    if (p == nullptr) {
        void *q = nullptr;
        e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (q == nullptr) return hipErrorInvalidSymbol;
        p = static_cast<int32_t *>(q);
        __atomic_store_n(&g_scratch[dev], p, __ATOMIC_RELEASE);
    }
    *out = p;
    return hipSuccess;
}

// One GEMM row per thread: its token's E8M0 tile scales, written per
// 128-block (each block's writes coalesced over consecutive rows).
__global__ __launch_bounds__(256) void k_gather_scales_km(int M, int nkb, int div, const int32_t *__restrict__ rows,
                                                          const uint8_t *__restrict__ scales,
                                                          uint8_t *__restrict__ out) {
    const int r = blockIdx.x * 256 + threadIdx.x;
    if (r >= M) return;
    const uint8_t *in = scales + (size_t)(rows ? rows[r] / div : r) * nkb;
    for (int kb = 0; kb < nkb; ++kb) out[(size_t)kb * M + r] = in[kb];
}

}  // namespace

hipError_t launch_gather_scales_kmajor(int M, int nkb, int div, const int32_t *rows, const uint8_t *scales,
                                       uint8_t *out, hipStream_t s) {
    hipLaunchKernelGGL(k_gather_scales_km, dim3((M + 255) / 256), dim3(256), 0, s, M, nkb, div, rows, scales, out);
    return hipGetLastError();
}

hipError_t launch_dispatch_noalloc(DispatchArgs a, hipStream_t s) {
    if (a.T > kDispatchScratchTokens) return hipErrorInvalidValue;  // the caller checks first
    hipError_t e = scratch_ptr(&a.block_base);
    if (e != hipSuccess) return e;
    return launch_dispatch(a, s);
}

hipError_t launch_dispatch(const DispatchArgs &a, hipStream_t s) {
    const int nblk = (a.T + kDispatchBlock - 1) / kDispatchBlock;
    hipLaunchKernelGGL(k_disp_count, dim3(nblk), dim3(kDispatchBlock), 0, s, a.T, a.idx, a.block_base);
    hipLaunchKernelGGL(k_disp_scan, dim3(1), dim3(kE), 0, s, nblk, a.block_base, a.counts, a.offsets);
    hipLaunchKernelGGL(k_disp_rank, dim3(nblk), dim3(kDispatchBlock), 0, s, a.T, a.idx, a.block_base,
                       a.row_src, a.row_of);
    if (a.x_perm == nullptr) return hipGetLastError();  // bookkeeping only: the GEMM gathers through row_src
    const dim3 ggrid((a.T + 3) / 4), gblock(256);
    if (a.wt == kE4M3) {
        hipLaunchKernelGGL(k_disp_gather_e4m3, ggrid, gblock, 0, s, a.T, a.d,
                           static_cast<const uint16_t *>(a.x), a.row_of, static_cast<uint8_t *>(a.x_perm),
                           a.x_perm_scale);
    } else {
        const int row_bytes = a.d * (a.act == kF32 ? 4 : 2);
        hipLaunchKernelGGL(k_disp_gather_copy, ggrid, gblock, 0, s, a.T, row_bytes,
                           static_cast<const uint8_t *>(a.x), a.row_of, static_cast<uint8_t *>(a.x_perm));
    }
    return hipGetLastError();
}

hipError_t launch_quant_rows_e4m3(int rows, int d, const uint16_t *x, uint8_t *q, uint8_t *scales, hipStream_t s) {
    hipLaunchKernelGGL(k_quant_rows_e4m3, dim3((rows + 3) / 4), dim3(256), 0, s, rows, d, x, q, scales);
    return hipGetLastError();
}

}  // namespace moe
