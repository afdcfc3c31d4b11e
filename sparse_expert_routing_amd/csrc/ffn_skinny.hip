// Grouped SwiGLU expert GEMMs for tiny groups (decode: a few rows per
// expert), bf16.
//
// Routed experts: DeepSeek V3 From Scratch, "The idea" (each token to its
// top 8 of many small experts); Scaling Efficiency: A Deep Dive into the
// DeepSeek-V3 Architecture, "Implementation: A Modular Look" (each expert
// runs on the tokens that chose it).
//
// With ~2 rows per expert the GEMMs are a stream of the touched experts'
// weights: every weight byte is used by a handful of rows once, so the design
// goal is HBM bandwidth, not MFMA rate.
//   - one workgroup = (expert, 64 h columns) for gate/up (B = its 64 gate and
//     64 up rows) or (expert, 128 output columns) for down: 128 B rows;
//   - the 4 waves split K in four; each streams its quarter of the 128 B rows
//     from HBM straight into registers (no LDS: every B element is used by
//     one wave only), two 64-wide K chunks in flight per wave (16 KB each);
//   - v_mfma_f32_16x16x32_bf16 on 16-row passes over the group (rows past
//     the group's end repeat a valid row and are not stored); a lane's 16-byte pieces sit at the same K
//     positions in its A and B operands, so any assignment of K to lanes is a
//     valid product as long as both operands use it;
//   - the four K quarters are added through LDS in wave order, then the
//     SwiGLU (gate/up, h rounded to bf16) or the bf16 store (down);
//   - groups of more than 16 rows loop over 16-row passes (each pass streams
//     the B tile again; the host uses this path only when groups average at
//     most 4 rows).
#include "device.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kE = 256;
constexpr int SB = 128;   // B rows per workgroup
constexpr int SKC = 64;   // K per chunk
constexpr int kWaves = 4;

struct SkinnyParams {
    const int32_t *offsets;   // [E+1]
    const uint16_t *A;        // rows of the group's input
    const int32_t *a_rows;    // optional: GEMM row r reads row a_rows[r] / a_div of A
    int a_div;
    int K;
    const uint16_t *B0, *B1;  // [E, N, K] (gate, up) or (down, unused)
    int N;                    // B rows per expert (I for gate/up, d for down)
    uint16_t *out;            // [rows, N_out] bf16 (h or y_perm)
};

// One chunk of B for this lane: 8 column blocks x 2 pieces of 16 bytes.
struct BChunk {
    i32x4 v[8][2];
};

struct AChunk {
    i32x4 v[2];
};

// Lane l of a 16 x 64 block (rows or B rows 16 wide, 64 of K) holds row l & 15
// and the K pieces 8 * (l >> 4) .. +7 and 32 + 8 * (l >> 4) .. +7: piece p of
// the lane feeds the MFMA of K half p.
__device__ __forceinline__ uint32_t piece_off(int lane, int p) { return (uint32_t)(p * 32 + 8 * (lane >> 4)); }

// B row of lane l in column block j: brow0 + j * jstride (elements).
__device__ __forceinline__ void k_loop(const uint16_t *__restrict__ brow0, size_t jstride,
                                       const uint16_t *__restrict__ brow4, const uint16_t *__restrict__ arow,
                                       int k0, int nch, f32x4 (&acc)[8]) {
    const int lane = threadIdx.x & 63;
    auto load_b = [&](BChunk &c, int kc) {
        const int kk = k0 + kc * SKC;
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int q = 0; q < 2; ++q)
                c.v[j][q] = *reinterpret_cast<const i32x4 *>(
                    (j < 4 ? brow0 + j * jstride : brow4 + (j - 4) * jstride) + kk + piece_off(lane, q));
    };
    auto load_a = [&](AChunk &c, int kc) {
        const int kk = k0 + kc * SKC;
#pragma unroll
        for (int q = 0; q < 2; ++q) c.v[q] = *reinterpret_cast<const i32x4 *>(arow + kk + piece_off(lane, q));
    };
    auto mma = [&](const BChunk &b, const AChunk &a) {
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a.v[q]),
                                                                 __builtin_bit_cast(bf16x8, b.v[j][q]), acc[j], 0, 0, 0);
    };
    // two chunks in flight: (b0, a0) and (b1, a1) alternate; nch is even.
    // Scheduling barriers keep each chunk's loads ahead of the MFMAs on the
    // previous chunk (left free, the scheduler sinks them and the wave ends
    // up waiting with one chunk in flight).
    BChunk b0, b1;
    AChunk a0, a1;
    load_b(b0, 0);
    load_a(a0, 0);
    for (int kc = 0; kc + 2 < nch; kc += 2) {
        load_b(b1, kc + 1);
        load_a(a1, kc + 1);
        __builtin_amdgcn_sched_barrier(0);
        mma(b0, a0);
        __builtin_amdgcn_sched_barrier(0);
        load_b(b0, kc + 2);
        load_a(a0, kc + 2);
        __builtin_amdgcn_sched_barrier(0);
        mma(b1, a1);
        __builtin_amdgcn_sched_barrier(0);
    }
    load_b(b1, nch - 1);
    load_a(a1, nch - 1);
    __builtin_amdgcn_sched_barrier(0);
    mma(b0, a0);
    __builtin_amdgcn_sched_barrier(0);
    mma(b1, a1);
}

template <bool DUAL>
__global__ __launch_bounds__(256, 2) void k_gemm_skinny(SkinnyParams p) {
    constexpr int OUTC = DUAL ? SB / 2 : SB;  // output columns per workgroup
    __shared__ float red[kWaves][16][SB + 4];

    const int e = blockIdx.y;
    const int g0 = p.offsets[e], cnt = p.offsets[e + 1] - g0;
    if (cnt <= 0) return;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n_out = p.N;               // output row width: I for h, d for y_perm
    const int c0 = blockIdx.x * OUTC;    // first output column

    // B rows of this lane: column block j (16 B rows) is row c0 + 16 j of
    // the down matrix, or for gate/up row c0 + 16 (j & 3) of the gate (j < 4)
    // or up matrix
    const size_t eoff = (size_t)e * p.N * p.K, jstride = (size_t)16 * p.K;
    const uint16_t *brow0 = p.B0 + eoff + (size_t)(c0 + (lane & 15)) * p.K;
    const uint16_t *brow4 = DUAL ? p.B1 + eoff + (size_t)(c0 + (lane & 15)) * p.K : brow0 + 4 * jstride;
    const int kq = p.K / kWaves;            // this wave's K range
    const int k0 = wave * kq, nch = kq / SKC;

    for (int r0 = 0; r0 < cnt; r0 += 16) {
        const int rows = min(16, cnt - r0);
        f32x4 acc[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        // rows past the group's end repeat its first row of this pass: an
        // output row depends on its own A row only, and those rows are not
        // stored
        const int lr = r0 + (lane & 15);
        int src = g0 + (lr < cnt ? lr : r0);
        if (p.a_rows) src = p.a_rows[src] / p.a_div;
        k_loop(brow0, jstride, brow4, p.A + (size_t)src * p.K, k0, nch, acc);

        // this wave's K-quarter sums -> LDS (16x16 block: lane holds column
        // lane & 15 and rows 4 * (lane >> 4) .. +3)
        if (r0 > 0) __syncthreads();  // the previous pass's readers are done
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) red[wave][4 * (lane >> 4) + i][16 * j + (lane & 15)] = acc[j][i];
        __syncthreads();
        // add the quarters in wave order; epilogue
        if (DUAL) {
            // 16 rows x 64 h columns: thread -> row tid / 16, columns 4 * (tid % 16) .. +3
            const int row = tid >> 4, cc = 4 * (tid & 15);
            if (row < rows) {
                uint32_t packed[2];
#pragma unroll
                for (int u = 0; u < 4; u += 2) {
                    float h2[2];
#pragma unroll
                    for (int v = 0; v < 2; ++v) {
                        const int c = cc + u + v;
                        float gs = red[0][row][c], us = red[0][row][64 + c];
#pragma unroll
                        for (int w = 1; w < kWaves; ++w) {
                            gs += red[w][row][c];
                            us += red[w][row][64 + c];
                        }
                        h2[v] = gs / (1.0f + expf(-gs)) * us;
                    }
                    packed[u / 2] = pack_bf16x2(h2[0], h2[1]);
                }
                *reinterpret_cast<uint2 *>(p.out + (size_t)(g0 + r0 + row) * n_out + c0 + cc) =
                    uint2{packed[0], packed[1]};
            }
        } else {
            // 16 rows x 128 columns: thread -> row tid / 16, columns 8 * (tid % 16) .. +7
            const int row = tid >> 4, cc = 8 * (tid & 15);
            if (row < rows) {
                uint32_t packed[4];
#pragma unroll
                for (int u = 0; u < 8; u += 2) {
                    float y2[2];
#pragma unroll
                    for (int v = 0; v < 2; ++v) {
                        const int c = cc + u + v;
                        float s = red[0][row][c];
#pragma unroll
                        for (int w = 1; w < kWaves; ++w) s += red[w][row][c];
                        y2[v] = s;
                    }
                    packed[u / 2] = pack_bf16x2(y2[0], y2[1]);
                }
                uint16_t *o = p.out + (size_t)(g0 + r0 + row) * n_out + c0 + cc;
                *reinterpret_cast<i32x4 *>(o) = i32x4{(int)packed[0], (int)packed[1], (int)packed[2], (int)packed[3]};
            }
        }
    }
}

}  // namespace

bool ffn_skinny_ok(const FfnArgs &a) {
    return a.offsets != nullptr && a.wt == kBF16 && a.E == kE && (long long)a.M <= 4LL * a.E &&
           a.d % (2 * kWaves * SKC) == 0 && a.I % (2 * kWaves * SKC) == 0 && a.I % (SB / 2) == 0 && a.d % SB == 0;
}

hipError_t launch_ffn_skinny(const FfnArgs &a, hipStream_t s) {
    if (a.phases & 1) {
        SkinnyParams p{};
        p.offsets = a.offsets;
        p.A = static_cast<const uint16_t *>(a.a);
        p.a_rows = a.a_rows;
        p.a_div = a.a_rows ? a.a_div : 1;
        p.K = a.d;
        p.B0 = static_cast<const uint16_t *>(a.w.gate);
        p.B1 = static_cast<const uint16_t *>(a.w.up);
        p.N = a.I;
        p.out = static_cast<uint16_t *>(a.h);
        hipLaunchKernelGGL(k_gemm_skinny<true>, dim3(a.I / (SB / 2), a.E), dim3(256), 0, s, p);
    }
    if (a.phases & 2) {
        SkinnyParams q{};
        q.offsets = a.offsets;
        q.A = static_cast<const uint16_t *>(a.h);
        q.a_div = 1;
        q.K = a.I;
        q.B0 = static_cast<const uint16_t *>(a.w.down);
        q.B1 = nullptr;
        q.N = a.d;
        q.out = static_cast<uint16_t *>(a.y);
        hipLaunchKernelGGL(k_gemm_skinny<false>, dim3(a.d / SB, a.E), dim3(256), 0, s, q);
    }
    return hipGetLastError();
}

}  // namespace moe
