// Grouped SwiGLU expert FFN: gate/up GEMM with a SwiGLU epilogue, down GEMM
// with a store or a combine epilogue.
//
// Routed experts: DeepSeek V3 From Scratch, "The idea" (many small routed
// experts, each token to its top 8); Scaling Efficiency: A Deep Dive into the
// DeepSeek-V3 Architecture, "Implementation: A Modular Look" (each expert runs
// on the tokens that chose it; shared output plus weighted routed outputs).
// Gated (SwiGLU) expert form: our reading, see the C ABI header.
//
// bf16 path (the dense contraction of the layer):
//   - v_mfma_f32_32x32x16_bf16, 4 waves per workgroup in a 2x2 layout,
//     workgroup tile 128 rows x 128 B-rows x 64 K, double-buffered in LDS with
//     an XOR swizzle of the 16-byte K chunks;
//   - gate/up: the B tile holds 64 gate rows and the matching 64 up rows, so
//     the epilogue forms h = silu(g) * u in registers (fp32) and stores bf16;
//   - down: plain bf16 store into y_perm, or (shared expert) the combine
//     y = acc + sum_j w_j * y_perm[row_of[t*k + j]] in fp32;
//   - tile -> (expert, first row) is computed on the device from `offsets`
//     (no host synchronisation); slots past the last tile exit at once;
//   - shared expert at small T (few row tiles): K is split over blockIdx.z
//     so about 256 workgroups stream the weights; each split stores fp32
//     partial sums and a second pass adds them in split order and applies
//     the SwiGLU (gate/up) or the combine (down).
// fp32 path: one thread per output, plain FMA loops (tiny fp32 layer only).
#include "device.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kE = 256;
constexpr int BM = 128;  // rows per workgroup tile
constexpr int BNB = 128; // B rows per workgroup tile
constexpr int BK = 64;   // K per stage

enum { EPI_SWIGLU = 0, EPI_STORE = 1, EPI_COMBINE = 2, EPI_PART_DUAL = 3, EPI_PART = 4 };

struct GemmParams {
    int M;                    // rows when offsets == nullptr
    const int32_t *offsets;   // [E+1] or nullptr
    const uint16_t *A;        // [rows, K]
    const int32_t *a_rows;    // optional row indirection into A: row a_rows[r] / a_div
    int a_div;
    int K;
    const uint16_t *B0, *B1;  // [G, N, K]: gate/up (dual) or down
    int N;                    // output columns (I for gate/up, d for down)
    uint16_t *out;            // bf16 [rows, N] (h or y_perm)
    float *yout;              // f32 [rows, N] (combine)
    const uint16_t *y_perm;   // [rows*k, N] (combine)
    const int32_t *row_of;    // [rows*k]
    const float *cw;          // [rows*k]
    int k;
    float *part;              // split K: fp32 partials [gridDim.z, rows, N] (x2 columns for gate/up)
};

// Map a row-tile slot to (expert, first row, end row).  All lanes of all waves
// compute the same answer, so the early exit is uniform over the workgroup.
__device__ __forceinline__ bool find_tile(const int32_t *__restrict__ offsets, int M, int slot, int &e,
                                          int &m0, int &m_end) {
    if (offsets == nullptr) {
        e = 0;
        m0 = slot * BM;
        m_end = M;
        return m0 < M;
    }
    const int lane = threadIdx.x & 63;
    const int base = lane * 4;
    int off[5];
#pragma unroll
    for (int i = 0; i < 5; ++i) off[i] = offsets[base + i];
    int nt[4], lane_t = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        nt[i] = (off[i + 1] - off[i] + BM - 1) / BM;
        lane_t += nt[i];
    }
    const int incl = wave_incl_scan(lane_t);
    const int excl = incl - lane_t;
    const int total = __shfl(incl, 63, 64);
    if (slot >= total) return false;
    const bool own = slot >= excl && slot < incl;
    const uint64_t bal = __ballot(own);
    const int owner = __ffsll((unsigned long long)bal) - 1;
    int my_e = 0, my_m0 = 0, my_end = 0;
    if (own) {
        int s = slot - excl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (s >= 0 && s < nt[i]) {
                my_e = base + i;
                my_m0 = off[i] + s * BM;
                my_end = off[i + 1];
            }
            s -= nt[i];
        }
    }
    e = __shfl(my_e, owner, 64);
    m0 = __shfl(my_m0, owner, 64);
    m_end = __shfl(my_end, owner, 64);
    return true;
}

__device__ __forceinline__ int swz(int row, int c16) { return c16 ^ (row & 7); }

template <int EPI>
__global__ __launch_bounds__(256) void k_gemm_bf16(GemmParams p) {
    constexpr bool DUAL = EPI == EPI_SWIGLU || EPI == EPI_PART_DUAL;
    constexpr int BN = DUAL ? BNB / 2 : BNB;      // output columns per workgroup
    constexpr int NT = DUAL ? 2 : 2;              // 32-wide B fragments per wave
    __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM * BK];
    __shared__ __attribute__((aligned(16))) uint16_t sB[2][BNB * BK];

    int e, m0, m_end;
    if (!find_tile(p.offsets, p.M, blockIdx.x, e, m0, m_end)) return;
    const int n0 = blockIdx.y * BN;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int K = p.K;
    // K range of this split (the whole K when gridDim.z == 1)
    const int nk_all = K / BK, z = blockIdx.z;
    const int kb0 = nk_all * z / (int)gridDim.z;
    const int nk = nk_all * (z + 1) / (int)gridDim.z - kb0;
    const int kbase = kb0 * BK;

    // global -> register staging: 4 chunks of 16 bytes per thread per operand.
    // Chunk i covers row tid/8 + 32*i and K columns (tid%8)*8 .. +8; for the
    // dual (gate/up) B tile, chunks 0-1 are gate rows and 2-3 the up rows.
    const int c16 = tid & 7;
    const uint16_t *Bg = p.B0 + (size_t)e * p.N * K;
    const uint16_t *Bu = DUAL ? p.B1 + (size_t)e * p.N * K : Bg;
    size_t aoff[4];  // A element offsets (the A operand can pass 2^32 elements: x_perm, h)
    uint32_t boff[4];
    int soff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = (tid >> 3) + 32 * i;
        int ar = m0 + row;
        ar = ar < m_end ? ar : m_end - 1;
        if (p.a_rows) ar = p.a_rows[ar] / p.a_div;
        aoff[i] = (size_t)ar * (size_t)K + c16 * 8;
        const int br = DUAL ? n0 + (row & 63) : n0 + row;
        boff[i] = (uint32_t)br * (uint32_t)K + c16 * 8;
        soff[i] = row * BK + swz(row, c16) * 8;
    }
    const uint16_t *Ab = p.A;

    f32x16 acc[2][NT];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    uint4 ra0, ra1, ra2, ra3, rb0, rb1, rb2, rb3;
    const uint16_t *Bu2 = DUAL ? Bu : Bg;  // B matrix of chunks 2 and 3

    for (int kt = -1; kt < nk; ++kt) {
        // stage kt+1: global -> registers (issued before the MFMAs of stage kt)
        if (kt + 1 < nk) {
            const int k0 = kbase + (kt + 1) * BK;
            ra0 = *reinterpret_cast<const uint4 *>(Ab + aoff[0] + k0);
            ra1 = *reinterpret_cast<const uint4 *>(Ab + aoff[1] + k0);
            ra2 = *reinterpret_cast<const uint4 *>(Ab + aoff[2] + k0);
            ra3 = *reinterpret_cast<const uint4 *>(Ab + aoff[3] + k0);
            rb0 = *reinterpret_cast<const uint4 *>(Bg + boff[0] + k0);
            rb1 = *reinterpret_cast<const uint4 *>(Bg + boff[1] + k0);
            rb2 = *reinterpret_cast<const uint4 *>(Bu2 + boff[2] + k0);
            rb3 = *reinterpret_cast<const uint4 *>(Bu2 + boff[3] + k0);
        }
        if (kt >= 0) {
            const int buf = kt & 1;
#pragma unroll
            for (int kk = 0; kk < BK; kk += 16) {
                const int kc = kk / 8 + (lane >> 5);
                bf16x8 af[2], bfr[NT];
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int row = wm * 64 + i * 32 + (lane & 31);
                    af[i] = *reinterpret_cast<const bf16x8 *>(&sA[buf][row * BK + swz(row, kc) * 8]);
                }
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    const int row = DUAL ? (j * 64 + wn * 32 + (lane & 31)) : (wn * 64 + j * 32 + (lane & 31));
                    bfr[j] = *reinterpret_cast<const bf16x8 *>(&sB[buf][row * BK + swz(row, kc) * 8]);
                }
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < NT; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
            }
        }
        // registers -> the other LDS buffer (its readers finished at the last barrier)
        if (kt + 1 < nk) {
            const int nb = (kt + 1) & 1;
            *reinterpret_cast<uint4 *>(&sA[nb][soff[0]]) = ra0;
            *reinterpret_cast<uint4 *>(&sA[nb][soff[1]]) = ra1;
            *reinterpret_cast<uint4 *>(&sA[nb][soff[2]]) = ra2;
            *reinterpret_cast<uint4 *>(&sA[nb][soff[3]]) = ra3;
            *reinterpret_cast<uint4 *>(&sB[nb][soff[0]]) = rb0;
            *reinterpret_cast<uint4 *>(&sB[nb][soff[1]]) = rb1;
            *reinterpret_cast<uint4 *>(&sB[nb][soff[2]]) = rb2;
            *reinterpret_cast<uint4 *>(&sB[nb][soff[3]]) = rb3;
        }
        __syncthreads();
    }

    // Epilogue.  32x32 C layout: lane holds column (lane & 31) and rows
    // 8*q + 4*(lane >> 5) + r for acc index 4*q + r.
    const int N = p.N;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = m0 + wm * 64 + i * 32 + 8 * q + 4 * (lane >> 5) + r;
                if (row >= m_end) continue;
                if (EPI == EPI_PART_DUAL) {
                    const int col = n0 + wn * 32 + (lane & 31);
                    float *pr = p.part + ((size_t)z * p.M + row) * (2 * N);
                    pr[col] = acc[i][0][4 * q + r];
                    pr[N + col] = acc[i][1][4 * q + r];
                } else if (DUAL) {
                    const int col = n0 + wn * 32 + (lane & 31);
                    const float g = acc[i][0][4 * q + r], u = acc[i][1][4 * q + r];
                    const float h = g / (1.0f + expf(-g)) * u;
                    p.out[(size_t)row * N + col] = (uint16_t)f32_to_bf16(h);
                } else {
#pragma unroll
                    for (int j = 0; j < NT; ++j) {
                        const int col = n0 + wn * 64 + j * 32 + (lane & 31);
                        const float v = acc[i][j][4 * q + r];
                        if (EPI == EPI_STORE) {
                            p.out[(size_t)row * N + col] = (uint16_t)f32_to_bf16(v);
                        } else if (EPI == EPI_PART) {
                            p.part[((size_t)z * p.M + row) * N + col] = v;
                        } else {
                            float y = v;
                            for (int jj = 0; jj < p.k; ++jj) {
                                const size_t f = (size_t)row * p.k + jj;
                                y += p.cw[f] * bf16_to_f32(p.y_perm[(size_t)p.row_of[f] * N + col]);
                            }
                            p.yout[(size_t)row * N + col] = y;
                        }
                    }
                }
            }
    }
}

// Split-K second passes, 4 columns per thread.
// h[r, c] = bf16(silu(g) * u), g and u the split partials added in split order.
__global__ __launch_bounds__(256) void k_split_swiglu(int M, int I, int S, const float *__restrict__ part,
                                                      uint16_t *__restrict__ h) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    const int w4 = I / 4;
    if (i >= M * w4) return;
    const int row = i / w4, c = (i - row * w4) * 4;
    const size_t zs = (size_t)M * 2 * I;
    const float *pg = part + (size_t)row * 2 * I + c;
    float4 g = *reinterpret_cast<const float4 *>(pg), u = *reinterpret_cast<const float4 *>(pg + I);
    for (int z = 1; z < S; ++z) {
        const float4 gz = *reinterpret_cast<const float4 *>(pg + z * zs);
        const float4 uz = *reinterpret_cast<const float4 *>(pg + z * zs + I);
        g.x += gz.x; g.y += gz.y; g.z += gz.z; g.w += gz.w;
        u.x += uz.x; u.y += uz.y; u.z += uz.z; u.w += uz.w;
    }
    const float hx = g.x / (1.0f + expf(-g.x)) * u.x, hy = g.y / (1.0f + expf(-g.y)) * u.y;
    const float hz = g.z / (1.0f + expf(-g.z)) * u.z, hw = g.w / (1.0f + expf(-g.w)) * u.w;
    uint2 o;
    o.x = f32_to_bf16(hx) | (f32_to_bf16(hy) << 16);
    o.y = f32_to_bf16(hz) | (f32_to_bf16(hw) << 16);
    *reinterpret_cast<uint2 *>(h + (size_t)row * I + c) = o;
}

// y[t, n] = (sum over splits of the shared down GEMM) + sum_j cw[t*k+j] * y_perm[row_of[t*k+j], n]
__global__ __launch_bounds__(256) void k_split_combine(int M, int d, int S, int k, const float *__restrict__ part,
                                                       const uint16_t *__restrict__ y_perm,
                                                       const int32_t *__restrict__ row_of,
                                                       const float *__restrict__ cw, float *__restrict__ y) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    const int w4 = d / 4;
    if (i >= M * w4) return;
    const int row = i / w4, c = (i - row * w4) * 4;
    const size_t zs = (size_t)M * d;
    const float *pp = part + (size_t)row * d + c;
    float4 v = *reinterpret_cast<const float4 *>(pp);
    for (int z = 1; z < S; ++z) {
        const float4 vz = *reinterpret_cast<const float4 *>(pp + z * zs);
        v.x += vz.x; v.y += vz.y; v.z += vz.z; v.w += vz.w;
    }
    for (int j = 0; j < k; ++j) {
        const size_t f = (size_t)row * k + j;
        const float w = cw[f];
        const uint2 b = *reinterpret_cast<const uint2 *>(y_perm + (size_t)row_of[f] * d + c);
        v.x += w * bf16_to_f32(b.x & 0xffffu);
        v.y += w * bf16_to_f32(b.x >> 16);
        v.z += w * bf16_to_f32(b.y & 0xffffu);
        v.w += w * bf16_to_f32(b.y >> 16);
    }
    *reinterpret_cast<float4 *>(y + (size_t)row * d + c) = v;
}

// Number of K splits for a GEMM of `tiles` workgroup tiles over nk K steps:
// about 256 workgroups, each split keeping at least 4 K steps.
int ksplits(int tiles, int nk) {
    const int cap = nk / 4;
    const int s = 256 / tiles;
    return s > cap ? (cap < 1 ? 1 : cap) : (s < 1 ? 1 : s);
}

// ---------------------------------------------------------------- fp32 path

__device__ __forceinline__ int expert_of_row(const int32_t *__restrict__ offsets, int row) {
    int lo = 0, hi = kE;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (offsets[mid] <= row) lo = mid; else hi = mid;
    }
    return lo;
}

// h[row, n] = silu(a_row . Wg[e, n]) * (a_row . Wu[e, n])
__global__ __launch_bounds__(256) void k_f32_gateup(int M, int d, int I, const int32_t *__restrict__ offsets,
                                                    const float *__restrict__ a, const int32_t *__restrict__ a_rows,
                                                    int a_div, const float *__restrict__ wg,
                                                    const float *__restrict__ wu, float *__restrict__ h) {
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int n = blockIdx.y * 64 + (threadIdx.x & 63);
    if (row >= M || n >= I) return;
    const int e = offsets ? expert_of_row(offsets, row) : 0;
    const float *x = a + (size_t)(a_rows ? a_rows[row] / a_div : row) * d;
    const float *g = wg + ((size_t)e * I + n) * d;
    const float *u = wu + ((size_t)e * I + n) * d;
    float sg = 0.f, su = 0.f;
    for (int j = 0; j < d; ++j) {
        sg += x[j] * g[j];
        su += x[j] * u[j];
    }
    h[(size_t)row * I + n] = sg / (1.0f + expf(-sg)) * su;
}

// y[row, n] = h_row . Wd[e, n]  (+ combine for the shared expert)
__global__ __launch_bounds__(256) void k_f32_down(int M, int d, int I, const int32_t *__restrict__ offsets,
                                                  const float *__restrict__ h, const float *__restrict__ wd,
                                                  float *__restrict__ y, int k, const float *__restrict__ y_perm,
                                                  const int32_t *__restrict__ row_of, const float *__restrict__ cw) {
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int n = blockIdx.y * 64 + (threadIdx.x & 63);
    if (row >= M || n >= d) return;
    const int e = offsets ? expert_of_row(offsets, row) : 0;
    const float *hr = h + (size_t)row * I;
    const float *w = wd + ((size_t)e * d + n) * I;
    float acc = 0.f;
    for (int i = 0; i < I; ++i) acc += hr[i] * w[i];
    if (y_perm != nullptr) {
        for (int j = 0; j < k; ++j) {
            const size_t f = (size_t)row * k + j;
            acc += cw[f] * y_perm[(size_t)row_of[f] * d + n];
        }
    }
    y[(size_t)row * d + n] = acc;
}

}  // namespace

// fp32 partial-sum bytes the shared expert's split-K passes need (0 when
// T is large enough not to split, or for other weight types).
size_t ffn_shared_split_bytes(int M, int d, int I, int wt) {
    if (wt != kBF16 || d % BK || I % BK) return 0;
    const int mt = (M + BM - 1) / BM;
    const int s_gu = ksplits(mt * (I / (BNB / 2)), d / BK), s_dn = ksplits(mt * (d / BNB), I / BK);
    const size_t gu = s_gu > 1 ? (size_t)s_gu * M * 2 * I * sizeof(float) : 0;
    const size_t dn = s_dn > 1 ? (size_t)s_dn * M * d * sizeof(float) : 0;
    return gu > dn ? gu : dn;
}

// Routed groups averaging 64 to 127 rows (a mid-size batch: T = 2048 tokens
// over 256 experts) also go to the persistent large-tile kernels, whose
// five-unit LDS ring keeps more of each expert's weight stream in flight than
// this file's double-buffered 128 x 128 tiles: at T=2048, d=2048, I=512 the
// routed gate/up took 0.224 ms against 0.250-0.254 and the down 0.138
// against 0.154-0.158 (one GPU, alternating runs).  The large kernels'
// own shape checks are applied at twice the rows: that meets their
// 128-rows-per-group floor exactly when the groups average 64, and their
// 32-bit offset bounds only get stricter.
static bool routed_mid_large_ok(const FfnArgs &a) {
    if (a.offsets == nullptr || a.M > (1 << 29) || (long long)a.M < 64LL * a.E) return false;
    FfnArgs b = a;
    b.M = 2 * a.M;
    return ffn_bf16_large_ok(b);
}

hipError_t launch_ffn(const FfnArgs &a, hipStream_t s) {
    const bool routed = a.offsets != nullptr;
    if (a.wt == kF32) {
        dim3 g1((a.M + 3) / 4, (a.I + 63) / 64), g2((a.M + 3) / 4, (a.d + 63) / 64);
        if (a.phases & 1)
            hipLaunchKernelGGL(k_f32_gateup, g1, dim3(256), 0, s, a.M, a.d, a.I, a.offsets,
                               static_cast<const float *>(a.a), a.a_rows, a.a_div, static_cast<const float *>(a.w.gate),
                               static_cast<const float *>(a.w.up), static_cast<float *>(a.h));
        if (a.phases & 2)
            hipLaunchKernelGGL(k_f32_down, g2, dim3(256), 0, s, a.M, a.d, a.I, a.offsets,
                               static_cast<const float *>(a.h), static_cast<const float *>(a.w.down),
                               static_cast<float *>(a.y), a.k,
                               a.combine ? static_cast<const float *>(a.y_perm) : nullptr, a.row_of, a.cw);
        return hipGetLastError();
    }
    if (a.wt == kBF16) {
        if (ffn_skinny_ok(a)) return launch_ffn_skinny(a, s);
        if (ffn_bf16_large_ok(a) || routed_mid_large_ok(a)) return launch_ffn_bf16_large(a, s);
        const int slots = (a.M + BM - 1) / BM + (routed ? kE : 0);
        GemmParams p{};
        p.M = a.M;
        p.offsets = a.offsets;
        p.A = static_cast<const uint16_t *>(a.a);
        p.a_rows = a.a_rows;
        p.a_div = a.a_div;
        p.K = a.d;
        p.B0 = static_cast<const uint16_t *>(a.w.gate);
        p.B1 = static_cast<const uint16_t *>(a.w.up);
        p.N = a.I;
        p.out = static_cast<uint16_t *>(a.h);
        const int mt = (a.M + BM - 1) / BM;
        const int s_gu = routed || !a.part ? 1 : ksplits(mt * (a.I / (BNB / 2)), a.d / BK);
        const int s_dn = routed || !a.part ? 1 : ksplits(mt * (a.d / BNB), a.I / BK);
        if ((a.phases & 1) && s_gu > 1) {
            p.part = a.part;
            hipLaunchKernelGGL(k_gemm_bf16<EPI_PART_DUAL>, dim3(slots, a.I / (BNB / 2), s_gu), dim3(256), 0, s, p);
            hipLaunchKernelGGL(k_split_swiglu, dim3((a.M * (a.I / 4) + 255) / 256), dim3(256), 0, s, a.M, a.I, s_gu,
                               a.part, static_cast<uint16_t *>(a.h));
        } else if (a.phases & 1) {
            hipLaunchKernelGGL(k_gemm_bf16<EPI_SWIGLU>, dim3(slots, a.I / (BNB / 2)), dim3(256), 0, s, p);
        }
        if (!(a.phases & 2)) return hipGetLastError();
        GemmParams q{};
        q.M = a.M;
        q.offsets = a.offsets;
        q.A = static_cast<const uint16_t *>(a.h);
        q.K = a.I;
        q.B0 = static_cast<const uint16_t *>(a.w.down);
        q.N = a.d;
        if (a.combine && s_dn > 1) {
            q.part = a.part;
            hipLaunchKernelGGL(k_gemm_bf16<EPI_PART>, dim3(slots, a.d / BNB, s_dn), dim3(256), 0, s, q);
            hipLaunchKernelGGL(k_split_combine, dim3((a.M * (a.d / 4) + 255) / 256), dim3(256), 0, s, a.M, a.d, s_dn,
                               a.k, a.part, static_cast<const uint16_t *>(a.y_perm), a.row_of, a.cw,
                               static_cast<float *>(a.y));
        } else if (a.combine) {
            q.yout = static_cast<float *>(a.y);
            q.y_perm = static_cast<const uint16_t *>(a.y_perm);
            q.row_of = a.row_of;
            q.cw = a.cw;
            q.k = a.k;
            hipLaunchKernelGGL(k_gemm_bf16<EPI_COMBINE>, dim3(slots, a.d / BNB), dim3(256), 0, s, q);
        } else {
            q.out = static_cast<uint16_t *>(a.y);
            hipLaunchKernelGGL(k_gemm_bf16<EPI_STORE>, dim3(slots, a.d / BNB), dim3(256), 0, s, q);
        }
        return hipGetLastError();
    }
    return launch_ffn_fp8(a, s);
}

}  // namespace moe
