// Grouped SwiGLU expert FFN in OCP fp8 e4m3 with fine-grained scales.
//
// crackai.dev DeepSeek-V3 summary, "How It Works": FP8 matmuls with a scale
// per tile and FP32 accumulation at chosen points; DeepSeek V3 From Scratch,
// "The idea": fine-grained quantisation tiles.  Tile shapes (ours): one E8M0
// scale byte per 1x128 activation tile (x_perm rows, h rows) and per 128x128
// weight block.
//
// Each 128-wide K block is one stage: the wave multiplies its e4m3 fragments
// with v_mfma_scale_f32_32x32x64_f8f6f4 (two per block) straight into the fp32
// accumulator, the E8M0 scales s_a[row, kb] and s_w[nb, kb] applied by the
// MFMA.
// Workgroup tile 128 rows x 128 output columns (gate/up: 128 gate + 128 up
// B rows), 4 waves in a 2x2 layout, LDS double-buffered with an XOR swizzle
// of the 16-byte K chunks.
// gate/up epilogue: h = silu(g) * u in fp32, then quantised per 1x128 tile of
// h: the row amax over the workgroup's 128 columns is combined across the two
// column waves through LDS; scale = the power of two at or above amax / 448,
// code = e4m3(h / scale).
// down epilogue: bf16 store of y_perm, or (shared expert) the fp32 combine.
#include "device.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kE = 256;
constexpr int BM = 128;   // rows per workgroup
constexpr int BN = 128;   // output columns per workgroup
constexpr int BK = 128;   // K bytes per stage = one scale block

enum { EPI_SWIGLU_Q = 0, EPI_STORE = 1, EPI_COMBINE = 2 };

struct Fp8Params {
    int M;
    const int32_t *offsets;
    const uint8_t *A;        // [rows, K] codes
    const uint8_t *As;       // [rows, K/128] E8M0
    const int32_t *a_rows;   // optional row indirection into A / As: row a_rows[r] / a_div
    int a_div;
    int K;
    const uint8_t *B0, *B1;  // [G, N, K] codes
    const uint8_t *S0, *S1;  // [G, N/128, K/128] E8M0
    int N;
    uint8_t *hq;             // EPI_SWIGLU_Q: [rows, N] codes
    uint8_t *hs;             // EPI_SWIGLU_Q: [rows, N/128] E8M0
    uint16_t *out;           // EPI_STORE: bf16 [rows, N]
    float *yout;             // EPI_COMBINE: f32 [rows, N]
    const uint16_t *y_perm;
    const int32_t *row_of;
    const float *cw;
    int k;
};

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

// 32 K-bytes of one operand row for v_mfma_scale_f32_32x32x64_f8f6f4: K half `hf`
// of the 128-byte row, lane group g = lane / 32 takes bytes 64*hf + 32*g.
__device__ __forceinline__ i32x8 frag(const uint8_t *tile, int row, int hf, int g) {
    const int c0 = 4 * hf + 2 * g;
    const i32x4 lo = *reinterpret_cast<const i32x4 *>(tile + row * BK + swz(row, c0) * 16);
    const i32x4 hi = *reinterpret_cast<const i32x4 *>(tile + row * BK + swz(row, c0 + 1) * 16);
    return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

template <int EPI>
__global__ __launch_bounds__(256) void k_gemm_fp8(Fp8Params p) {
    constexpr bool DUAL = EPI == EPI_SWIGLU_Q;
    constexpr int BROWS = DUAL ? 2 * BN : BN;  // B rows per stage
    constexpr int NJ = DUAL ? 4 : 2;           // 32-wide B fragments per wave (gate 0-1, up 2-3)
    constexpr int BCH = BROWS * 8 / 256;       // 16-byte B chunks per thread per stage
    __shared__ __attribute__((aligned(16))) uint8_t sA[2][BM * BK];
    __shared__ __attribute__((aligned(16))) uint8_t sB[2][BROWS * BK];
    __shared__ int sAs[2][BM];  // E8M0 bytes

    int e, m0, m_end;
    if (!find_tile(p.offsets, p.M, blockIdx.x, e, m0, m_end)) return;
    const int n0 = blockIdx.y * BN;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1, g = lane >> 5;
    const int K = p.K, nkb = K / BK;
    const int c16 = tid & 7;

    const uint8_t *Ab = p.A;
    const uint8_t *Bg = p.B0 + (size_t)e * p.N * K;
    const uint8_t *Bu = DUAL ? p.B1 + (size_t)e * p.N * K : Bg;
    const uint8_t *Sg = p.S0 + ((size_t)e * (p.N / 128) + n0 / 128) * nkb;
    const uint8_t *Su = DUAL ? p.S1 + ((size_t)e * (p.N / 128) + n0 / 128) * nkb : Sg;

    size_t aoff[4];  // A byte offsets (the A operand can pass 4 GiB: x_perm, h)
    uint32_t boff[BCH];
    int soffa[4], soffb[BCH];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = (tid >> 3) + 32 * i;
        int ar = m0 + row;
        ar = ar < m_end ? ar : m_end - 1;
        if (p.a_rows) ar = p.a_rows[ar] / p.a_div;
        aoff[i] = (size_t)ar * (size_t)K + c16 * 16;
        soffa[i] = row * BK + swz(row, c16) * 16;
    }
#pragma unroll
    for (int i = 0; i < BCH; ++i) {
        const int row = (tid >> 3) + 32 * i;
        const int br = n0 + (row % BN);
        boff[i] = (uint32_t)br * (uint32_t)K + c16 * 16;
        soffb[i] = row * BK + swz(row, c16) * 16;
    }
    // activation scale staging: threads 0..127, one row each
    int as_row = m0 + (tid & (BM - 1));
    as_row = as_row < m_end ? as_row : m_end - 1;
    if (p.a_rows) as_row = p.a_rows[as_row] / p.a_div;
    const uint8_t *asp = p.As + (size_t)as_row * nkb;

    f32x16 acc[2][NJ];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    i32x4 ra[4], rb[BCH];
    int ras = 0;
    for (int kt = -1; kt < nkb; ++kt) {
        if (kt + 1 < nkb) {
            const int k0 = (kt + 1) * BK;
#pragma unroll
            for (int i = 0; i < 4; ++i) ra[i] = *reinterpret_cast<const i32x4 *>(Ab + aoff[i] + k0);
#pragma unroll
            for (int i = 0; i < BCH; ++i)
                rb[i] = *reinterpret_cast<const i32x4 *>((DUAL && i >= BCH / 2 ? Bu : Bg) + boff[i] + k0);
            if (tid < BM) ras = asp[kt + 1];
        }
        if (kt >= 0) {
            const int buf = kt & 1;
            const int ebg = Sg[kt], ebu = Su[kt];
            i32x8 af[2][2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) af[i][hf] = frag(sA[buf], wm * 64 + i * 32 + (lane & 31), hf, g);
            // the E8M0 scale bytes go to the MFMA as they are: lanes l and
            // l+32 of the A operand carry row l % 32's; the weight block's is
            // the same for every lane
            int ea[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) ea[i] = sAs[buf][wm * 64 + i * 32 + (lane & 31)];
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int brow = DUAL ? ((j >> 1) * BN + wn * 64 + (j & 1) * 32 + (lane & 31))
                                      : (wn * 64 + j * 32 + (lane & 31));
                const i32x8 b0 = frag(sB[buf], brow, 0, g), b1 = frag(sB[buf], brow, 1, g);
                const int eb = (DUAL && j >= 2) ? ebu : ebg;
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i][0], b0, acc[i][j], 0, 0, 0, ea[i], 0, eb);
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i][1], b1, acc[i][j], 0, 0, 0, ea[i], 0, eb);
                }
            }
        }
        if (kt + 1 < nkb) {
            const int nb = (kt + 1) & 1;
#pragma unroll
            for (int i = 0; i < 4; ++i) *reinterpret_cast<i32x4 *>(&sA[nb][soffa[i]]) = ra[i];
#pragma unroll
            for (int i = 0; i < BCH; ++i) *reinterpret_cast<i32x4 *>(&sB[nb][soffb[i]]) = rb[i];
            if (tid < BM) sAs[nb][tid] = ras;
        }
        __syncthreads();
    }

    // 32x32 C layout: lane holds column (lane & 31), rows 8*(r>>2) + 4*g + (r&3).
    if (DUAL) {
        // h = silu(g) * u; per-row amax over this wave's 64 columns
        float h[2][2][16];
        float pm[2][16];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float m = 0.f;
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const float gv = acc[i][j][r], uv = acc[i][2 + j][r];
                    const float hv = gv / (1.0f + expf(-gv)) * uv;
                    h[i][j][r] = hv;
                    m = fmaxf(m, fabsf(hv));
                }
                // across the 32 lanes that hold the other columns of the same rows
#pragma unroll
                for (int s = 1; s < 32; s <<= 1) m = fmaxf(m, __shfl_xor(m, s, 64));
                pm[i][r] = m;
            }
        float *xch = reinterpret_cast<float *>(&sA[0][0]);  // [2 waves-in-N][BM]
        if ((lane & 31) == 0) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    xch[wn * BM + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * g + (r & 3)] = pm[i][r];
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int tr = wm * 64 + i * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
                const int row = m0 + tr;
                const float amax = fmaxf(pm[i][r], xch[(wn ^ 1) * BM + tr]);
                const float s = e4m3_tile_scale(amax);
                if (row < m_end) {
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const int col = n0 + wn * 64 + j * 32 + (lane & 31);
                        p.hq[(size_t)row * p.N + col] = (uint8_t)f32_to_e4m3(h[i][j][r] / s);
                    }
                    if (wn == 0 && (lane & 31) == 0) p.hs[(size_t)row * (p.N / 128) + n0 / 128] = (uint8_t)e8m0_of(s);
                }
            }
    } else {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
                if (row >= m_end) continue;
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const int col = n0 + wn * 64 + j * 32 + (lane & 31);
                    const float v = acc[i][j][r];
                    if (EPI == EPI_STORE)
                        p.out[(size_t)row * p.N + col] = (uint16_t)f32_to_bf16(v);
                    else  // the shared expert's fp32 output; the routed sum is added by k_combine_add
                        p.yout[(size_t)row * p.N + col] = v;
                }
            }
    }
}

}  // namespace

hipError_t launch_ffn_fp8(const FfnArgs &a, hipStream_t s) {
    if (ffn_fp8_mx_ok(a)) return launch_ffn_fp8_mx(a, s);
    const bool routed = a.offsets != nullptr;
    const int slots = (a.M + BM - 1) / BM + (routed ? kE : 0);
    Fp8Params p{};
    p.M = a.M;
    p.offsets = a.offsets;
    p.A = static_cast<const uint8_t *>(a.a);
    p.As = a.a_scale;
    p.a_rows = a.a_rows;
    p.a_div = a.a_div;
    p.K = a.d;
    p.B0 = static_cast<const uint8_t *>(a.w.gate);
    p.B1 = static_cast<const uint8_t *>(a.w.up);
    p.S0 = a.w.s_gate;
    p.S1 = a.w.s_up;
    p.N = a.I;
    p.hq = static_cast<uint8_t *>(a.h);
    p.hs = a.h_scale;
    if (a.phases & 1) hipLaunchKernelGGL(k_gemm_fp8<EPI_SWIGLU_Q>, dim3(slots, a.I / BN), dim3(256), 0, s, p);
    if (!(a.phases & 2)) return hipGetLastError();
    Fp8Params q{};
    q.M = a.M;
    q.offsets = a.offsets;
    q.A = static_cast<const uint8_t *>(a.h);
    q.As = a.h_scale;
    q.K = a.I;
    q.B0 = static_cast<const uint8_t *>(a.w.down);
    q.S0 = a.w.s_down;
    q.N = a.d;
    if (a.combine) {
        q.yout = static_cast<float *>(a.y);
        q.y_perm = static_cast<const uint16_t *>(a.y_perm);
        q.row_of = a.row_of;
        q.cw = a.cw;
        q.k = a.k;
        hipLaunchKernelGGL(k_gemm_fp8<EPI_COMBINE>, dim3(slots, a.d / BN), dim3(256), 0, s, q);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        return launch_combine_add(a.M, a.d, a.k, static_cast<const uint16_t *>(a.y_perm), a.row_of, a.cw,
                                  static_cast<float *>(a.y), s);
    } else {
        q.out = static_cast<uint16_t *>(a.y);
        hipLaunchKernelGGL(k_gemm_fp8<EPI_STORE>, dim3(slots, a.d / BN), dim3(256), 0, s, q);
    }
    return hipGetLastError();
}

}  // namespace moe
