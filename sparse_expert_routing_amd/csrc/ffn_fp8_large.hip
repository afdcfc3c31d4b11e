// Grouped SwiGLU expert GEMMs in OCP fp8 e4m3 with fine-grained scales, for
// large groups (prefill): persistent workgroups, 256x256 tiles.
//
// crackai.dev DeepSeek-V3 summary, "How It Works": FP8 matmuls with a scale
// per tile and FP32 accumulation at chosen points; DeepSeek V3 From Scratch,
// "The idea": fine-grained quantisation tiles.  Tile shapes (ours, as in the
// rest of the library): one power-of-two scale per 1x128 activation tile and
// per 128x128 weight block, applied inside the MFMA; fp32 accumulation.
//
// Design for gfx950 (shared with the bf16 large-tile kernel where it can be):
//   - 8 waves (2 per SIMD) in a 2x4 layout, each a 128x64 block of the
//     256x256 tile; its fp32 accumulators (128 per lane) live in VGPRs;
//   - one stage = 128 of K = one scale block: A and B slabs of 256 rows x
//     128 bytes (whole L2 lines) in a ring of five 32 KB LDS units filled by
//     buffer_load_dwordx4 ... lds (scalar resource, fixed per-lane offset,
//     stage offset in an SGPR); during stage s, after its one barrier,
//     B_{s+1} and A_{s+2} stream into the two units stage s-1 left, one load
//     per output block, so B has about a stage and A two stages to land;
//   - each 32x32 output block takes two v_mfma_scale_f32_32x32x64_f8f6f4
//     per stage that accumulate straight into the fp32 accumulator, the
//     stage's scales given to the matrix unit as E8M0 exponents: the
//     weight block's for the first operand (every lane), each A row's for
//     the second (lanes l and l+32 carry row l % 32); no vector fold;
//   - the MFMA operands are swapped, so a lane owns one tile row and runs
//     of 4 consecutive output columns: per-row activation scales are per
//     lane, weight scales per wave;
//   - the activation scales of the next stage are loaded before its slot
//     loads, so one vmcnt wait per stage covers both;
//   - epilogues: gate/up forms h = silu(g) * u in fp32 and quantises it per
//     1x128 tile (the tile's 128 h columns; the row amax is combined across
//     the four column waves through LDS), scale = the power of two at or
//     above amax / 448 (1 for an all-zero tile), code = e4m3(h / scale); down
//     stores bf16 y_perm, or (the
//     shared expert) forms y = acc + sum_j w_j * y_perm[row_of[t*k + j]] in
//     fp32, ascending j, staging the tile through LDS in 64-row chunks so
//     each routed row is gathered as one 512-byte run per half-wave.
#include "device.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kE = 256;
constexpr int LM = 256;      // rows per tile
constexpr int LB = 256;      // B rows per tile
constexpr int LK = 128;      // K (bytes) per stage = one scale block
constexpr int NUNIT = 5;     // LDS ring units (5 x 32 KB)
constexpr int UNIT_BYTES = LM * LK;
constexpr int kGroupM = 8;   // row tiles per ordering group

// EPI_F32: a plain fp32 product (the layer backward's GEMMs), row stride ldo.
enum { EPI_SWIGLU_Q = 0, EPI_STORE = 1, EPI_COMBINE = 2, EPI_F32 = 3 };
// A buffer-store offset past the end of every fp32 output (the host keeps
// them below kOobOff - 1 MB): stores of padding rows are dropped.
constexpr uint32_t kOobOff = 0xFFFF0000u;

typedef __attribute__((address_space(3))) void lds_void_t;
typedef int i32x2 __attribute__((ext_vector_type(2)));

struct F8Params {
    int M;
    const int32_t *offsets;
    const uint8_t *A;         // [rows, K] codes
    const float *As;          // [rows, K/128]
    const int32_t *a_rows;    // optional: GEMM row r reads row a_rows[r] / a_div of A / As
    int a_div;
    int K;
    const uint8_t *B0, *B1;   // [G, N, K] codes
    const float *S0, *S1;     // [G, N/128, K/128]
    int N;
    uint8_t *hq;              // EPI_SWIGLU_Q: [M, H] codes
    float *hs;                // EPI_SWIGLU_Q: [M, H/128]
    int H;                    // EPI_SWIGLU_Q: h columns (= N)
    uint16_t *out;            // EPI_STORE: bf16 [M, N]
    float *yout;              // EPI_COMBINE: f32 [M, N]; EPI_F32: f32 rows of ldo
    int ldo;                  // EPI_F32
    const uint16_t *y_perm;   // EPI_COMBINE: routed outputs [M*k, N] bf16
    const int32_t *row_of;    // EPI_COMBINE: [M*k]
    const float *cw;          // EPI_COMBINE: combine weights [M*k]
};

struct TileMap {
    int off[5];
    int nt[4];
    int excl, total;
};

__device__ __forceinline__ void tilemap_init(TileMap &tm, const int32_t *__restrict__ offsets) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < 5; ++i) tm.off[i] = offsets[lane * 4 + i];
    int s = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        tm.nt[i] = (tm.off[i + 1] - tm.off[i] + LM - 1) / LM;
        s += tm.nt[i];
    }
    const int incl = wave_incl_scan(s);
    tm.excl = incl - s;
    tm.total = __shfl(incl, 63, 64);
}

__device__ __forceinline__ void tilemap_find(const TileMap &tm, int mt, int &e, int &m0, int &m_end) {
    const int lane = threadIdx.x & 63;
    const int mine = tm.nt[0] + tm.nt[1] + tm.nt[2] + tm.nt[3];
    const bool own = mt >= tm.excl && mt < tm.excl + mine;
    const int owner = __ffsll((unsigned long long)__ballot(own)) - 1;
    int my_e = 0, my_m0 = 0, my_end = 0;
    if (own) {
        int s = mt - tm.excl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (s >= 0 && s < tm.nt[i]) {
                my_e = lane * 4 + i;
                my_m0 = tm.off[i] + s * LM;
                my_end = tm.off[i + 1];
            }
            s -= tm.nt[i];
        }
    }
    e = __shfl(my_e, owner, 64);
    m0 = __shfl(my_m0, owner, 64);
    m_end = __shfl(my_end, owner, 64);
}

// Byte offset, inside one operand unit, of the 16-byte piece c (K bytes
// 16c .. 16c+15) of tile row `row`: the same XOR swizzle as the bf16 kernel.
__device__ __forceinline__ int piece(int row, int c) {
    return row * LK + ((c ^ (row & 7) ^ ((row >> 3) & 1)) * 16);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt_lds() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ const void *uniform_ptr(const void *p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<const void *>(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ void dma_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint8_t *lds_block) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)(lds_block), 16, voff, soff, 0, 0);
}

// 32 bytes of K (pieces c and c+1 of the row) as one MFMA operand.
__device__ __forceinline__ i32x8 frag32(const uint8_t *unit, int row, int c) {
    const i32x4 lo = *reinterpret_cast<const i32x4 *>(unit + piece(row, c));
    const i32x4 hi = *reinterpret_cast<const i32x4 *>(unit + piece(row, c + 1));
    return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// The E8M0 exponent of a power-of-two fp32 scale (its biased exponent field).
__device__ __forceinline__ int e8m0(float pow2) { return (int)((__float_as_uint(pow2) >> 23) & 0xffu); }

__device__ __forceinline__ float swiglu(float g, float u) {
    return g * u * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * g));
}

// Eight waves (two per SIMD), each owning 128 rows x 64 columns of the
// 256x256 tile: its 128 fp32 accumulators fit in VGPRs, and while one wave of a SIMD waits on
// its MFMA result, LDS or the barrier, the other issues.  A wave's DMA
// share is 4 of the 32 one-KB blocks of each operand slab.
template <int EPI, bool ROUTED>
__global__ __launch_bounds__(512, 1) void k_gemm_fp8_large(F8Params p) {
    constexpr bool DUAL = EPI == EPI_SWIGLU_Q;
    constexpr int BN = DUAL ? LB / 2 : LB;  // output columns per tile
    __shared__ __attribute__((aligned(1024))) uint8_t smem[NUNIT * UNIT_BYTES];  // 160 KB

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3, g = lane >> 5;
    const int K = p.K, nk = K / LK;

    // (the tile map is rebuilt per tile rather than kept: its registers are
    // needed by the K loop)
    int Mt;
    if (ROUTED) {
        TileMap tm0;
        tilemap_init(tm0, p.offsets);
        Mt = tm0.total;
    } else {
        Mt = (p.M + LM - 1) / LM;
    }
    const int NT = p.N / BN;
    const int total = Mt * NT;
    const int P = gridDim.x;

    // DMA geometry: wave w moves blocks w + 8i (i < 4) of each operand slab;
    // lane l fills physical piece (l & 7) of row 8*blk + (l >> 3).
    int drow[4], dcol[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 8 * (wave + 8 * i) + (lane >> 3);
        drow[i] = row;
        dcol[i] = ((lane & 7) ^ (row & 7) ^ ((row >> 3) & 1)) * 16;
    }
    const uint32_t a_rows_total = p.a_rows ? (uint32_t)(p.M / p.a_div) : (uint32_t)p.M;
    const __amdgpu_buffer_rsrc_t rA = buf_rsrc(p.A, a_rows_total * (uint32_t)K);
    const __amdgpu_buffer_rsrc_t rAs = buf_rsrc(p.As, a_rows_total * (uint32_t)nk * 4u);
    const uint32_t b_bytes = (uint32_t)p.N * (uint32_t)K;
    const int nbk = p.N / 128;  // weight scale blocks along N

#define UNIT(u) (smem + (u) * UNIT_BYTES)

    for (int t = (blockIdx.x & 7) * (P >> 3) + (blockIdx.x >> 3); t < total; t += P) {
        const int gsz = kGroupM * NT;
        const int grp = t / gsz, within = t - grp * gsz;
        const int mfirst = grp * kGroupM;
        const int gm = min(kGroupM, Mt - mfirst);
        const int mt = mfirst + within % gm, nt = within / gm;
        int e, m0, m_end;
        if (ROUTED) {
            TileMap tm;
            tilemap_init(tm, p.offsets);
            tilemap_find(tm, mt, e, m0, m_end);
        } else {
            e = 0;
            m0 = mt * LM;
            m_end = p.M;
        }
        e = __builtin_amdgcn_readfirstlane(e);
        m0 = __builtin_amdgcn_readfirstlane(m0);
        m_end = __builtin_amdgcn_readfirstlane(m_end);
        const int n0 = nt * BN;

        const __amdgpu_buffer_rsrc_t rBg = buf_rsrc(uniform_ptr(p.B0 + (size_t)e * p.N * K), b_bytes);
        const __amdgpu_buffer_rsrc_t rBu = DUAL ? buf_rsrc(uniform_ptr(p.B1 + (size_t)e * p.N * K), b_bytes) : rBg;
        uint32_t aoff[4], boff[4];
        {
            int ar_[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) ar_[i] = min(m0 + drow[i], m_end - 1);
            if (p.a_rows) {
#pragma unroll
                for (int i = 0; i < 4; ++i) ar_[i] = p.a_rows[ar_[i]];
#pragma unroll
                for (int i = 0; i < 4; ++i) ar_[i] /= p.a_div;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                aoff[i] = (uint32_t)ar_[i] * (uint32_t)K + (uint32_t)dcol[i];
                const int r = drow[i];
                const int br = DUAL ? n0 + (r & (BN - 1)) : n0 + r;
                boff[i] = (uint32_t)br * (uint32_t)K + (uint32_t)dcol[i];
            }
        }
        // this lane's 4 tile rows (wm*128 + 32i + (lane & 31)): activation-
        // scale byte offsets (rows past the group repeat its last)
        uint32_t soff[4];
        {
            int sr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) sr[i] = min(m0 + wm * 128 + 32 * i + (lane & 31), m_end - 1);
            if (p.a_rows) {
#pragma unroll
                for (int i = 0; i < 4; ++i) sr[i] = p.a_rows[sr[i]] / p.a_div;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) soff[i] = (uint32_t)sr[i] * (uint32_t)nk * 4u;
        }
        // weight scales: the 128-column block of this wave's columns (gate
        // and up blocks of the SwiGLU tile), [G, N/128, K/128]
        const float *swg_p = p.S0 + ((size_t)e * nbk + (DUAL ? n0 : n0 + wn * 64) / 128) * nk;
        const float *swu_p = DUAL ? p.S1 + ((size_t)e * nbk + n0 / 128) * nk : swg_p;

#define ISSUE_A(st_, i, unit_)                                                                 \
        dma_buf(rA, aoff[i], (uint32_t)min((st_), nk - 1) * LK, (unit_) + (wave + 8 * (i)) * 1024)
#define ISSUE_B(st_, i, unit_)                                                                 \
        dma_buf((DUAL && (i) >= 2) ? rBu : rBg, boff[i], (uint32_t)min((st_), nk - 1) * LK,        \
                (unit_) + (wave + 8 * (i)) * 1024)
#define LOAD_SCALES(st_, sa_, sw_)                                                             \
        {                                                                                      \
            const int kb_ = min((st_), nk - 1);                                                \
            _Pragma("unroll") for (int i = 0; i < 4; ++i)                                      \
                sa_[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rAs, soff[i] + kb_ * 4u, 0, 0)); \
            sw_[0] = swg_p[kb_];                                                               \
            sw_[1] = DUAL ? swu_p[kb_] : sw_[0];                                               \
        }

        f32x16 acc[4][2];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

        // Prologue: scales(0), A_0, B_0, A_1 in flight.
        float sa[4], sw[2], sa_n[4], sw_n[2];
        LOAD_SCALES(0, sa, sw);
#pragma unroll
        for (int i = 0; i < 4; ++i) ISSUE_A(0, i, UNIT(0));
#pragma unroll
        for (int i = 0; i < 4; ++i) ISSUE_B(0, i, UNIT(1));
#pragma unroll
        for (int i = 0; i < 4; ++i) ISSUE_A(1, i, UNIT(2));

        int u0 = 0;  // unit of A_kt (2kt mod 5)
        for (int kt = 0; kt < nk; ++kt) {
            const int u1 = u0 + 1 - (u0 + 1 >= NUNIT ? NUNIT : 0);
            const int u3 = u0 + 3 - (u0 + 3 >= NUNIT ? NUNIT : 0);
            const int u4 = u0 + 4 - (u0 + 4 >= NUNIT ? NUNIT : 0);
            // A_kt, B_kt and this stage's scales landed (only A_{kt+1}, 4
            // loads, may still be in flight) for every wave; the units of
            // stage kt-1 are no longer read by anyone.
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            wait_vmcnt_lds<4>();
            __builtin_amdgcn_s_barrier();
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            LOAD_SCALES(kt + 1, sa_n, sw_n);
            uint8_t *fB = UNIT(u3), *fA = UNIT(u4);  // B_{kt+1}, A_{kt+2}: one load per block below

            const uint8_t *cA = UNIT(u0), *cB = UNIT(u1);
            // B fragments of the whole stage (2 column blocks x 2 K halves);
            // A fragments per row block.  The tile scales are powers of two,
            // applied by the MFMA itself as E8M0 exponents: the weight block's
            // (the same for every lane of the first operand) and each A row's
            // (lanes l and l+32 of the second operand carry row l % 32), so
            // the products accumulate straight into acc.
            i32x8 bf[2][2], af[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int brow = (DUAL ? (j * 128 + wn * 32) : (wn * 64 + j * 32)) + (lane & 31);
#pragma unroll
                for (int s = 0; s < 2; ++s) bf[j][s] = frag32(cB, brow, 4 * s + 2 * g);
            }
            const int eb0 = e8m0(sw[0]), eb1 = DUAL ? e8m0(sw[1]) : eb0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
#pragma unroll
                for (int s = 0; s < 2; ++s) af[s] = frag32(cA, wm * 128 + 32 * i + (lane & 31), 4 * s + 2 * g);
                const int ea = e8m0(sa[i]);
                // the two column blocks' first K halves, then their second
                // halves (consecutive MFMAs independent); one slot load after
                // each pair (B first: it has one stage to land)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bf[j][h], af[h], acc[i][j], 0, 0, 0,
                                                                                     j ? eb1 : eb0, 0, ea);
                    const int n = 2 * i + h;
                    if (n < 4) ISSUE_B(kt + 1, n, fB);
                    else ISSUE_A(kt + 2, n - 4, fA);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) sa[i] = sa_n[i];
            sw[0] = sw_n[0];
            sw[1] = sw_n[1];
            u0 = u0 + 2 - (u0 + 2 >= NUNIT ? NUNIT : 0);
        }
#undef ISSUE_A
#undef ISSUE_B
#undef LOAD_SCALES
        __syncthreads();  // every wave done with the ring (and all its loads landed)

        // lane: tile rows wm*128 + 32i + (lane & 31); per 32-column block j,
        // columns 8q + 4g + u (u = 0..3) in acc[i][j][4q + u]
        const int c4 = 4 * g;
        if constexpr (DUAL) {
            // h columns of this wave: wn*32 + 8q + 4g + u; the tile's 128 h
            // columns are one quantisation tile, spread over the 4 column waves
            float *xch = reinterpret_cast<float *>(UNIT(4));  // [4][256] partial row amax
            float hv[4][16];
            float am[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float m = 0.f;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float h = swiglu(acc[i][0][r], acc[i][1][r]);
                    hv[i][r] = h;
                    m = fmaxf(m, fabsf(h));
                }
                m = fmaxf(m, __shfl_xor(m, 32, 64));  // the other 16 columns of this wave
                am[i] = m;
                if (g == 0) xch[wn * 256 + wm * 128 + 32 * i + lane] = m;
            }
            __syncthreads();
            const __amdgpu_buffer_rsrc_t rQ = buf_rsrc(p.hq, (uint32_t)p.M * (uint32_t)p.H);
            const __amdgpu_buffer_rsrc_t rS = buf_rsrc(p.hs, (uint32_t)p.M * (uint32_t)(p.H / 128) * 4u);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tr = wm * 128 + 32 * i + (lane & 31);
                const int row = m0 + tr;
                float amax = am[i];
#pragma unroll
                for (int w = 0; w < 4; ++w) amax = fmaxf(amax, xch[w * 256 + tr]);
                const float s = e4m3_tile_scale(amax);
                const bool ok = row < m_end;
                const uint32_t qbase = ok ? (uint32_t)row * (uint32_t)p.H + (uint32_t)n0 : 0xfffff000u;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    uint32_t w = 0;
#pragma unroll
                    for (int u = 0; u < 4; ++u) w |= f32_to_e4m3(hv[i][4 * q + u] / s) << (8 * u);
                    __builtin_amdgcn_raw_buffer_store_b32((int)w, rQ, qbase + (uint32_t)(wn * 32 + 8 * q + c4), 0, 0);
                }
                if (wn == 0 && g == 0) {
                    const uint32_t so = ok ? ((uint32_t)row * (uint32_t)(p.H / 128) + (uint32_t)(n0 / 128)) * 4u
                                           : 0xfffff000u;
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(s), rS, so, 0, 0);
                }
            }
            __syncthreads();  // xch read by all before the next tile's loads reuse the ring
        } else if constexpr (EPI == EPI_STORE) {
            const __amdgpu_buffer_rsrc_t rOut = buf_rsrc(p.out, (uint32_t)p.M * (uint32_t)p.N * 2u);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = m0 + wm * 128 + 32 * i + (lane & 31);
                const uint32_t obase = row < m_end ? ((uint32_t)row * (uint32_t)p.N + (uint32_t)n0) * 2u : 0xfffff000u;
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const uint32_t lo = pack_bf16x2(acc[i][j][4 * q], acc[i][j][4 * q + 1]);
                        const uint32_t hi = pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
                        const int col = wn * 64 + j * 32 + 8 * q + c4;
                        __builtin_amdgcn_raw_buffer_store_b64(i32x2{(int)lo, (int)hi}, rOut, obase + (uint32_t)col * 2u,
                                                              0, 0);
                    }
            }
        } else if constexpr (EPI == EPI_F32) {
            // one 16-byte store per run of 4 columns; padding rows go to kOobOff
            const __amdgpu_buffer_rsrc_t rOutF = buf_rsrc(p.yout, (uint32_t)p.M * (uint32_t)p.ldo * 4u);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = m0 + wm * 128 + 32 * i + (lane & 31);
                const uint32_t obase = row < m_end ? ((uint32_t)row * (uint32_t)p.ldo + (uint32_t)n0) * 4u : kOobOff;
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int col = wn * 64 + j * 32 + 8 * q + c4;
                        __builtin_amdgcn_raw_buffer_store_b128(
                            i32x4{__float_as_int(acc[i][j][4 * q]), __float_as_int(acc[i][j][4 * q + 1]),
                                  __float_as_int(acc[i][j][4 * q + 2]), __float_as_int(acc[i][j][4 * q + 3])},
                            rOutF, obase + (uint32_t)col * 4u, 0, 0);
                    }
            }
        } else {
            // four 64-row chunks of the fp32 tile through LDS (the ring is
            // free), then each half-wave gathers one routed output row as a
            // contiguous 512-byte run
            constexpr int kChRows = 64, kChLd = LB + 4;
            float *ch = reinterpret_cast<float *>(smem);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                if (wm == (c >> 1)) {
#pragma unroll
                    for (int ii = 0; ii < 2; ++ii) {
                        const int i = 2 * (c & 1) + ii;
                        const int rl = ii * 32 + (lane & 31);
#pragma unroll
                        for (int j = 0; j < 2; ++j)
#pragma unroll
                            for (int q = 0; q < 4; ++q) {
                                const int col = wn * 64 + j * 32 + 8 * q + c4;
                                *reinterpret_cast<f32x4 *>(ch + rl * kChLd + col) =
                                    f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
                            }
                    }
                }
                __syncthreads();
                const int cl = 8 * (lane & 31);
#pragma unroll 2
                for (int it = 0; it < 4; ++it) {
                    const int rl = wave * 8 + 2 * it + g;
                    const int row = m0 + c * kChRows + rl;
                    if (row < m_end) {
                        int rof[8];
                        float wj[8];
#pragma unroll
                        for (int jj = 0; jj < 8; ++jj) {
                            rof[jj] = p.row_of[(size_t)row * 8 + jj];
                            wj[jj] = p.cw[(size_t)row * 8 + jj];
                        }
                        i32x4 yv[8];
#pragma unroll
                        for (int jj = 0; jj < 8; ++jj)
                            yv[jj] = *reinterpret_cast<const i32x4 *>(p.y_perm + (size_t)rof[jj] * p.N + n0 + cl);
                        const float *cr = ch + rl * kChLd + cl;
                        const f32x4 s0 = *reinterpret_cast<const f32x4 *>(cr);
                        const f32x4 s1 = *reinterpret_cast<const f32x4 *>(cr + 4);
                        float v[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
#pragma unroll
                        for (int jj = 0; jj < 8; ++jj)
#pragma unroll
                            for (int u = 0; u < 4; ++u) {
                                v[2 * u] += wj[jj] * bf16_to_f32((uint32_t)yv[jj][u] & 0xffffu);
                                v[2 * u + 1] += wj[jj] * bf16_to_f32((uint32_t)yv[jj][u] >> 16);
                            }
                        float *yo = p.yout + (size_t)row * p.N + n0 + cl;
                        *reinterpret_cast<f32x4 *>(yo) = f32x4{v[0], v[1], v[2], v[3]};
                        *reinterpret_cast<f32x4 *>(yo + 4) = f32x4{v[4], v[5], v[6], v[7]};
                    }
                }
                __syncthreads();
            }
        }
    }
#undef UNIT
}

int cu_count() {
    static int cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

}  // namespace

bool ffn_fp8_large_ok(const FfnArgs &a) {
    const int groups = a.offsets ? a.E : 1;
    const unsigned long long lim = 1ULL << 32;
    const bool fits = (unsigned long long)a.M * a.d < lim && (unsigned long long)a.M * a.I * 2 < lim &&
                      (unsigned long long)a.M * a.d * 4 < lim && (unsigned long long)a.I * a.d < lim;
    return fits && (long long)a.M >= 128LL * groups && a.I % 128 == 0 && a.d % 256 == 0 && a.d % LK == 0 &&
           a.I % LK == 0;
}

bool fp8_large_gemm_ok(const Fp8GemmArgs &g) {
    const int groups = g.offsets ? kE : 1;
    const unsigned long long lim = 1ULL << 32;
    const unsigned long long a_rows = g.a_rows ? (unsigned long long)g.a_src_rows : (unsigned long long)g.M;
    return (long long)g.M >= 128LL * groups && g.N % LB == 0 && g.K % LK == 0 && a_rows * g.K < lim &&
           a_rows * (g.K / LK) * 4 < lim && (unsigned long long)g.N * g.K < lim &&
           (unsigned long long)g.M * g.ldo * 4 < kOobOff - (1ULL << 20) && g.ldo >= g.N;
}

hipError_t launch_fp8_large_gemm(const Fp8GemmArgs &g, hipStream_t s) {
    const int P = (cu_count() / 8) * 8;
    F8Params p{};
    p.M = g.M;
    p.offsets = g.offsets;
    p.A = g.A;
    p.As = g.As;
    p.a_rows = g.a_rows;
    p.a_div = g.a_rows ? g.a_div : 1;
    p.K = g.K;
    p.B0 = g.B;
    p.S0 = g.Bs;
    p.N = g.N;
    p.yout = g.out;
    p.ldo = g.ldo;
    if (g.offsets) hipLaunchKernelGGL((k_gemm_fp8_large<EPI_F32, true>), dim3(P), dim3(512), 0, s, p);
    else hipLaunchKernelGGL((k_gemm_fp8_large<EPI_F32, false>), dim3(P), dim3(512), 0, s, p);
    return hipGetLastError();
}

// Phase 1 (gate/up, fused SwiGLU + h quantisation) and / or phase 2 (down:
// bf16 y_perm, or the shared expert's output with the weighted combine).
hipError_t launch_ffn_fp8_large(const FfnArgs &a, hipStream_t s) {
    const int P = (cu_count() / 8) * 8;
    const bool routed = a.offsets != nullptr;
    if (a.phases & 1) {
        F8Params p{};
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
        p.N = a.I;  // rows of each of gate / up; a tile takes 128 of each
        p.hq = static_cast<uint8_t *>(a.h);
        p.hs = a.h_scale;
        p.H = a.I;
        if (routed)
            hipLaunchKernelGGL((k_gemm_fp8_large<EPI_SWIGLU_Q, true>), dim3(P), dim3(512), 0, s, p);
        else
            hipLaunchKernelGGL((k_gemm_fp8_large<EPI_SWIGLU_Q, false>), dim3(P), dim3(512), 0, s, p);
    }
    if (a.phases & 2) {
        F8Params q{};
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
            // the combine belongs to the shared expert (one group)
            hipLaunchKernelGGL((k_gemm_fp8_large<EPI_COMBINE, false>), dim3(P), dim3(512), 0, s, q);
            return hipGetLastError();
        }
        q.out = static_cast<uint16_t *>(a.y);
        if (routed)
            hipLaunchKernelGGL((k_gemm_fp8_large<EPI_STORE, true>), dim3(P), dim3(512), 0, s, q);
        else
            hipLaunchKernelGGL((k_gemm_fp8_large<EPI_STORE, false>), dim3(P), dim3(512), 0, s, q);
    }
    return hipGetLastError();
}

}  // namespace moe
