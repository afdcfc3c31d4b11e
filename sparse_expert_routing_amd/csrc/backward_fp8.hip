// Backward of the MoE layer with e4m3 expert weights: every GEMM of the
// backward on e4m3 operands with an E8M0 scale per tile and fp32 accumulation.
//
// crackai.dev DeepSeek-V3 summary, "How It Works": FP8 in the forward and
// the backward pass, a scale per tile, FP32 accumulation at chosen points.
// Where the tiles lie is our reading: along each GEMM's reduction, 128 wide.
//   - data-gradient GEMMs (dh = dy_out W_down, dx = (da | db) (W_gate | W_up))
//     reduce along a row: the output gradient per 1x128 tile of d and the
//     SwiGLU input gradients per 1x128 tile of I (k_q8_rows), against the
//     stored 128x128 weight blocks, transposed as blocks (k_t8, k_tscale);
//   - the pre-activations are recomputed by the forward's own product
//     (x per 1x128 tile of d against the gate and up blocks);
//   - weight-gradient GEMMs reduce over an expert's rows: the rows, in
//     dispatch order, are laid out column-major in groups of 128 (an
//     expert's rows start at a 128-aligned position, zero-padded), and each
//     column of a group is one tile (k_q8_cols), quantised from the fp32
//     values (the bf16 x for dW_gate and dW_up);
//   - the router, the combine backward and the dx assembly stay fp32 (the
//     steps shared with the bf16 backward).
//
// The M-grouped and plain products with block-scaled weights (the recompute
// and the data gradients) run on the forward's persistent e4m3 kernel with an
// fp32 epilogue, and the weight gradients on its K-grouped form, when the
// shape fits it; k_fgemm takes the rest.
// k_fgemm: C = A B^T with both operands K-contiguous e4m3 codes, 128x128
// tiles, one 128-wide scale block per stage (two v_mfma_scale 32x32x64 fp8
// per 32x32 block, accumulating in fp32, the E8M0 scales s_a[row, kb] and
// s_b[col, kb] applied by the MFMA); register-staged
// LDS double buffer with an XOR swizzle of the 16-byte chunks.  Groups split M (a B per expert: the data
// gradients) or K (an expert's padded rows: the weight gradients, a C per
// expert).
#include "backward.h"
#include "device.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kE = 256;
constexpr int FM = 128, FN = 128, FK = 128;  // tile rows, columns; K bytes per stage (one scale block)

enum { FG_NONE = 0, FG_M = 1, FG_K = 2 };

struct FGemm {
    int M, N, K;              // FG_K: K = the padded row count
    const int32_t *offsets;   // [E+1]: FG_M row ranges; FG_K 128-aligned K ranges
    const uint8_t *A;         // A(m, k) = A[m*lda + k]
    int64_t lda;
    const uint8_t *As;        // s_a(m, kb) = As[m*ldas + kb] (E8M0)
    int64_t ldas;
    const int32_t *a_rows;    // optional: row m reads row a_rows[m] / a_div of A and As
    int a_div;
    const uint8_t *B;         // B(n, k) = B[g*bstride + n*ldb + k]
    int64_t ldb, bstride;
    const uint8_t *Bs;        // s_b(n, kb) = Bs[g*bsstride + (n / bdiv)*ldbs + kb] (E8M0)
    int64_t ldbs, bsstride;
    int bdiv;                 // 128: weight blocks; 1: a scale per row
    float *C;                 // C[g*cstride + m*ldc + n]
    int64_t ldc, cstride;
};

// Row-tile slot -> (group, first row, end row) over sum_e ceil(c_e / 128)
// tiles (one wave's scan; all lanes agree).
__device__ __forceinline__ bool fg_find_tile(const int32_t *__restrict__ offsets, int slot, int &gi, int &m0,
                                             int &m_end) {
    const int lane = threadIdx.x & 63;
    const int base = lane * 4;
    int off[5];
#pragma unroll
    for (int i = 0; i < 5; ++i) off[i] = offsets[base + i];
    int nt[4], lane_t = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        nt[i] = (off[i + 1] - off[i] + FM - 1) / FM;
        lane_t += nt[i];
    }
    const int incl = wave_incl_scan(lane_t);
    const int excl = incl - lane_t;
    const int total = __shfl(incl, 63, 64);
    if (slot >= total) return false;
    const bool own = slot >= excl && slot < incl;
    const int owner = __ffsll((unsigned long long)__ballot(own)) - 1;
    int my_g = 0, my_m0 = 0, my_end = 0;
    if (own) {
        int q = slot - excl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (q >= 0 && q < nt[i]) {
                my_g = base + i;
                my_m0 = off[i] + q * FM;
                my_end = off[i + 1];
            }
            q -= nt[i];
        }
    }
    gi = __shfl(my_g, owner, 64);
    m0 = __shfl(my_m0, owner, 64);
    m_end = __shfl(my_end, owner, 64);
    return true;
}

__device__ __forceinline__ int swz8(int row, int c16) { return c16 ^ (row & 7); }

// 32 K-bytes of one operand row for v_mfma_scale_f32_32x32x64_f8f6f4: K half `hf`
// of the 128-byte row; lane group g = lane / 32 takes bytes 64*hf + 32*g.
__device__ __forceinline__ i32x8 frag8(const uint8_t *tile, int row, int hf, int g) {
    const int c0 = 4 * hf + 2 * g;
    const i32x4 lo = *reinterpret_cast<const i32x4 *>(tile + row * FK + swz8(row, c0) * 16);
    const i32x4 hi = *reinterpret_cast<const i32x4 *>(tile + row * FK + swz8(row, c0 + 1) * 16);
    return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

template <int GROUP>
__global__ __launch_bounds__(256, 2) void k_fgemm(FGemm p) {
    __shared__ __attribute__((aligned(16))) uint8_t sA[2][FM * FK];
    __shared__ __attribute__((aligned(16))) uint8_t sB[2][FN * FK];
    __shared__ int sAs[2][FM], sBs[2][FN];  // E8M0 bytes
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1, g = lane >> 5, c16 = tid & 7;

    int gi = 0, m0, m_end, k_begin = 0, k_end = p.K;
    const int n0 = blockIdx.y * FN;
    if (GROUP == FG_M) {
        if (!fg_find_tile(p.offsets, blockIdx.x, gi, m0, m_end)) return;
    } else {
        m0 = blockIdx.x * FM;
        m_end = p.M;
        if (GROUP == FG_K) {
            gi = blockIdx.z;
            k_begin = p.offsets[gi];
            k_end = p.offsets[gi + 1];
        }
    }
    const uint8_t *B = p.B + (GROUP == FG_M ? (int64_t)gi * p.bstride : 0);
    const uint8_t *Bs = p.Bs + (GROUP == FG_M ? (int64_t)gi * p.bsstride : 0);
    float *C = p.C + (GROUP == FG_K ? (int64_t)gi * p.cstride : 0);

    // this thread's 16-byte chunks of the A and B stage tiles: rows
    // tid / 8 + 32 i, chunk tid % 8 (rows past m_end repeat the last row;
    // they are not stored)
    int64_t aoff[4], boff[4];
    int soff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = (tid >> 3) + 32 * i;
        int ar = m0 + row;
        ar = ar < m_end ? ar : m_end - 1;
        if (p.a_rows) ar = p.a_rows[ar] / p.a_div;
        aoff[i] = (int64_t)ar * p.lda + c16 * 16;
        boff[i] = (int64_t)(n0 + row) * p.ldb + c16 * 16;
        soff[i] = row * FK + swz8(row, c16) * 16;
    }
    // scale staging: threads 0..127 carry A row tid, 128..255 B row tid - 128
    const uint8_t *sp;
    if (tid < FM) {
        int ar = m0 + tid;
        ar = ar < m_end ? ar : m_end - 1;
        if (p.a_rows) ar = p.a_rows[ar] / p.a_div;
        sp = p.As + (int64_t)ar * p.ldas;
    } else {
        sp = Bs + (int64_t)((n0 + tid - FM) / p.bdiv) * p.ldbs;
    }

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int nkb = (k_end - k_begin) / FK;  // K ranges are whole stages
    i32x4 ra[4], rb[4];
    int rs = 0;
    for (int kt = -1; kt < nkb; ++kt) {
        if (kt + 1 < nkb) {
            const int64_t k0 = k_begin + (int64_t)(kt + 1) * FK;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                ra[i] = *reinterpret_cast<const i32x4 *>(p.A + aoff[i] + k0);
                rb[i] = *reinterpret_cast<const i32x4 *>(B + boff[i] + k0);
            }
            rs = sp[k0 / FK];
        }
        if (kt >= 0) {
            const int buf = kt & 1;
            i32x8 af[2][2], bq[2][2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    af[i][hf] = frag8(sA[buf], wm * 64 + i * 32 + (lane & 31), hf, g);
                    bq[i][hf] = frag8(sB[buf], wn * 64 + i * 32 + (lane & 31), hf, g);
                }
            // the stage's E8M0 scales go to the MFMA as they are: lanes l and
            // l+32 of each operand carry the scale of the operand row l % 32
            // they hold (A rows, B rows = C columns)
            int ea[2], eb[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                ea[i] = sAs[buf][wm * 64 + i * 32 + (lane & 31)];
                eb[i] = sBs[buf][wn * 64 + i * 32 + (lane & 31)];
            }
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i][hf], bq[j][hf], acc[i][j], 0, 0,
                                                                                     0, ea[i], 0, eb[j]);
        }
        if (kt + 1 < nkb) {
            const int nb = (kt + 1) & 1;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                *reinterpret_cast<i32x4 *>(&sA[nb][soff[i]]) = ra[i];
                *reinterpret_cast<i32x4 *>(&sB[nb][soff[i]]) = rb[i];
            }
            if (tid < FM) sAs[nb][tid] = rs;
            else sBs[nb][tid - FM] = rs;
        }
        __syncthreads();
    }
    // 32x32 C layout: lane holds column (lane & 31), rows 8 (r / 4) + 4 g + r % 4
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
            if (row >= m_end) continue;
#pragma unroll
            for (int j = 0; j < 2; ++j) C[(int64_t)row * p.ldc + n0 + wn * 64 + j * 32 + (lane & 31)] = acc[i][j][r];
        }
}

template <int GROUP>
hipError_t fgemm(const FGemm &p, hipStream_t s) {
    dim3 grid;
    if (GROUP == FG_M) grid = dim3((p.M + FM - 1) / FM + kE, p.N / FN);
    else if (GROUP == FG_K) grid = dim3(p.M / FM, p.N / FN, kE);
    else grid = dim3((p.M + FM - 1) / FM, p.N / FN);
    hipLaunchKernelGGL(k_fgemm<GROUP>, grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

// -------------------------------------------------------------- quantisers

// Rows of C values (C % 128 == 0; fp32, or bf16 bits when BF16_IN; row
// stride ldi) -> e4m3 per 1x128 tile: scale = the power of two at or above
// amax / 448 (1 for an all-zero tile), code = e4m3(v / scale); codes [R, C] (row stride
// ldo), E8M0 scales [R, C/128].  16 lanes per tile, 8 values per lane.
template <bool BF16_IN>
__global__ __launch_bounds__(256) void k_q8_rows(int64_t R, int C, const void *__restrict__ in, int64_t ldi,
                                                 uint8_t *__restrict__ q, int64_t ldo, uint8_t *__restrict__ sc) {
    const int tpr = C / 128;
    const int64_t tile = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
    if (tile >= R * tpr) return;  // whole 16-lane groups leave together
    const int64_t r = tile / tpr;
    const int tb = (int)(tile - r * tpr), l = threadIdx.x & 15;
    const int64_t c0 = (int64_t)tb * 128 + l * 8;
    float v[8];
    if (BF16_IN) {
        const i32x4 u = *reinterpret_cast<const i32x4 *>(static_cast<const uint16_t *>(in) + r * ldi + c0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = bf16_to_f32((uint32_t)u[i] & 0xffffu);
            v[2 * i + 1] = bf16_to_f32((uint32_t)u[i] >> 16);
        }
    } else {
        const float *src = static_cast<const float *>(in) + r * ldi + c0;
        const f32x4 a = *reinterpret_cast<const f32x4 *>(src), b = *reinterpret_cast<const f32x4 *>(src + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[i] = a[i];
            v[4 + i] = b[i];
        }
    }
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
#pragma unroll
    for (int s = 1; s < 16; s <<= 1) m = fmaxf(m, __shfl_xor(m, s, 64));
    const float s = e4m3_tile_scale(m);
    const float inv = 1.0f / s;  // a power of two: v * inv == v / s exactly
    const uint32_t w0 = e4m3x4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
    const uint32_t w1 = e4m3x4(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
    *reinterpret_cast<uint2 *>(q + r * ldo + c0) = uint2{w0, w1};
    if (l == 0) sc[r * tpr + tb] = (uint8_t)e8m0_of(s);
}

// Column tiles over groups of 128 row positions.  Grouped (off != nullptr):
// group e's rows [off[e], off[e+1]) land at positions poff[e] + (r - off[e])
// and the positions up to poff[e+1] are zeros; plain: rows [0, R) at their
// own positions, zeros up to Rp.  Every (column, 128 positions) tile is
// quantised like a row tile: codes out[c*ldo + pos] (ldo % 128 == 0), scales
// sc[c*ldso + pos/128].  Source row r: fp32 in[r*ldi + c], or (BF16_IN) bf16
// row rows[r] / rdiv (or r) of in.  Workgroup: 128 positions x 64 columns;
// wave w reduces and quantises positions 32w .. 32w+31 of column c0 + lane.
template <bool BF16_IN>
__global__ __launch_bounds__(256) void k_q8_cols(int R, const void *__restrict__ in, int64_t ldi,
                                                 const int32_t *__restrict__ rows, int rdiv,
                                                 const int32_t *__restrict__ off, const int32_t *__restrict__ poff,
                                                 int Rp, uint8_t *__restrict__ out, int64_t ldo,
                                                 uint8_t *__restrict__ sc, int64_t ldso) {
    __shared__ float tile[128][65];
    __shared__ float red[4][64];
    // blockIdx.x: the 64-column block (consecutive workgroups read consecutive
    // pieces of the same rows); blockIdx.y: the 128-position slot
    const int c0 = blockIdx.x * 64, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int r0, rend, pos0;
    if (off) {
        // slot -> (group e, tile t) over sum_e ceil(c_e / 128) tiles
        int o[5], nt[4], lt = 0;
#pragma unroll
        for (int i = 0; i < 5; ++i) o[i] = off[lane * 4 + i];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            nt[i] = (o[i + 1] - o[i] + 127) / 128;
            lt += nt[i];
        }
        const int incl = wave_incl_scan(lt), excl = incl - lt;
        const int slot = blockIdx.y;
        if (slot >= __shfl(incl, 63, 64)) return;
        const bool own = slot >= excl && slot < incl;
        const int owner = __ffsll((unsigned long long)__ballot(own)) - 1;
        int my_e = 0, my_t = 0;
        if (own) {
            int q = slot - excl;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (q >= 0 && q < nt[i]) {
                    my_e = lane * 4 + i;
                    my_t = q;
                }
                q -= nt[i];
            }
        }
        const int e = __shfl(my_e, owner, 64), t = __shfl(my_t, owner, 64);
        r0 = off[e] + 128 * t;
        rend = off[e + 1];
        pos0 = poff[e] + 128 * t;
    } else {
        r0 = blockIdx.y * 128;
        if (r0 >= Rp) return;
        rend = R;
        pos0 = r0;
    }
    if (BF16_IN) {
        // 64 bf16 = 128 bytes per row: 8 threads per row, 32 rows per pass
#pragma unroll
        for (int pass = 0; pass < 4; ++pass) {
            const int rr = pass * 32 + (tid >> 3), cc = (tid & 7) * 8;
            const int r = r0 + rr;
            i32x4 u = i32x4{0, 0, 0, 0};
            if (r < rend) {
                const int64_t src = rows ? rows[r] / rdiv : r;
                u = *reinterpret_cast<const i32x4 *>(static_cast<const uint16_t *>(in) + src * ldi + c0 + cc);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                tile[rr][cc + 2 * i] = bf16_to_f32((uint32_t)u[i] & 0xffffu);
                tile[rr][cc + 2 * i + 1] = bf16_to_f32((uint32_t)u[i] >> 16);
            }
        }
    } else {
        // 64 fp32 = 256 bytes per row: 16 threads per row, 16 rows per pass
#pragma unroll
        for (int pass = 0; pass < 8; ++pass) {
            const int rr = pass * 16 + (tid >> 4), cc = (tid & 15) * 4;
            const int r = r0 + rr;
            f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
            if (r < rend) v = *reinterpret_cast<const f32x4 *>(static_cast<const float *>(in) + (int64_t)r * ldi + c0 + cc);
#pragma unroll
            for (int i = 0; i < 4; ++i) tile[rr][cc + i] = v[i];
        }
    }
    __syncthreads();
    float m = 0.f;
#pragma unroll 8
    for (int i = 0; i < 32; ++i) m = fmaxf(m, fabsf(tile[32 * wave + i][lane]));
    red[wave][lane] = m;
    __syncthreads();
    const float amax = fmaxf(fmaxf(red[0][lane], red[1][lane]), fmaxf(red[2][lane], red[3][lane]));
    const float s = e4m3_tile_scale(amax);
    const float inv = 1.0f / s;  // a power of two: v * inv == v / s exactly
    uint32_t w[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int r0 = 32 * wave + 4 * q;
        w[q] = e4m3x4(tile[r0][lane] * inv, tile[r0 + 1][lane] * inv, tile[r0 + 2][lane] * inv, tile[r0 + 3][lane] * inv);
    }
    i32x4 *o = reinterpret_cast<i32x4 *>(out + (int64_t)(c0 + lane) * ldo + pos0 + 32 * wave);
    o[0] = i32x4{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
    o[1] = i32x4{(int)w[4], (int)w[5], (int)w[6], (int)w[7]};
    if (wave == 0) sc[(int64_t)(c0 + lane) * ldso + pos0 / 128] = (uint8_t)e8m0_of(s);
}

// e4m3 codes transposed per group: out[g][c*ldo + coff + r] = in[g][r*C + c]
// (R, C multiples of 128), 128x128-byte tiles.  Thread (a = tid / 8,
// b = tid % 8) reads 16 bytes of each of rows 4a .. 4a+3 at columns
// 16b .. 16b+15 (four 16-byte loads in flight), transposes the four 4x4
// blocks in registers and puts word a of output rows 16b .. 16b+15 in LDS;
// then each output row's 128 bytes go out as eight 16-byte stores.  In LDS,
// output row c holds its 32 words with bits 3-4 of the word index flipped by
// (c / 16) % 4, so the 64 lanes of a write hit 32 distinct banks twice.
__global__ __launch_bounds__(256) void k_t8(int C, const uint8_t *__restrict__ in, int64_t gin,
                                            uint8_t *__restrict__ out, int64_t ldo, int64_t gout, int coff) {
    __shared__ __attribute__((aligned(16))) uint32_t tile[128 * 32];
    const int r0 = blockIdx.x * 128, c0 = blockIdx.y * 128, g = blockIdx.z, tid = threadIdx.x;
    in += (int64_t)g * gin;
    out += (int64_t)g * gout;
    {
        // eight consecutive threads take one row's whole 128 bytes, so each
        // load instruction reads eight full lines
        const int a = tid >> 3, b = tid & 7;
        i32x4 v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            v[i] = *reinterpret_cast<const i32x4 *>(in + (int64_t)(r0 + 4 * a + i) * C + c0 + 16 * b);
        const int sw = 8 * (b & 3);  // output rows 16b .. 16b+15 share (c / 16) % 4 = b % 4
#pragma unroll
        for (int sblk = 0; sblk < 4; ++sblk)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                // byte j of the four rows' word sblk: output row 16b + 4 sblk + j, rows 4a .. 4a+3
                const uint32_t w = (((uint32_t)v[0][sblk] >> (8 * j)) & 0xffu) |
                                   ((((uint32_t)v[1][sblk] >> (8 * j)) & 0xffu) << 8) |
                                   ((((uint32_t)v[2][sblk] >> (8 * j)) & 0xffu) << 16) |
                                   ((((uint32_t)v[3][sblk] >> (8 * j)) & 0xffu) << 24);
                tile[(16 * b + 4 * sblk + j) * 32 + (a ^ sw)] = w;
            }
    }
    __syncthreads();
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
        const int c = 32 * pass + (tid >> 3), q = tid & 7;
        const i32x4 v = *reinterpret_cast<const i32x4 *>(&tile[c * 32 + ((4 * q) ^ (8 * ((c >> 4) & 3)))]);
        *reinterpret_cast<i32x4 *>(out + (int64_t)(c0 + c) * ldo + coff + r0 + 16 * q) = v;
    }
}

// Block scales transposed per group: out[g][cb*ldo + coff + rb] = in[g][rb*Cb + cb].
__global__ __launch_bounds__(256) void k_tscale(int Rb, int Cb, const uint8_t *__restrict__ in,
                                                uint8_t *__restrict__ out, int ldo, int coff) {
    const int g = blockIdx.y, i = blockIdx.x * 256 + threadIdx.x;
    if (i >= Rb * Cb) return;
    const int rb = i / Cb, cb = i - rb * Cb;
    out[(int64_t)g * Cb * ldo + (int64_t)cb * ldo + coff + rb] = in[(int64_t)g * Rb * Cb + i];
}

hipError_t t8(int R, int C, int G, const void *in, uint8_t *out, int64_t ldo, int coff, hipStream_t s) {
    if (R % 128 != 0 || C % 128 != 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_t8, dim3(R / 128, C / 128, G), dim3(256), 0, s, C, static_cast<const uint8_t *>(in),
                       (int64_t)R * C, out, ldo, (int64_t)C * ldo, coff);
    return hipGetLastError();
}

hipError_t tscale(int R, int C, int G, const uint8_t *in, uint8_t *out, int ldo, int coff, hipStream_t s) {
    const int n = (R / 128) * (C / 128);
    hipLaunchKernelGGL(k_tscale, dim3((n + 255) / 256, G), dim3(256), 0, s, R / 128, C / 128, in, out, ldo, coff);
    return hipGetLastError();
}

template <bool BF16_IN>
hipError_t q8_rows(int64_t R, int C, const void *in, int64_t ldi, uint8_t *q, uint8_t *sc, hipStream_t s) {
    const int64_t tiles = R * (C / 128);
    hipLaunchKernelGGL(k_q8_rows<BF16_IN>, dim3((unsigned)((tiles + 15) / 16)), dim3(256), 0, s, R, C, in, ldi, q,
                       (int64_t)C, sc);
    return hipGetLastError();
}

// Column tiles of C columns: grouped over `off` (the 256 experts' rows) into
// [C, Rp] at the 128-aligned positions poff, or plain rows [0, R) into [C, Rp].
template <bool BF16_IN>
hipError_t q8_cols(int R, int C, const void *in, int64_t ldi, const int32_t *rows, int rdiv, const int32_t *off,
                   const int32_t *poff, int64_t Rp, uint8_t *out, uint8_t *sc, hipStream_t s) {
    const int slots = off ? R / 128 + kE + 1 : (int)(Rp / 128);
    if (slots > 65535) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_q8_cols<BF16_IN>, dim3(C / 64, slots), dim3(256), 0, s, R, in, ldi, rows, rdiv, off, poff,
                       (int)Rp, out, Rp, sc, Rp / 128);
    return hipGetLastError();
}

// The workspace, carved in a fixed order (base == nullptr: sizes only).
struct Bw8 {
    uint8_t *xq, *dyq, *dabq;                 // row-quantised: [T, d], [R, d], [R, 2I]
    uint8_t *xqs, *dyqs, *dabqs;              //   their E8M0 scales
    float *dyo, *P, *dh, *h, *dab, *dxi;      // fp32 rows [R, *] (routed rows, then T shared rows)
    float *dl, *dg, *dwr_part;
    int32_t *poff;
    uint8_t *wdT, *wguT, *sdT, *sguT;         // transposed weights
    uint8_t *wdTs, *wguTs, *sdTs, *sguTs;     //   their block scales
    uint8_t *xT, *dyT, *hT, *dabT;            // column-quantised [*, Rp]
    uint8_t *xTs, *dyTs, *hTs, *dabTs;
    uint8_t *xsT, *dysT, *hsT, *dabsT;        // shared expert: [*, Tp]
    uint8_t *xsTs, *dysTs, *hsTs, *dabsTs;
    size_t bytes;
};

Bw8 carve8(char *base, int T, int d, int I, int k) {
    Bw8 w{};
    size_t o = 0;
    const size_t A = (size_t)T * k, R = A + T, Rp = A + 128 * (size_t)kE, Tp = ((size_t)T + 127) / 128 * 128;
    const size_t E = kE;
    auto take = [&](size_t n) -> char * {
        char *p = base ? base + o : nullptr;
        o += (n + 255) / 256 * 256;
        return p;
    };
    auto u8 = [&](size_t n) { return reinterpret_cast<uint8_t *>(take(n)); };
    auto f32 = [&](size_t n) { return reinterpret_cast<float *>(take(n * 4)); };
    w.xq = u8((size_t)T * d);
    w.xqs = u8((size_t)T * d / 128);
    w.dyq = u8(R * d);
    w.dyqs = u8(R * d / 128);
    w.dabq = u8(R * 2 * I);
    w.dabqs = u8(R * 2 * I / 128);
    w.dyo = f32(R * d);
    w.P = f32(R * 2 * I);
    w.dh = f32(R * I);
    w.h = f32(R * I);
    w.dab = f32(R * 2 * I);
    w.dxi = f32(R * d);
    w.dl = f32(A);
    w.dg = f32(A);
    w.dwr_part = reinterpret_cast<float *>(take(bwd::dwr_part_bytes(d)));
    w.poff = reinterpret_cast<int32_t *>(take((E + 1) * 4));
    w.wdT = u8(E * I * d);
    w.wdTs = u8(E * (I / 128) * (d / 128));
    w.wguT = u8(E * d * 2 * I);
    w.wguTs = u8(E * (d / 128) * (2 * I / 128));
    w.sdT = u8((size_t)I * d);
    w.sdTs = u8((size_t)(I / 128) * (d / 128));
    w.sguT = u8((size_t)d * 2 * I);
    w.sguTs = u8((size_t)(d / 128) * (2 * I / 128));
    w.xT = u8(d * Rp);
    w.xTs = u8(d * Rp / 128);
    w.dyT = u8(d * Rp);
    w.dyTs = u8(d * Rp / 128);
    w.hT = u8(I * Rp);
    w.hTs = u8(I * Rp / 128);
    w.dabT = u8(2 * I * Rp);
    w.dabTs = u8(2 * I * Rp / 128);
    w.xsT = u8(d * Tp);
    w.xsTs = u8(d * Tp / 128);
    w.dysT = u8(d * Tp);
    w.dysTs = u8(d * Tp / 128);
    w.hsT = u8(I * Tp);
    w.hsTs = u8(I * Tp / 128);
    w.dabsT = u8(2 * I * Tp);
    w.dabsTs = u8(2 * I * Tp / 128);
    w.bytes = o;
    return w;
}

}  // namespace

size_t backward_fp8_ws_bytes(int T, int d, int I, int k) { return carve8(nullptr, T, d, I, k).bytes; }

hipError_t launch_backward_fp8(const BackwardArgs &a, void *ws, hipStream_t s) {
    const int T = a.T, d = a.d, I = a.I, k = a.k;
    const int A = T * k;
    const int64_t Rp = (int64_t)A + 128 * kE, Tp = ((int64_t)T + 127) / 128 * 128;
    const Bw8 w = carve8(static_cast<char *>(ws), T, d, I, k);
    float *dg = a.dg ? a.dg : w.dg;
    const uint16_t *x = static_cast<const uint16_t *>(a.x);
    const FfnWeights &ex = a.experts, &sh = a.shared;
    // rows A .. A+T of the row buffers are the shared expert's (token order)
    float *dys = w.dyo + (int64_t)A * d, *Ps = w.P + (int64_t)A * 2 * I, *dhs = w.dh + (int64_t)A * I;
    float *hs = w.h + (int64_t)A * I, *dabs = w.dab + (int64_t)A * 2 * I, *dxs = w.dxi + (int64_t)A * d;
    hipError_t e;
#define CHK(call)                      \
    if ((e = (call)) != hipSuccess) return e;

    // 0. 128-aligned row positions; weights transposed as 128x128 blocks
    CHK(bwd::pad_offsets(a.offsets, w.poff, 128, s));
    CHK(t8(d, I, kE, ex.down, w.wdT, d, 0, s));                        // [E, I, d]
    CHK(tscale(d, I, kE, ex.s_down, w.wdTs, d / 128, 0, s));
    CHK(t8(I, d, kE, ex.gate, w.wguT, 2 * I, 0, s));                   // [E, d, 2I]: gate | up
    CHK(t8(I, d, kE, ex.up, w.wguT, 2 * I, I, s));
    CHK(tscale(I, d, kE, ex.s_gate, w.wguTs, 2 * I / 128, 0, s));
    CHK(tscale(I, d, kE, ex.s_up, w.wguTs, 2 * I / 128, I / 128, s));
    CHK(t8(d, I, 1, sh.down, w.sdT, d, 0, s));
    CHK(tscale(d, I, 1, sh.s_down, w.sdTs, d / 128, 0, s));
    CHK(t8(I, d, 1, sh.gate, w.sguT, 2 * I, 0, s));
    CHK(t8(I, d, 1, sh.up, w.sguT, 2 * I, I, s));
    CHK(tscale(I, d, 1, sh.s_gate, w.sguTs, 2 * I / 128, 0, s));
    CHK(tscale(I, d, 1, sh.s_up, w.sguTs, 2 * I / 128, I / 128, s));

    // 1. combine backward (fp32 output gradients) and x per 1x128 tile of d
    CHK(bwd::combine(T, d, a.dy, static_cast<const uint16_t *>(a.y_perm), a.row_of, a.weights, w.dyo, dys, dg, true,
                     s));
    CHK(q8_rows<true>(T, d, x, d, w.xq, w.xqs, s));

    FGemm base{};
    base.bdiv = 128;
    // M-grouped (routed) or plain products with row-quantised A and
    // block-scaled B: the forward's persistent e4m3 kernel when the shape
    // fits it, else k_fgemm
    auto mg = [&](const FGemm &p, bool routed) -> hipError_t {
        Fp8GemmArgs g{};
        g.M = p.M; g.offsets = routed ? p.offsets : nullptr; g.A = p.A; g.As = p.As; g.a_rows = p.a_rows;
        g.a_div = p.a_div; g.a_src_rows = T; g.K = p.K; g.B = p.B; g.Bs = p.Bs; g.N = p.N; g.out = p.C; g.ldo = (int)p.ldc;
        if (p.lda == p.K && p.ldas == p.K / FK && p.ldb == p.K && p.ldbs == p.K / FK && p.bdiv == 128 &&
            (!routed || (p.bstride == (int64_t)p.N * p.K && p.bsstride == (int64_t)(p.N / 128) * (p.K / FK))) &&
            fp8_mx_gemm_ok(g))
            return launch_fp8_mx_gemm(g, s);
        return routed ? fgemm<FG_M>(p, s) : fgemm<FG_NONE>(p, s);
    };
    // 2. pre-activations, as the forward forms them: routed rows gather the
    //    quantised x through row_src; gate into columns 0..I, up into I..2I
    for (int half = 0; half < 2; ++half) {
        FGemm p = base;
        p.M = A; p.N = I; p.K = d; p.offsets = a.offsets;
        p.A = w.xq; p.lda = d; p.As = w.xqs; p.ldas = d / 128; p.a_rows = a.row_src; p.a_div = k;
        p.B = static_cast<const uint8_t *>(half ? ex.up : ex.gate); p.ldb = d; p.bstride = (int64_t)I * d;
        p.Bs = half ? ex.s_up : ex.s_gate; p.ldbs = d / 128; p.bsstride = (int64_t)(I / 128) * (d / 128);
        p.C = w.P + (half ? I : 0); p.ldc = 2 * I;
        CHK(mg(p, true));
        FGemm q = p;
        q.M = T; q.offsets = nullptr; q.a_rows = nullptr; q.a_div = 1;
        q.B = static_cast<const uint8_t *>(half ? sh.up : sh.gate); q.Bs = half ? sh.s_up : sh.s_gate;
        q.C = Ps + (half ? I : 0);
        CHK(mg(q, false));
    }
    // 3. dh = Q(output gradient) W_down: rows per 1x128 tile of d; W_down as [E, I, d] blocks
    CHK(q8_rows<false>((int64_t)A + T, d, w.dyo, d, w.dyq, w.dyqs, s));
    {
        FGemm p = base;
        p.M = A; p.N = I; p.K = d; p.offsets = a.offsets;
        p.A = w.dyq; p.lda = d; p.As = w.dyqs; p.ldas = d / 128; p.a_div = 1;
        p.B = w.wdT; p.ldb = d; p.bstride = (int64_t)I * d;
        p.Bs = w.wdTs; p.ldbs = d / 128; p.bsstride = (int64_t)(I / 128) * (d / 128);
        p.C = w.dh; p.ldc = I;
        CHK(mg(p, true));
        FGemm q = p;
        q.M = T; q.offsets = nullptr; q.A = w.dyq + (int64_t)A * d; q.As = w.dyqs + (int64_t)A * (d / 128);
        q.B = w.sdT; q.Bs = w.sdTs; q.C = dhs;
        CHK(mg(q, false));
    }
    // 4. SwiGLU backward in fp32 (routed and shared rows in one pass)
    CHK(bwd::swiglu((int64_t)A + T, I, w.P, w.dh, w.h, w.dab, true, s));
    // 5. input gradients: Q(da | db) per 1x128 tile of I, against (W_gate | W_up) as [E, d, 2I] blocks
    CHK(q8_rows<false>((int64_t)A + T, 2 * I, w.dab, 2 * I, w.dabq, w.dabqs, s));
    {
        FGemm p = base;
        p.M = A; p.N = d; p.K = 2 * I; p.offsets = a.offsets;
        p.A = w.dabq; p.lda = 2 * I; p.As = w.dabqs; p.ldas = 2 * I / 128; p.a_div = 1;
        p.B = w.wguT; p.ldb = 2 * I; p.bstride = (int64_t)d * 2 * I;
        p.Bs = w.wguTs; p.ldbs = 2 * I / 128; p.bsstride = (int64_t)(d / 128) * (2 * I / 128);
        p.C = w.dxi; p.ldc = d;
        CHK(mg(p, true));
        FGemm q = p;
        q.M = T; q.offsets = nullptr; q.A = w.dabq + (int64_t)A * 2 * I; q.As = w.dabqs + (int64_t)A * (2 * I / 128);
        q.B = w.sguT; q.Bs = w.sguTs; q.C = dxs;
        CHK(mg(q, false));
    }
    // 6. weight gradients: every operand column-quantised over 128-row groups
    //    of the expert's rows (positions poff), then K-grouped GEMMs
    CHK(q8_cols<true>(A, d, x, d, a.row_src, k, a.offsets, w.poff, Rp, w.xT, w.xTs, s));
    CHK(q8_cols<false>(A, d, w.dyo, d, nullptr, 1, a.offsets, w.poff, Rp, w.dyT, w.dyTs, s));
    CHK(q8_cols<false>(A, I, w.h, I, nullptr, 1, a.offsets, w.poff, Rp, w.hT, w.hTs, s));
    CHK(q8_cols<false>(A, 2 * I, w.dab, 2 * I, nullptr, 1, a.offsets, w.poff, Rp, w.dabT, w.dabTs, s));
    // K-grouped products (row scales on both operands): the persistent e4m3
    // kernel's K-grouped form when the shape fits it (it skips empty groups,
    // which are zeroed here), else k_fgemm
    auto kg = [&](const FGemm &p, bool grouped) -> hipError_t {
        Fp8KgArgs g{};
        g.M = p.M; g.N = p.N; g.K = p.K; g.kseg = grouped ? p.offsets : nullptr; g.A = p.A; g.As = p.As;
        g.B = p.B; g.Bs = p.Bs; g.out = p.C; g.ldo = (int)p.ldc; g.cstride = p.cstride;
        if (p.lda == p.K && p.ldb == p.K && p.ldas == p.K / FK && p.ldbs == p.K / FK && fp8_mx_kg_ok(g)) {
            const hipError_t r = launch_fp8_mx_kg(g, s);
            if (r != hipSuccess || !grouped) return r;
            return bwd::zero_empty((int64_t)p.M * p.ldc, p.offsets, p.C, s);
        }
        return grouped ? fgemm<FG_K>(p, s) : fgemm<FG_NONE>(p, s);
    };
    {
        FGemm p{};
        p.K = (int)Rp; p.offsets = w.poff; p.lda = Rp; p.ldas = Rp / 128; p.a_div = 1; p.ldb = Rp; p.ldbs = Rp / 128;
        p.bdiv = 1;
        // dW_gate[e] = Q(da)^T Q(x), dW_up[e] = Q(db)^T Q(x): [I, d]
        p.M = I; p.N = d; p.B = w.xT; p.Bs = w.xTs; p.ldc = d; p.cstride = (int64_t)I * d;
        p.A = w.dabT; p.As = w.dabTs; p.C = a.dw_gate;
        CHK(kg(p, true));
        p.A = w.dabT + (int64_t)I * Rp; p.As = w.dabTs + (int64_t)I * (Rp / 128); p.C = a.dw_up;
        CHK(kg(p, true));
        // dW_down[e] = Q(output gradient)^T Q(h): [d, I]
        p.M = d; p.N = I; p.A = w.dyT; p.As = w.dyTs; p.B = w.hT; p.Bs = w.hTs; p.ldc = I; p.cstride = (int64_t)d * I;
        p.C = a.dw_down;
        CHK(kg(p, true));
    }
    // the shared expert: its T rows in token order, groups of 128 tokens
    CHK(q8_cols<true>(T, d, x, d, nullptr, 1, nullptr, nullptr, Tp, w.xsT, w.xsTs, s));
    CHK(q8_cols<false>(T, d, dys, d, nullptr, 1, nullptr, nullptr, Tp, w.dysT, w.dysTs, s));
    CHK(q8_cols<false>(T, I, hs, I, nullptr, 1, nullptr, nullptr, Tp, w.hsT, w.hsTs, s));
    CHK(q8_cols<false>(T, 2 * I, dabs, 2 * I, nullptr, 1, nullptr, nullptr, Tp, w.dabsT, w.dabsTs, s));
    {
        FGemm p{};
        p.K = (int)Tp; p.lda = Tp; p.ldas = Tp / 128; p.a_div = 1; p.ldb = Tp; p.ldbs = Tp / 128; p.bdiv = 1;
        p.M = I; p.N = d; p.B = w.xsT; p.Bs = w.xsTs; p.ldc = d;
        p.A = w.dabsT; p.As = w.dabsTs; p.C = a.ds_gate;
        CHK(kg(p, false));
        p.A = w.dabsT + (int64_t)I * Tp; p.As = w.dabsTs + (int64_t)I * (Tp / 128); p.C = a.ds_up;
        CHK(kg(p, false));
        p.M = d; p.N = I; p.A = w.dysT; p.As = w.dysTs; p.B = w.hsT; p.Bs = w.hsTs; p.ldc = I; p.C = a.ds_down;
        CHK(kg(p, false));
    }
    // 7. router (fp32): dl and its share of dx, then the router gradient
    CHK(bwd::router(T, d, x, a.w_router, a.idx, dg, w.dl, a.dx, s));
    CHK(bwd::dwr(d, a.offsets, a.row_src, w.dl, x, w.dwr_part, a.dw_router, s));
    // 8. dx += shared + routed input gradients
    CHK(bwd::dx(T, d, dxs, w.dxi, a.row_of, a.dx, s));
#undef CHK
    return hipSuccess;
}

}  // namespace moe
