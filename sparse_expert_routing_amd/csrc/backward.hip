// Backward of the MoE layer (bf16 experts): gradients of the layer output
// for the routing the forward chose.
//
// What is differentiated: DeepSeek V3 From Scratch, "The idea" and "In code"
// (sigmoid affinities, top-8 by biased score, combine weights = the chosen
// unbiased affinities renormalised); Scaling Efficiency: A Deep Dive into the
// DeepSeek-V3 Architecture, "Implementation: A Modular Look" (shared output
// plus the weighted routed outputs).  The choice is piecewise constant and
// carries no gradient; the bias enters only the choice, so it gets none
// (kbwen.com DeepSeek feed, "A bias term for each expert": the bias adds no
// gradient of its own).
//
// Kernels:
//   - k_transpose: weights, and the rows each expert's weight gradient
//     reduces over, transposed through LDS tiles so every GEMM below reads
//     both operands K-contiguous; an expert's rows start at a 32-aligned
//     position and are zero-padded to it;
//   - the data-gradient GEMMs and the pre-activation recompute (NT, grouped
//     over the experts' rows): the forward's persistent 256x256-tile kernel
//     with an fp32 epilogue, or k_bgemm for small groups;
//   - k_bgemm: a grouped GEMM C = A B on v_mfma_f32_32x32x16_bf16 with fp32
//     accumulation, 128x128 tiles, 32 of K per stage, register-staged double
//     buffer in LDS; groups split M (B per expert) or K (an expert's padded
//     rows are the reduction: the weight gradients, C per expert);
//   - k_bwd_combine: per token, dg_j = dy . y_perm_j, the routed output
//     gradient g_j dy (bf16) and the shared one dy (bf16);
//   - k_bwd_swiglu: h, and the SwiGLU input gradients from the recomputed
//     pre-activations (all rounded to bf16 as the forward rounds h);
//   - k_bwd_router: per token, the chosen experts' affinities recomputed in
//     fp32, ds_j = (dg_j - sum_i g_i dg_i) / sum_i s_i, dl_j = ds_j s_j (1-s_j),
//     and the router's share of dx;
//   - k_bwd_dwr / k_bwd_dwr_sum: router weight gradient, each expert's rows
//     summed in 16 ordered shares, the shares added in order;
//   - k_bwd_dx: dx += shared input gradient + sum_j routed input gradients.
#include "backward.h"
#include "device.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kE = 256;
constexpr int GM = 128, GN = 128, GK = 32;
constexpr int LDK = GK + 8;  // LDS row stride (elements): 80 bytes

enum { GROUP_NONE = 0, GROUP_M = 1, GROUP_K = 2 };

struct BGemm {
    int M, N, K;              // K: the reduction length (GROUP_K: total rows)
    const int32_t *offsets;   // [G+1] (GROUP_M: row ranges; GROUP_K: reduction ranges)
    const uint16_t *A;        // A(m, k) = A[m*lda + k]
    int64_t lda;
    const int32_t *a_rows;    // optional: row m reads row a_rows[m] / a_div
    int a_div;
    const uint16_t *B;        // B(k, n) = B[n*ldb + k]
    int64_t ldb, bstride;     // bstride: per-group B offset (GROUP_M)
    float *C;                 // C[m*ldc + n] (+ cstride per group for GROUP_K)
    int64_t ldc, cstride;
};

// Row-tile slot -> (group, first row, end row) for GROUP_M (all lanes agree).
__device__ __forceinline__ bool bg_find_tile(const int32_t *__restrict__ offsets, int slot, int &gi, int &m0,
                                             int &m_end) {
    const int lane = threadIdx.x & 63;
    const int base = lane * 4;
    int off[5];
#pragma unroll
    for (int i = 0; i < 5; ++i) off[i] = offsets[base + i];
    int nt[4], lane_t = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        nt[i] = (off[i + 1] - off[i] + GM - 1) / GM;
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
        int s = slot - excl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (s >= 0 && s < nt[i]) {
                my_g = base + i;
                my_m0 = off[i] + s * GM;
                my_end = off[i + 1];
            }
            s -= nt[i];
        }
    }
    gi = __shfl(my_g, owner, 64);
    m0 = __shfl(my_m0, owner, 64);
    m_end = __shfl(my_end, owner, 64);
    return true;
}

// One operand tile (128 rows of M or N x 32 of K, K-contiguous) global ->
// registers -> LDS: two 16-byte pieces per thread.  Rows past `rows_end`
// read as zeros; row r reads source row rows[r] / rdiv when rows is given.
struct TileLoad {
    i32x4 v[2];
    __device__ __forceinline__ void load(const uint16_t *__restrict__ P, int64_t ld, const int32_t *__restrict__ rows,
                                         int rdiv, int r0, int rows_end, int k0) {
        const int tid = threadIdx.x;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int c = tid + 256 * h;
            const int row = c >> 2, kc = (c & 3) * 8;
            const int gr = r0 + row;
            v[h] = i32x4{0, 0, 0, 0};
            if (gr < rows_end) {
                const int64_t src = rows ? rows[gr] / rdiv : gr;
                v[h] = *reinterpret_cast<const i32x4 *>(P + src * ld + k0 + kc);
            }
        }
    }
    __device__ __forceinline__ void store(uint16_t *__restrict__ S) const {
        const int tid = threadIdx.x;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int c = tid + 256 * h;
            const int row = c >> 2, kc = (c & 3) * 8;
            *reinterpret_cast<i32x4 *>(S + row * LDK + kc) = v[h];
        }
    }
};

template <int GROUP, bool ACC>
__global__ __launch_bounds__(256) void k_bgemm(BGemm p) {
    __shared__ __attribute__((aligned(16))) uint16_t sA[2][GM * LDK];
    __shared__ __attribute__((aligned(16))) uint16_t sB[2][GN * LDK];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    int gi = 0, m0, m_end, k_begin = 0, k_end = p.K;
    const int n0 = blockIdx.y * GN;
    if (GROUP == GROUP_M) {
        if (!bg_find_tile(p.offsets, blockIdx.x, gi, m0, m_end)) return;
    } else {
        m0 = blockIdx.x * GM;
        m_end = p.M;
        if (GROUP == GROUP_K) {
            gi = blockIdx.z;
            k_begin = p.offsets[gi];
            k_end = p.offsets[gi + 1];
        }
    }
    const uint16_t *B = p.B + (GROUP == GROUP_M ? (int64_t)gi * p.bstride : 0);
    float *C = p.C + (GROUP == GROUP_K ? (int64_t)gi * p.cstride : 0);

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

    TileLoad la, lb;
    // A rows: M (row indirection only for a K-contiguous A); B: N, with the
    // row indirection on K for an N-contiguous B
    const int nst = (k_end - k_begin + GK - 1) / GK;
    if (nst > 0) {
        la.load(p.A, p.lda, p.a_rows, p.a_div, m0, m_end, k_begin);
        lb.load(B, p.ldb, nullptr, 1, n0, p.N, k_begin);
        la.store(sA[0]);
        lb.store(sB[0]);
    }
    __syncthreads();
    for (int st = 0; st < nst; ++st) {
        const int buf = st & 1;
        const bool more = st + 1 < nst;
        if (more) {
            const int k0 = k_begin + (st + 1) * GK;
            la.load(p.A, p.lda, p.a_rows, p.a_div, m0, m_end, k0);
            lb.load(B, p.ldb, nullptr, 1, n0, p.N, k0);
        }
#pragma unroll
        for (int ks = 0; ks < GK / 16; ++ks) {
            const int kc = ks * 16 + (lane >> 5) * 8;
            bf16x8 af[2], bfr[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                af[i] = *reinterpret_cast<const bf16x8 *>(&sA[buf][(wm * 64 + i * 32 + (lane & 31)) * LDK + kc]);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                bfr[j] = *reinterpret_cast<const bf16x8 *>(&sB[buf][(wn * 64 + j * 32 + (lane & 31)) * LDK + kc]);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        if (more) {
            la.store(sA[buf ^ 1]);
            lb.store(sB[buf ^ 1]);
        }
        __syncthreads();
    }
    // C layout of a 32x32 block: lane holds column (lane & 31), rows
    // 8q + 4(lane >> 5) + r in register 4q + r
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = m0 + wm * 64 + i * 32 + 8 * q + 4 * (lane >> 5) + r;
                if (row >= m_end) continue;
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int col = n0 + wn * 64 + j * 32 + (lane & 31);
                    float *c = C + (int64_t)row * p.ldc + col;
                    const float v = acc[i][j][4 * q + r];
                    *c = ACC ? *c + v : v;
                }
            }
}

// ------------------------------------------------------------- transposes

// out[g][c*ldo + coff + pos] = in[g][src(r)*ldi + c], bf16, through 64x64
// LDS tiles (both sides coalesced; 8-byte stores).  src(r) = rows[r] / rdiv
// (a row gather) or r.  Grouped (off != nullptr): the tiles run over each
// group's rows [off[e], off[e+1]) and row r of group e lands at
// pos = poff[e] + r - off[e]; positions up to poff[e+1] past the group's rows
// are written as zeros (the padding).  Plain: pos = r for r < R, and zeros
// for R <= pos < dend.
__global__ __launch_bounds__(256) void k_transpose(int R, const uint16_t *__restrict__ in, int64_t ldi,
                                                   int64_t gin, const int32_t *__restrict__ rows, int rdiv,
                                                   const int32_t *__restrict__ off, const int32_t *__restrict__ poff,
                                                   int dend_plain, uint16_t *__restrict__ out, int64_t ldo,
                                                   int64_t gout, int coff) {
    __shared__ uint16_t tile[64][66];
    // blockIdx.x: the 64-column block (consecutive workgroups read consecutive
    // pieces of the same rows); blockIdx.y: the row tile or slot
    const int c0 = blockIdx.x * 64, g = blockIdx.z;
    const int tid = threadIdx.x;
    int r0, rend, d0, dend;
    if (off) {
        // slot -> (group e, tile t) over sum_e ceil(c_e / 64) tiles (one wave's scan)
        const int lane = tid & 63;
        int o[5], nt[4], lt = 0;
#pragma unroll
        for (int i = 0; i < 5; ++i) o[i] = off[lane * 4 + i];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            nt[i] = (o[i + 1] - o[i] + 63) / 64;
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
        r0 = off[e] + 64 * t;
        rend = off[e + 1];
        d0 = poff[e] + 64 * t;
        dend = min(d0 + 64, poff[e + 1]);
    } else {
        r0 = blockIdx.y * 64;
        rend = R;
        d0 = r0;
        dend = min(d0 + 64, dend_plain);
        if (d0 >= dend) return;
    }
    in += (int64_t)g * gin;
    out += (int64_t)g * gout;
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
        const int rr = pass * 16 + (tid >> 4), cc = (tid & 15) * 4;
        const int r = r0 + rr;
        uint2 v = uint2{0u, 0u};
        if (r < rend) {
            const int64_t src = rows ? rows[r] / rdiv : r;
            v = *reinterpret_cast<const uint2 *>(in + src * ldi + c0 + cc);
        }
        tile[rr][cc] = (uint16_t)(v.x & 0xffffu);
        tile[rr][cc + 1] = (uint16_t)(v.x >> 16);
        tile[rr][cc + 2] = (uint16_t)(v.y & 0xffffu);
        tile[rr][cc + 3] = (uint16_t)(v.y >> 16);
    }
    __syncthreads();
    // 64 output rows (columns c) x 16 runs of 4 positions, one 8-byte store per run
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
        const int cc = pass * 16 + (tid >> 4), rq = (tid & 15) * 4;
        const int pos = d0 + rq;
        uint16_t *o = out + (int64_t)(c0 + cc) * ldo + coff + pos;
        if (pos + 3 < dend) {
            uint2 v;
            v.x = (uint32_t)tile[rq][cc] | ((uint32_t)tile[rq + 1][cc] << 16);
            v.y = (uint32_t)tile[rq + 2][cc] | ((uint32_t)tile[rq + 3][cc] << 16);
            *reinterpret_cast<uint2 *>(o) = v;
        } else {
            for (int i = 0; i < 4 && pos + i < dend; ++i) o[i] = tile[rq + i][cc];
        }
    }
}

// Padded row positions: poff = exclusive scan of the group sizes rounded up
// to ALIGN (one wave; 256 groups, 4 per lane).
template <int ALIGN>
__global__ __launch_bounds__(64) void k_pad_offsets(const int32_t *__restrict__ off, int32_t *__restrict__ poff) {
    const int lane = threadIdx.x;
    int c[4], s = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = lane * 4 + i;
        c[i] = (off[e + 1] - off[e] + ALIGN - 1) / ALIGN * ALIGN;
        s += c[i];
    }
    const int incl = wave_incl_scan(s);
    int run = incl - s;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        poff[lane * 4 + i] = run;
        run += c[i];
    }
    if (lane == 63) poff[kE] = incl;
}

// ------------------------------------------------------------ elementwise

// out[e] = 0 (per elements each, per % 4 == 0) for the groups with no rows,
// in 16-byte stores.
__global__ __launch_bounds__(256) void k_zero_empty(int64_t per, const int32_t *__restrict__ off,
                                                    float *__restrict__ out) {
    const int e = blockIdx.y;
    if (off[e + 1] > off[e]) return;
    f32x4 *o = reinterpret_cast<f32x4 *>(out + (int64_t)e * per);
    const int64_t n4 = per / 4;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256)
        o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// Stores two consecutive fp32 values as bf16 or fp32.
template <bool F32>
__device__ __forceinline__ void put2(void *base, int64_t i, float a, float b) {
    if (F32) *reinterpret_cast<float2 *>(static_cast<float *>(base) + i) = float2{a, b};
    else *reinterpret_cast<uint32_t *>(static_cast<uint16_t *>(base) + i) = pack_bf16x2(a, b);
}

// Per token t (one wave): dg_j = sum_n dy[t,n] y_perm[r_j,n] (r_j =
// row_of[t*k+j]); dyp[r_j] = g_j dy[t]; dys[t] = dy[t] (bf16, or fp32 when F32).
template <bool F32>
__global__ __launch_bounds__(256) void k_bwd_combine(int T, int d, const float *__restrict__ dy,
                                                     const uint16_t *__restrict__ y_perm,
                                                     const int32_t *__restrict__ row_of, const float *__restrict__ g,
                                                     void *__restrict__ dyp, void *__restrict__ dys,
                                                     float *__restrict__ dg) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const float *dyt = dy + (int64_t)t * d;
    int r[8];
    float gw[8], dot[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        r[j] = row_of[(int64_t)t * 8 + j];
        gw[j] = g[(int64_t)t * 8 + j];
        dot[j] = 0.f;
    }
    for (int n = lane * 2; n < d; n += 128) {
        const float2 v = *reinterpret_cast<const float2 *>(dyt + n);
        put2<F32>(dys, (int64_t)t * d + n, v.x, v.y);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t yp = *reinterpret_cast<const uint32_t *>(y_perm + (int64_t)r[j] * d + n);
            dot[j] += v.x * bf16_to_f32(yp & 0xffffu) + v.y * bf16_to_f32(yp >> 16);
            put2<F32>(dyp, (int64_t)r[j] * d + n, gw[j] * v.x, gw[j] * v.y);
        }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        float v = dot[j];
#pragma unroll
        for (int s = 32; s >= 1; s >>= 1) v += __shfl_xor(v, s, 64);
        if (lane == j) dg[(int64_t)t * 8 + j] = v;
    }
}

// From the pre-activations P [rows, 2I] (gate | up, fp32) and dh [rows, I]:
// h = silu(a) b [rows, I], and dab [rows, 2I] = (da | db) with
// da = dh b sig(a) (1 + a (1 - sig(a))), db = dh silu(a); stored as bf16, or
// fp32 when F32.
template <bool F32>
__device__ __forceinline__ void put1(void *base, int64_t i, float v) {
    if (F32) static_cast<float *>(base)[i] = v;
    else static_cast<uint16_t *>(base)[i] = (uint16_t)f32_to_bf16(v);
}

template <bool F32>
__global__ __launch_bounds__(256) void k_bwd_swiglu(int64_t n, int I, const float *__restrict__ P,
                                                    const float *__restrict__ dh, void *__restrict__ h,
                                                    void *__restrict__ dab) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const int64_t row = i / I, c = i - row * I;
    const float a = P[row * 2 * I + c], b = P[row * 2 * I + I + c], g = dh[i];
    const float sg = 1.0f / (1.0f + expf(-a));
    put1<F32>(h, i, a * sg * b);
    put1<F32>(dab, row * 2 * I + c, g * b * sg * (1.0f + a * (1.0f - sg)));
    put1<F32>(dab, row * 2 * I + I + c, g * a * sg);
}

// Per token t (one workgroup): s_j = sigmoid(x_t . wr_{e_j}) in fp32, then
// ds_j, dl_j (stored) and dx[t] = sum_j dl_j wr_{e_j} (written).
__global__ __launch_bounds__(256) void k_bwd_router(int d, const uint16_t *__restrict__ x,
                                                    const float *__restrict__ wr, const int32_t *__restrict__ idx,
                                                    const float *__restrict__ dg, float *__restrict__ dl,
                                                    float *__restrict__ dx) {
    __shared__ float part[4][8];
    __shared__ float dls[8];
    const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint16_t *xt = x + (int64_t)t * d;
    int e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = idx[(int64_t)t * 8 + j];
    float l[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) l[j] = 0.f;
    for (int n = tid; n < d; n += 256) {
        const float xv = bf16_to_f32(xt[n]);
#pragma unroll
        for (int j = 0; j < 8; ++j) l[j] += xv * wr[(int64_t)e[j] * d + n];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        float v = l[j];
#pragma unroll
        for (int s = 32; s >= 1; s >>= 1) v += __shfl_xor(v, s, 64);
        if (lane == 0) part[wave][j] = v;
    }
    __syncthreads();
    if (tid == 0) {
        float s[8], S = 0.f, gdg = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float lj = part[0][j] + part[1][j] + part[2][j] + part[3][j];
            s[j] = 1.0f / (1.0f + expf(-lj));
            S += s[j];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) gdg += s[j] / S * dg[(int64_t)t * 8 + j];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float ds = (dg[(int64_t)t * 8 + j] - gdg) / S;
            const float v = ds * s[j] * (1.0f - s[j]);
            dls[j] = v;
            dl[(int64_t)t * 8 + j] = v;
        }
    }
    __syncthreads();
    for (int n = tid; n < d; n += 256) {
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc += dls[j] * wr[(int64_t)e[j] * d + n];
        dx[(int64_t)t * d + n] = acc;
    }
}

// Router weight gradient dwr[e, n] = sum over e's rows r (ascending) of
// dl[row_src[r]] x[row_src[r] / 8, n]: each of kDwrChunks workgroups per
// (expert, 256 columns) sums an equal share of the rows into part[chunk],
// then k_bwd_dwr_sum adds the shares in chunk order (deterministic).
constexpr int kDwrChunks = 16;
__global__ __launch_bounds__(256) void k_bwd_dwr(int d, const int32_t *__restrict__ offsets,
                                                 const int32_t *__restrict__ row_src, const float *__restrict__ dl,
                                                 const uint16_t *__restrict__ x, float *__restrict__ part) {
    const int e = blockIdx.y, ch = blockIdx.z, n = blockIdx.x * 256 + threadIdx.x;
    if (n >= d) return;
    const int b = offsets[e], c = offsets[e + 1] - b;
    const int r0 = b + (int)((int64_t)c * ch / kDwrChunks), r1 = b + (int)((int64_t)c * (ch + 1) / kDwrChunks);
    float acc = 0.f;
    for (int r = r0; r < r1; ++r) {
        const int f = row_src[r];
        acc += dl[f] * bf16_to_f32(x[(int64_t)(f / 8) * d + n]);
    }
    part[((int64_t)ch * kE + e) * d + n] = acc;
}

__global__ __launch_bounds__(256) void k_bwd_dwr_sum(int64_t n, const float *__restrict__ part,
                                                     float *__restrict__ dwr) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    float acc = part[i];
#pragma unroll
    for (int ch = 1; ch < kDwrChunks; ++ch) acc += part[ch * n + i];
    dwr[i] = acc;
}

// dx[t] += dxs[t] + sum_j dxp[row_of[t*8 + j]] (j ascending), 4 columns per thread.
__global__ __launch_bounds__(256) void k_bwd_dx(int T, int d, const float *__restrict__ dxs,
                                                const float *__restrict__ dxp, const int32_t *__restrict__ row_of,
                                                float *__restrict__ dx) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int w4 = d / 4;
    if (i >= (int64_t)T * w4) return;
    const int64_t t = i / w4;
    const int c = (int)(i - t * w4) * 4;
    f32x4 v = *reinterpret_cast<const f32x4 *>(dx + t * d + c);
    const f32x4 s = *reinterpret_cast<const f32x4 *>(dxs + t * d + c);
    v += s;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int r = row_of[t * 8 + j];
        v += *reinterpret_cast<const f32x4 *>(dxp + (int64_t)r * d + c);
    }
    *reinterpret_cast<f32x4 *>(dx + t * d + c) = v;
}

template <int GROUP, bool ACC>
hipError_t bgemm(const BGemm &p, int G, hipStream_t s) {
    dim3 grid;
    if (GROUP == GROUP_M) grid = dim3((p.M + GM - 1) / GM + G, p.N / GN);
    else if (GROUP == GROUP_K) grid = dim3(p.M / GM, p.N / GN, G);
    else grid = dim3((p.M + GM - 1) / GM, p.N / GN);
    hipLaunchKernelGGL((k_bgemm<GROUP, ACC>), grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace

namespace bwd {

hipError_t pad_offsets(const int32_t *off, int32_t *poff, int align, hipStream_t s) {
    if (align == 128) hipLaunchKernelGGL(k_pad_offsets<128>, dim3(1), dim3(64), 0, s, off, poff);
    else hipLaunchKernelGGL(k_pad_offsets<64>, dim3(1), dim3(64), 0, s, off, poff);
    return hipGetLastError();
}

hipError_t combine(int T, int d, const float *dy, const uint16_t *y_perm, const int32_t *row_of, const float *g,
                   void *dyp, void *dys, float *dg, bool f32_out, hipStream_t s) {
    if (f32_out)
        hipLaunchKernelGGL(k_bwd_combine<true>, dim3((T + 3) / 4), dim3(256), 0, s, T, d, dy, y_perm, row_of, g, dyp,
                           dys, dg);
    else
        hipLaunchKernelGGL(k_bwd_combine<false>, dim3((T + 3) / 4), dim3(256), 0, s, T, d, dy, y_perm, row_of, g, dyp,
                           dys, dg);
    return hipGetLastError();
}

hipError_t swiglu(int64_t rows, int I, const float *P, const float *dh, void *h, void *dab, bool f32_out,
                  hipStream_t s) {
    const int64_t n = rows * I;
    const dim3 grid((unsigned)((n + 255) / 256));
    if (f32_out) hipLaunchKernelGGL(k_bwd_swiglu<true>, grid, dim3(256), 0, s, n, I, P, dh, h, dab);
    else hipLaunchKernelGGL(k_bwd_swiglu<false>, grid, dim3(256), 0, s, n, I, P, dh, h, dab);
    return hipGetLastError();
}

hipError_t router(int T, int d, const uint16_t *x, const float *wr, const int32_t *idx, const float *dg, float *dl,
                  float *dx, hipStream_t s) {
    hipLaunchKernelGGL(k_bwd_router, dim3(T), dim3(256), 0, s, d, x, wr, idx, dg, dl, dx);
    return hipGetLastError();
}

size_t dwr_part_bytes(int d) { return (size_t)kDwrChunks * kE * d * 4; }

hipError_t dwr(int d, const int32_t *offsets, const int32_t *row_src, const float *dl, const uint16_t *x,
               float *part, float *dwr_out, hipStream_t s) {
    hipLaunchKernelGGL(k_bwd_dwr, dim3((d + 255) / 256, kE, kDwrChunks), dim3(256), 0, s, d, offsets, row_src, dl, x,
                       part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n = (int64_t)kE * d;
    hipLaunchKernelGGL(k_bwd_dwr_sum, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, n, part, dwr_out);
    return hipGetLastError();
}

hipError_t zero_empty(int64_t per, const int32_t *off, float *out, hipStream_t s) {
    hipLaunchKernelGGL(k_zero_empty, dim3(256, kE), dim3(256), 0, s, per, off, out);
    return hipGetLastError();
}

hipError_t dx(int T, int d, const float *dxs, const float *dxp, const int32_t *row_of, float *dx_out, hipStream_t s) {
    const int64_t n = (int64_t)T * (d / 4);
    hipLaunchKernelGGL(k_bwd_dx, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, T, d, dxs, dxp, row_of, dx_out);
    return hipGetLastError();
}

}  // namespace bwd

namespace {

// The backward's workspace, carved in a fixed order (base == nullptr: sizes only).
struct BwdWs {
    uint16_t *dyo;         // [R, d] output gradients: routed rows, then shared rows (bf16)
    float *P;              // [R, 2I] pre-activations (gate | up)
    float *dh;             // [R, I]
    uint16_t *h16;         // [R, I]
    uint16_t *dab;         // [R, 2I] SwiGLU input gradients (da | db)
    float *dxi;            // [R, d] input gradients
    float *dl, *dg;        // [T*k]
    int32_t *poff;         // [E+1]
    float *dwr_part;       // [16, E, d] router-gradient partial sums
    uint16_t *wdT;         // [E, I, d] down weights transposed
    uint16_t *wguT;        // [E, d, 2I] gate | up weights transposed
    uint16_t *sdT, *sguT;  // the shared expert's: [I, d], [d, 2I]
    uint16_t *xT, *dyoT, *hT, *dabT;       // routed rows transposed, padded per expert: [*, Rp]
    uint16_t *xsT, *dysT, *hsT, *dabsT;    // shared rows transposed: [*, Tp]
    size_t bytes;
};

// Which data-gradient products the persistent kernel takes with K-major
// weights (dh, dx; routed, shared): a function of the shape only.  Those that
// it does not take need transposed weight copies in the workspace.
struct KnPlan {
    bool dh, dhs, dx, dxs;
};

LargeGemmArgs kn_args(int M, const int32_t *offsets, int K, int N, int ksplit) {
    LargeGemmArgs g{};
    g.M = M; g.offsets = offsets; g.a_div = 1; g.a_src_rows = M; g.K = K; g.N = N; g.ldo = N;
    g.b_kn = true; g.ksplit = ksplit;
    return g;
}

KnPlan kn_plan(int T, int d, int I, int k) {
    static const int32_t grouped = 0;  // stands for an offsets array: only its presence is read
    const int A = T * k;
    return KnPlan{bf16_large_gemm_ok(kn_args(A, &grouped, d, I, 0)), bf16_large_gemm_ok(kn_args(T, nullptr, d, I, 0)),
                  bf16_large_gemm_ok(kn_args(A, &grouped, 2 * I, d, I)),
                  bf16_large_gemm_ok(kn_args(T, nullptr, 2 * I, d, I))};
}

BwdWs carve(char *base, int T, int d, int I, int k) {
    BwdWs w{};
    const KnPlan kn = kn_plan(T, d, I, k);
    size_t o = 0;
    const size_t A = (size_t)T * k, R = A + T, Rp = A + 64 * (size_t)kE, Tp = ((size_t)T + 31) / 32 * 32;
    auto take = [&](size_t n) -> char * {
        char *p = base ? base + o : nullptr;
        o += (n + 255) / 256 * 256;
        return p;
    };
    w.dyo = reinterpret_cast<uint16_t *>(take(R * d * 2));
    w.P = reinterpret_cast<float *>(take(R * 2 * I * 4));
    w.dh = reinterpret_cast<float *>(take(R * I * 4));
    w.h16 = reinterpret_cast<uint16_t *>(take(R * I * 2));
    w.dab = reinterpret_cast<uint16_t *>(take(R * 2 * I * 2));
    w.dxi = reinterpret_cast<float *>(take(R * d * 4));
    w.dl = reinterpret_cast<float *>(take(A * 4));
    w.dg = reinterpret_cast<float *>(take(A * 4));
    w.poff = reinterpret_cast<int32_t *>(take((kE + 1) * 4));
    w.dwr_part = reinterpret_cast<float *>(take(bwd::dwr_part_bytes(d)));
    // transposed weights, only for products that do not read them K-major
    w.wdT = kn.dh ? nullptr : reinterpret_cast<uint16_t *>(take((size_t)kE * I * d * 2));
    w.wguT = kn.dx ? nullptr : reinterpret_cast<uint16_t *>(take((size_t)kE * d * 2 * I * 2));
    w.sdT = kn.dhs ? nullptr : reinterpret_cast<uint16_t *>(take((size_t)I * d * 2));
    w.sguT = kn.dxs ? nullptr : reinterpret_cast<uint16_t *>(take((size_t)d * 2 * I * 2));
    w.xT = reinterpret_cast<uint16_t *>(take((size_t)d * Rp * 2));
    w.dyoT = reinterpret_cast<uint16_t *>(take((size_t)d * Rp * 2));
    w.hT = reinterpret_cast<uint16_t *>(take((size_t)I * Rp * 2));
    w.dabT = reinterpret_cast<uint16_t *>(take((size_t)2 * I * Rp * 2));
    w.xsT = reinterpret_cast<uint16_t *>(take((size_t)d * Tp * 2));
    w.dysT = reinterpret_cast<uint16_t *>(take((size_t)d * Tp * 2));
    w.hsT = reinterpret_cast<uint16_t *>(take((size_t)I * Tp * 2));
    w.dabsT = reinterpret_cast<uint16_t *>(take((size_t)2 * I * Tp * 2));
    w.bytes = o;
    return w;
}

// Weights transposed per group: out[g][c*ldo + coff + r] = in[g][r*C + c]
// (bf16; R a multiple of 64, C of 128), 64-row x 128-column tiles.  Thread
// (a = tid % 16, b = tid / 16) reads 16 bytes (8 values) of each of rows
// 4a .. 4a+3 at columns 8b .. 8b+7 (four 16-byte loads in flight), and
// writes each column's 4 values as one 8-byte LDS word of output row 8b + j;
// each output row's 128 bytes then go out as eight 16-byte stores.
__global__ __launch_bounds__(256) void k_t16(int C, const uint16_t *__restrict__ in, int64_t gin,
                                             uint16_t *__restrict__ out, int64_t ldo, int64_t gout, int coff) {
    __shared__ __attribute__((aligned(16))) uint64_t tile[128 * 16];
    const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 128, g = blockIdx.z, tid = threadIdx.x;
    in += (int64_t)g * gin;
    out += (int64_t)g * gout;
    {
        const int a = tid & 15, b = tid >> 4;
        i32x4 v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            v[i] = *reinterpret_cast<const i32x4 *>(in + (int64_t)(r0 + 4 * a + i) * C + c0 + 8 * b);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            // value j of each row (word j / 2, half j % 2): output row 8b + j, rows 4a .. 4a+3
            const int sh = 16 * (j & 1);
            const uint32_t lo = (((uint32_t)v[0][j >> 1] >> sh) & 0xffffu) | ((((uint32_t)v[1][j >> 1] >> sh) & 0xffffu) << 16);
            const uint32_t hi = (((uint32_t)v[2][j >> 1] >> sh) & 0xffffu) | ((((uint32_t)v[3][j >> 1] >> sh) & 0xffffu) << 16);
            tile[(8 * b + j) * 16 + a] = (uint64_t)lo | ((uint64_t)hi << 32);
        }
    }
    __syncthreads();
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
        const int c = 32 * pass + (tid >> 3), q = tid & 7;
        const i32x4 v = *reinterpret_cast<const i32x4 *>(&tile[c * 16 + 2 * q]);
        *reinterpret_cast<i32x4 *>(out + (int64_t)(c0 + c) * ldo + coff + r0 + 8 * q) = v;
    }
}

hipError_t t16(int R, int C, int G, const uint16_t *in, uint16_t *out, int64_t ldo, int coff, hipStream_t s) {
    if (R % 64 != 0 || C % 128 != 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_t16, dim3(R / 64, C / 128, G), dim3(256), 0, s, C, in, (int64_t)R * C, out, ldo,
                       (int64_t)C * ldo, coff);
    return hipGetLastError();
}

// out[g] = in[g] transposed (R x C -> C x R), see k_transpose.  Plain: dend
// positions (zeros past R).  Grouped (off, poff): R = the total rows.
hipError_t transpose(int R, int C, int G, const uint16_t *in, int64_t ldi, int64_t gin, const int32_t *rows,
                     int rdiv, const int32_t *off, const int32_t *poff, int dend, uint16_t *out, int64_t ldo,
                     int64_t gout, int coff, hipStream_t s) {
    const int tiles = off ? R / 64 + kE + 1 : (dend + 63) / 64;
    if (tiles <= 0) return hipSuccess;
    if (tiles > 65535) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_transpose, dim3(C / 64, tiles, G), dim3(256), 0, s, R, in, ldi, gin, rows, rdiv, off,
                       poff, dend, out, ldo, gout, coff);
    return hipGetLastError();
}

}  // namespace

size_t backward_ws_bytes(int T, int d, int I, int k) { return carve(nullptr, T, d, I, k).bytes; }

bool backward_ok(int d, int I) { return d % 128 == 0 && I % 128 == 0; }

hipError_t launch_backward(const BackwardArgs &a, void *ws, hipStream_t s) {
    const int T = a.T, d = a.d, I = a.I, k = a.k, E = kE;
    const int A = T * k;
    const int64_t Rp = (int64_t)A + 64 * kE, Tp = ((int64_t)T + 31) / 32 * 32;
    const BwdWs w = carve(static_cast<char *>(ws), T, d, I, k);
    float *dg = a.dg ? a.dg : w.dg;
    const uint16_t *x = static_cast<const uint16_t *>(a.x);
    const uint16_t *eg = static_cast<const uint16_t *>(a.experts.gate), *eu = static_cast<const uint16_t *>(a.experts.up),
                   *ed = static_cast<const uint16_t *>(a.experts.down);
    const uint16_t *sg = static_cast<const uint16_t *>(a.shared.gate), *su = static_cast<const uint16_t *>(a.shared.up),
                   *sd = static_cast<const uint16_t *>(a.shared.down);
    // shared-expert slices of the row-major buffers
    uint16_t *dys = w.dyo + (int64_t)A * d;
    float *Ps = w.P + (int64_t)A * 2 * I, *dhs = w.dh + (int64_t)A * I, *dxs = w.dxi + (int64_t)A * d;
    uint16_t *hs = w.h16 + (int64_t)A * I, *dabs = w.dab + (int64_t)A * 2 * I;
    hipError_t e;
#define CHK(call)                      \
    if ((e = (call)) != hipSuccess) return e;

    // The data-gradient products dh = (output gradient) W_down and
    // dx = (da | db) (W_gate | W_up) reduce along the weights' rows: the
    // persistent kernel reads such a B K-major, as stored (W_down [E, d, I]:
    // K = d; W_gate and W_up [E, I, d]: K = 2I, gate rows then up rows).
    // Shapes it does not take run on k_bgemm from transposed copies.
    const LargeGemmArgs gdh{A, a.offsets, w.dyo, nullptr, 1, A, d, ed, nullptr, I, w.dh, I, 0, false,
                            nullptr, 0, 0, true, 0};
    const LargeGemmArgs gdhs{T, nullptr, dys, nullptr, 1, T, d, sd, nullptr, I, dhs, I, 0, false, nullptr, 0, 0, true, 0};
    const LargeGemmArgs gdx{A, a.offsets, w.dab, nullptr, 1, A, 2 * I, eg, eu, d, w.dxi, d, 0, false,
                            nullptr, 0, 0, true, I};
    const LargeGemmArgs gdxs{T, nullptr, dabs, nullptr, 1, T, 2 * I, sg, su, d, dxs, d, 0, false, nullptr, 0, 0, true, I};
    // the workspace holds transposed copies exactly where the plan says so
    const KnPlan kn = kn_plan(T, d, I, k);
    const bool kn_dh = kn.dh, kn_dhs = kn.dhs, kn_dx = kn.dx, kn_dxs = kn.dxs;
    if (kn_dh != bf16_large_gemm_ok(gdh) || kn_dhs != bf16_large_gemm_ok(gdhs) || kn_dx != bf16_large_gemm_ok(gdx) ||
        kn_dxs != bf16_large_gemm_ok(gdxs))
        return hipErrorInvalidValue;

    // 0. padded row positions of the expert groups; transposed weights where needed
    CHK(bwd::pad_offsets(a.offsets, w.poff, 64, s));
    if (!kn_dh) CHK(t16(d, I, E, ed, w.wdT, d, 0, s));  // [E, I, d]
    if (!kn_dx) {
        CHK(t16(I, d, E, eg, w.wguT, 2 * I, 0, s));  // [E, d, 2I]: gate | up
        CHK(t16(I, d, E, eu, w.wguT, 2 * I, I, s));
    }
    if (!kn_dhs) CHK(t16(d, I, 1, sd, w.sdT, d, 0, s));
    if (!kn_dxs) {
        CHK(t16(I, d, 1, sg, w.sguT, 2 * I, 0, s));
        CHK(t16(I, d, 1, su, w.sguT, 2 * I, I, s));
    }

    // 1. combine backward
    CHK(bwd::combine(T, d, a.dy, static_cast<const uint16_t *>(a.y_perm), a.row_of, a.weights, w.dyo, dys, dg, false,
                     s));
    // The data-gradient GEMMs (and the recompute) are NT GEMMs grouped over
    // M: the forward's persistent 256x256-tile kernel with an fp32 epilogue
    // when the groups are large enough, else k_bgemm.
    auto nt = [&](const LargeGemmArgs &g, const int32_t *offsets, int64_t lda) -> hipError_t {
        if (bf16_large_gemm_ok(g)) return launch_bf16_large_gemm(g, s);
        for (int half = 0; half < (g.dual ? 2 : 1); ++half) {
            BGemm p{};
            p.M = g.M; p.N = g.N; p.K = g.K; p.offsets = offsets; p.A = g.A; p.lda = lda;
            p.a_rows = g.a_rows; p.a_div = g.a_div; p.B = half ? g.B1 : g.B0; p.ldb = g.K;
            p.bstride = (int64_t)g.N * g.K; p.C = g.out + (half ? g.up_off : 0); p.ldc = g.ldo;
            const hipError_t r = offsets ? bgemm<GROUP_M, false>(p, E, s)
                                         : bgemm<GROUP_NONE, false>(p, 1, s);
            if (r != hipSuccess) return r;
        }
        return hipSuccess;
    };
    // 2. pre-activations: routed rows gather x through row_src; shared rows are x
    CHK(nt(LargeGemmArgs{A, a.offsets, x, a.row_src, k, T, d, eg, eu, I, w.P, 2 * I, I, true}, a.offsets, d));
    CHK(nt(LargeGemmArgs{T, nullptr, x, nullptr, 1, T, d, sg, su, I, Ps, 2 * I, I, true}, nullptr, d));
    // 3. dh = (output gradient) W_down (K-major W_down, or transposed to [E, I, d])
    CHK(kn_dh ? launch_bf16_large_gemm(gdh, s)
              : nt(LargeGemmArgs{A, a.offsets, w.dyo, nullptr, 1, A, d, w.wdT, nullptr, I, w.dh, I, 0, false}, a.offsets, d));
    CHK(kn_dhs ? launch_bf16_large_gemm(gdhs, s)
               : nt(LargeGemmArgs{T, nullptr, dys, nullptr, 1, T, d, w.sdT, nullptr, I, dhs, I, 0, false}, nullptr, d));
    // 4. SwiGLU backward (routed and shared rows in one pass)
    CHK(bwd::swiglu((int64_t)A + T, I, w.P, w.dh, w.h16, w.dab, false, s));
    // 5. input gradients: (da | db) [rows, 2I] times (W_gate | W_up) (K-major, or transposed to [E, d, 2I])
    CHK(kn_dx ? launch_bf16_large_gemm(gdx, s)
              : nt(LargeGemmArgs{A, a.offsets, w.dab, nullptr, 1, A, 2 * I, w.wguT, nullptr, d, w.dxi, d, 0, false},
                   a.offsets, 2 * I));
    CHK(kn_dxs ? launch_bf16_large_gemm(gdxs, s)
               : nt(LargeGemmArgs{T, nullptr, dabs, nullptr, 1, T, 2 * I, w.sguT, nullptr, d, dxs, d, 0, false}, nullptr,
                    2 * I));
    // 6. weight gradients.  The rows each expert reduces over are transposed
    //    into [*, Rp] buffers where expert e's rows start at poff[e] (64-aligned,
    //    zero-padded), so both operands are K-contiguous and every K range is
    //    whole 64-wide stages.
    {
        CHK(transpose(A, d, 1, x, d, 0, a.row_src, k, a.offsets, w.poff, 0, w.xT, Rp, 0, 0, s));
        CHK(transpose(A, d, 1, w.dyo, d, 0, nullptr, 1, a.offsets, w.poff, 0, w.dyoT, Rp, 0, 0, s));
        CHK(transpose(A, I, 1, w.h16, I, 0, nullptr, 1, a.offsets, w.poff, 0, w.hT, Rp, 0, 0, s));
        CHK(transpose(A, 2 * I, 1, w.dab, 2 * I, 0, nullptr, 1, a.offsets, w.poff, 0, w.dabT, Rp, 0, 0, s));
        // out_e = A[:, K_e] B[:, K_e]^T: the large-tile kernel in its K-grouped
        // form (experts with no rows are zeroed separately), else k_bgemm
        auto kg = [&](int M, int N, const uint16_t *Aop, const uint16_t *Bop, float *out) -> hipError_t {
            LargeGemmArgs g{};
            g.M = M; g.A = Aop; g.a_div = 1; g.K = (int)Rp; g.B0 = Bop; g.N = N; g.out = out; g.ldo = N;
            g.kseg = w.poff; g.ldk = (int)Rp; g.cstride = (int64_t)M * N;
            if (bf16_large_gemm_ok(g)) {
                const hipError_t r = launch_bf16_large_gemm(g, s);
                if (r != hipSuccess) return r;
                hipLaunchKernelGGL(k_zero_empty, dim3(256, E), dim3(256), 0, s, (int64_t)M * N, a.offsets, out);
                return hipGetLastError();
            }
            BGemm p{};
            p.M = M; p.N = N; p.K = (int)Rp; p.offsets = w.poff; p.A = Aop; p.lda = Rp; p.a_div = 1;
            p.B = Bop; p.ldb = Rp; p.C = out; p.ldc = N; p.cstride = (int64_t)M * N;
            return bgemm<GROUP_K, false>(p, E, s);
        };
        CHK(kg(I, d, w.dabT, w.xT, a.dw_gate));
        CHK(kg(I, d, w.dabT + (int64_t)I * Rp, w.xT, a.dw_up));
        CHK(kg(d, I, w.dyoT, w.hT, a.dw_down));
        // shared expert: one group over all T rows (padded to Tp with zeros)
        CHK(transpose(T, d, 1, x, d, 0, nullptr, 1, nullptr, nullptr, (int)Tp, w.xsT, Tp, 0, 0, s));
        CHK(transpose(T, d, 1, dys, d, 0, nullptr, 1, nullptr, nullptr, (int)Tp, w.dysT, Tp, 0, 0, s));
        CHK(transpose(T, I, 1, hs, I, 0, nullptr, 1, nullptr, nullptr, (int)Tp, w.hsT, Tp, 0, 0, s));
        CHK(transpose(T, 2 * I, 1, dabs, 2 * I, 0, nullptr, 1, nullptr, nullptr, (int)Tp, w.dabsT, Tp, 0, 0, s));
        // plain NT products over K = Tp: the persistent kernel when it takes them
        const int tp = (int)Tp;
        CHK(nt(LargeGemmArgs{I, nullptr, w.dabsT, nullptr, 1, I, tp, w.xsT, nullptr, d, a.ds_gate, d, 0, false}, nullptr,
               Tp));
        CHK(nt(LargeGemmArgs{I, nullptr, w.dabsT + (int64_t)I * Tp, nullptr, 1, I, tp, w.xsT, nullptr, d, a.ds_up, d, 0,
                             false},
               nullptr, Tp));
        CHK(nt(LargeGemmArgs{d, nullptr, w.dysT, nullptr, 1, d, tp, w.hsT, nullptr, I, a.ds_down, I, 0, false}, nullptr,
               Tp));
    }
    // 7. router: dl and its share of dx (written), then the router gradient
    CHK(bwd::router(T, d, x, a.w_router, a.idx, dg, w.dl, a.dx, s));
    CHK(bwd::dwr(d, a.offsets, a.row_src, w.dl, x, w.dwr_part, a.dw_router, s));
    // 8. dx += shared + routed input gradients
    CHK(bwd::dx(T, d, dxs, w.dxi, a.row_of, a.dx, s));
#undef CHK
    return hipSuccess;
}

}  // namespace moe
