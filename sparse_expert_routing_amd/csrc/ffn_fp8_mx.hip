// Grouped SwiGLU expert GEMMs in OCP fp8 e4m3 for large groups (prefill),
// with the tile scales applied by the block-scaled MFMA: persistent
// workgroups, 256x256 tiles, the bf16 large-tile kernel's schedule.
//
// crackai.dev DeepSeek-V3 summary, "How It Works": FP8 matmuls with a scale
// per tile and FP32 accumulation; DeepSeek V3 From Scratch, "The idea":
// fine-grained quantisation tiles.  Tiles (ours, as in the rest of the
// library): one scale per 1x128 activation tile and per 128x128 weight
// block, each an E8M0 byte (OCP MX: byte e is 2^(e-127)).
//
// Design for gfx950:
//   - a stage is 128 of K (one scale block): A and B slabs of 256 rows x 128
//     bytes, the same 32 KB operand units, five-unit LDS ring and DMA
//     geometry (buffer_load_dwordx4 ... lds) as the bf16 kernel, whose K
//     stage is 64 bf16 of the same 128 bytes;
//   - 4 waves (2x2), each a 128x128 block as 4x4 v_mfma_scale_f32_32x32x64
//     accumulators in AGPRs; a stage is two steps of 64 of K, 16 MFMAs each,
//     so the MFMA cycles and LDS fragment bytes per stage equal the bf16
//     kernel's (each fragment is 32 bytes: two 16-byte pieces of the row);
//   - the E8M0 scale bytes go to the MFMA as they are: the weight block's for
//     every lane of the weight operand, the A row's for lanes l and l+32 of
//     the activation operand (row l % 32), so the products accumulate in
//     fp32 with no vector work; a stage's A-row scales are loaded one stage
//     ahead (before that stage's slot loads, so the stage waits cover them),
//     from a layout with each 128-block's scales in GEMM row order (one
//     contiguous run per stage and 32-row block);
//   - schedule: the ring holds A_s, B_s, A_{s+1}, B_{s+1} and A_{s+2} (in
//     flight); step 0 reads step 1's fragments, B's first, then a barrier
//     frees B_s's unit and B_{s+2} streams into it; a mid-stage barrier
//     (A_{s+1}, B_{s+1} landed) frees A_s's unit, and step 1 streams A_{s+3}
//     into it and reads stage s+1's first fragments: eight loads per step,
//     each with two steps or more to land;
//   - epilogues as in the bf16 kernel (register stores from the transposed
//     accumulators, bf16 as 16-byte stores after a lane-half swap, the next
//     tile's first two stages already in flight; the combine stages 64-row
//     chunks through LDS), the gate/up one
//     forming h = silu(g) u in fp32 and quantising it per 1x128 tile (the
//     tile's 128 h columns; the row amax of the two column waves meets in
//     the free fifth LDS unit);
//   - for the layer backward: an fp32 epilogue (M-grouped or plain
//     products), and a K-grouped form for the weight gradients (a group per
//     expert over its 128-aligned K range, both operands with a scale per
//     row and 128 of K, which each lane passes to the MFMA for its own
//     rows; groups with no rows are skipped).
#include "device.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kE = 256;
constexpr int LM = 256;        // rows per tile
constexpr int LB = 256;        // B rows per tile
constexpr int LKB = 128;       // K per stage (bytes = e4m3 elements): one scale block
constexpr int NUNIT = 5;       // LDS ring units (5 x 32 KB)
constexpr int UNIT_BYTES = LM * LKB;
constexpr int kGroupM = 8;     // row tiles per ordering group
constexpr int kChRows = 64;    // combine epilogue chunk rows
constexpr int kChLd = LB + 4;
// An offset past the end of every output resource: stores of padding rows
// are dropped.
constexpr uint32_t kOobOff = 0xFFFF0000u;

enum { MX_SWIGLU_Q = 0, MX_STORE = 1, MX_COMBINE = 2, MX_F32 = 3 };

struct MxParams {
    int M;
    const int32_t *offsets;   // routed: [E+1] row ranges
    const uint8_t *A;         // [rows, K] codes
    const uint8_t *As;        // [rows, K/128] E8M0 scales (byte e: 2^(e-127)); as_km: [K/128, M]
    int as_km;                // As per 128-block in GEMM row order (no gather of the scales)
    const int32_t *a_rows;    // optional: GEMM row r reads row a_rows[r] / a_div of A / As
    int a_div;
    int K;
    const uint8_t *B0, *B1;   // [G, N, K] codes (gate, up; or down)
    const uint8_t *S0, *S1;   // [G, N/128, K/128] E8M0 block scales
    int N;                    // B rows per expert (SwiGLU: rows of each of gate / up)
    uint8_t *hq;              // MX_SWIGLU_Q: [M, N] codes
    uint8_t *hs;              // MX_SWIGLU_Q: [N/128, M] E8M0, per 128-block in row order
    uint16_t *out;            // MX_STORE: bf16 [M, N]
    float *yout;              // MX_COMBINE: f32 [M, N]; MX_F32: f32 rows of ldo
    int ldo;
    const uint16_t *y_perm;   // MX_COMBINE: routed outputs [M*k, N] bf16
    const int32_t *row_of;    // MX_COMBINE: [M*k]
    const float *cw;          // MX_COMBINE: combine weights [M*k]
    // K-grouped form (weight gradients, MX_F32): group e reduces over K in
    // [kseg[e], kseg[e+1]) (multiples of 128) of A [M, K] and B0 [N, K], both
    // with a scale per row and 128 of K (As [M, K/128], Bs [N, K/128]), into
    // yout + e * cstride; groups with an empty range are skipped.
    const int32_t *kseg;
    const uint8_t *Bs;
    int64_t cstride;
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

// Routed tile t -> expert e, rows [m0, m_end) of its row tile and column
// tile nt.  Tiles run expert by expert (an expert with n row tiles owns
// NT * n consecutive tiles); inside an expert, groups of at most kGroupM
// row tiles with the row tile fastest, so the row tiles that read one
// weight column slice run side by side and no group spans two experts'
// weights.
__device__ __forceinline__ void tilemap_tile(const TileMap &tm, int t, int NT, int &e, int &m0, int &m_end,
                                             int &nt) {
    const int lane = threadIdx.x & 63;
    const int rt = t / NT;
    const int mine = tm.nt[0] + tm.nt[1] + tm.nt[2] + tm.nt[3];
    const bool own = rt >= tm.excl && rt < tm.excl + mine;
    const int owner = __ffsll((unsigned long long)__ballot(own)) - 1;
    int my_e = 0, my_first = 0, my_n = 1, my_off = 0, my_end = 0;
    if (own) {
        int s = rt - tm.excl, first = tm.excl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (s >= 0 && s < tm.nt[i]) {
                my_e = lane * 4 + i;
                my_first = first;
                my_n = tm.nt[i];
                my_off = tm.off[i];
                my_end = tm.off[i + 1];
            }
            s -= tm.nt[i];
            first += tm.nt[i];
        }
    }
    e = __shfl(my_e, owner, 64);
    const int first = __shfl(my_first, owner, 64), n = __shfl(my_n, owner, 64);
    const int off = __shfl(my_off, owner, 64);
    m_end = __shfl(my_end, owner, 64);
    const int u = t - NT * first;
    const int j = u / (kGroupM * NT);
    const int gm = min(kGroupM, n - kGroupM * j);
    const int within = u - j * kGroupM * NT;
    m0 = off + (kGroupM * j + within % gm) * LM;
    nt = within / gm;
}

// K-grouped tile map: lane owns groups 4*lane .. 4*lane+3; a group with a
// non-empty K range has `per` tiles.  No kseg: one group over [0, K).
__device__ __forceinline__ void kgmap_init(TileMap &tm, const int32_t *__restrict__ kseg, int K, int per) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < 5; ++i) tm.off[i] = kseg ? kseg[lane * 4 + i] : (lane == 0 && i == 0 ? 0 : K);
    int s = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        tm.nt[i] = tm.off[i + 1] > tm.off[i] ? per : 0;
        s += tm.nt[i];
    }
    const int incl = wave_incl_scan(s);
    tm.excl = incl - s;
    tm.total = __shfl(incl, 63, 64);
}

__device__ __forceinline__ void kgmap_find(const TileMap &tm, int slot, int &e, int &local) {
    const int lane = threadIdx.x & 63;
    const int mine = tm.nt[0] + tm.nt[1] + tm.nt[2] + tm.nt[3];
    const bool own = slot >= tm.excl && slot < tm.excl + mine;
    const int owner = __ffsll((unsigned long long)__ballot(own)) - 1;
    int my_e = 0, my_l = 0;
    if (own) {
        int s = slot - tm.excl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (s >= 0 && s < tm.nt[i]) {
                my_e = lane * 4 + i;
                my_l = s;
            }
            s -= tm.nt[i];
        }
    }
    e = __shfl(my_e, owner, 64);
    local = __shfl(my_l, owner, 64);
}

// Byte offset, inside one operand unit, of the 16-byte piece c of tile row
// `row`: piece c sits at position c ^ (row & 7) ^ ((row >> 3) & 1), so the
// 32 lanes reading one logical piece of 32 consecutive rows hit distinct banks.
__device__ __forceinline__ int piece(int row, int c) { return row * LKB + ((c ^ (row & 7) ^ ((row >> 3) & 1)) * 16); }

template <int N>
__device__ __forceinline__ void wait_vmcnt_lds() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef int i32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ const void *uniform_ptr(const void *p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<const void *>(((uint64_t)hi << 32) | lo);
}

// One 1 KB block (8 rows of 128 B) of a stage operand, global -> LDS.
__device__ __forceinline__ void dma_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint8_t *lds_block) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)(lds_block), 16, voff, soff, 0, 0);
}

// 32 bytes of K (pieces c and c+1 of the row) as one MFMA operand.
__device__ __forceinline__ i32x8 frag32(const uint8_t *unit, int row, int c) {
    const i32x4 lo = *reinterpret_cast<const i32x4 *>(unit + piece(row, c));
    const i32x4 hi = *reinterpret_cast<const i32x4 *>(unit + piece(row, c + 1));
    return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// acc += A x B^T for one 32x32 block and 64 of K, the scales (E8M0) of the A
// row this lane carries (ea) and of the B rows (eb).  TRANS swaps the
// operands, so the accumulator holds the transposed block: lane l owns tile
// row l % 32 and, in registers 4q .. 4q+3, the 4 consecutive tile columns
// 8q + 4(l / 32) .. +3.
template <bool TRANS>
__device__ __forceinline__ f32x16 mma(i32x8 a, i32x8 b, f32x16 c, int ea, int eb) {
    if constexpr (TRANS) return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c, 0, 0, 0, eb, 0, ea);
    else return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, ea, 0, eb);
}

__device__ __forceinline__ float acc_read(float x) {
    float r;
    asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(r) : "a"(x));
    return r;
}

__device__ __forceinline__ float swiglu(float g, float u) {
    return g * u * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * g));
}

template <int EPI, bool ROUTED, bool KG = false>
__global__ __launch_bounds__(256, 1) void k_gemm_fp8_mx(MxParams p) {
    static_assert(!KG || (EPI == MX_F32 && !ROUTED), "the K-grouped form has an fp32 output, one B");
    constexpr bool DUAL = EPI == MX_SWIGLU_Q;
    constexpr bool TRANS = EPI != MX_COMBINE;
    constexpr int BN = DUAL ? LB / 2 : LB;  // output columns per tile
    // buffer stores per lane per register epilogue: gate/up 4 x (8 codes + 1 scale); store 64; fp32 64
    constexpr int kEpiStores = TRANS ? (DUAL ? 36 : EPI == MX_STORE ? 32 : 64) : 0;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[NUNIT * UNIT_BYTES];  // 160 KB

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1, g = lane >> 5;
    const int K = p.K, nkall = K / LKB;  // K: the row stride of A and B (bytes)
    int nk = nkall;                     // stages of the tile (K-grouped: set per tile)

    TileMap tm;
    int Mt, total;
    const int NT = p.N / BN;
    if (ROUTED) {
        tilemap_init(tm, p.offsets);
        Mt = tm.total;
        total = Mt * NT;
    } else if (KG) {
        Mt = p.M / LM;
        kgmap_init(tm, p.kseg, K, Mt * NT);
        total = tm.total;
    } else {
        Mt = (p.M + LM - 1) / LM;
        total = Mt * NT;
    }
    const int P = gridDim.x;

    // DMA geometry: each operand (256 rows x 128 B = 32 blocks of 1 KB) is
    // moved by 8 instructions per wave: wave w takes blocks w + 4*i; lane l
    // fills physical piece (l & 7) of row 8*blk + (l >> 3).
    int drow[8], dcol[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = 8 * (wave + 4 * i) + (lane >> 3);
        drow[i] = row;
        dcol[i] = ((lane & 7) ^ (row & 7) ^ ((row >> 3) & 1)) * 16;
    }

    int e = 0, m0 = 0, m_end = 0, n0 = 0, kbase = 0;
    const uint32_t a_rows_total = p.a_rows ? (uint32_t)(p.M / p.a_div) : (uint32_t)p.M;
    const __amdgpu_buffer_rsrc_t rA = buf_rsrc(p.A, a_rows_total * (uint32_t)K);
    const __amdgpu_buffer_rsrc_t rAs = buf_rsrc(p.As, (p.as_km ? (uint32_t)p.M : a_rows_total) * (uint32_t)nkall);
    const uint32_t sstride = p.as_km ? (uint32_t)p.M : 1u;  // A-row scale bytes between 128-blocks
    const __amdgpu_buffer_rsrc_t rBs = buf_rsrc(KG ? p.Bs : p.As, KG ? (uint32_t)p.N * (uint32_t)nkall : 1u);
    const uint32_t b_bytes = (uint32_t)p.N * (uint32_t)K;
    const int nbk = p.N / 128;  // weight scale blocks along N
    const uint8_t *pBg = p.B0, *pBu = p.B1;
    const uint8_t *swg_p = p.S0, *swu_p = p.S0;
    uint32_t aoff[8], boff[8], soff[4], bsoff[4];

#define UNIT(u) (smem + (u) * UNIT_BYTES)
#define ISSUE_A(st_, i, unit_)                                                                 \
        dma_buf(rA, aoff[i], (uint32_t)min((st_), nk - 1) * LKB, (unit_) + (wave + 4 * (i)) * 1024)
#define B_RSRC()                                                                               \
        const __amdgpu_buffer_rsrc_t rBg_ = buf_rsrc(uniform_ptr(pBg), b_bytes);               \
        const __amdgpu_buffer_rsrc_t rBu_ = DUAL ? buf_rsrc(uniform_ptr(pBu), b_bytes) : rBg_;
#define ISSUE_B(st_, i, unit_)                                                                 \
        dma_buf((DUAL && (i) >= 4) ? rBu_ : rBg_, boff[i], (uint32_t)min((st_), nk - 1) * LKB, \
                (unit_) + (wave + 4 * (i)) * 1024)
    // The stage's A-row scales of this lane's 4 rows (one per 32-row block)
    // and the weight block scales of this wave's columns (gate and up): E8M0
    // bytes, which the block-scaled MFMA takes as they are.
#define LOAD_SCALES(st_, sa_, sw_, sb_)                                                        \
        {                                                                                      \
            const int kb_ = min((st_), nk - 1);                                                \
            _Pragma("unroll") for (int i = 0; i < 4; ++i)                                      \
                sa_[i] = __builtin_amdgcn_raw_buffer_load_b8(rAs, soff[i] + kb_ * sstride, 0, 0); \
            if (KG) {                                                                          \
                _Pragma("unroll") for (int j = 0; j < 4; ++j)                                  \
                    sb_[j] = __builtin_amdgcn_raw_buffer_load_b8(rBs, bsoff[j] + kb_, 0, 0);   \
            } else {                                                                           \
                sw_[0] = swg_p[kb_];                                                           \
                sw_[1] = DUAL ? swu_p[kb_] : sw_[0];                                           \
            }                                                                                  \
        }
#define TILE_SETUP(tt)                                                                         \
    {                                                                                          \
        int mt_, nt_;                                                                          \
        if (KG) {                                                                              \
            int loc_;                                                                          \
            kgmap_find(tm, (tt), e, loc_);                                                     \
            mt_ = loc_ % Mt;                                                                   \
            nt_ = loc_ / Mt;                                                                   \
            m0 = mt_ * LM;                                                                     \
            m_end = p.M;                                                                       \
            kbase = p.kseg ? __builtin_amdgcn_readfirstlane(p.kseg[e]) : 0;                    \
            nk = p.kseg ? __builtin_amdgcn_readfirstlane((p.kseg[e + 1] - kbase) / LKB) : nkall; \
        } else if (ROUTED) {                                                                   \
            tilemap_tile(tm, (tt), NT, e, m0, m_end, nt_);                                     \
        } else {                                                                               \
            const int gsz_ = kGroupM * NT;                                                     \
            const int grp_ = (tt) / gsz_, within_ = (tt) - grp_ * gsz_;                        \
            const int mfirst_ = grp_ * kGroupM;                                                \
            const int gm_ = min(kGroupM, Mt - mfirst_);                                        \
            mt_ = mfirst_ + within_ % gm_;                                                     \
            nt_ = within_ / gm_;                                                               \
            e = 0;                                                                             \
            m0 = mt_ * LM;                                                                     \
            m_end = p.M;                                                                       \
        }                                                                                      \
        e = __builtin_amdgcn_readfirstlane(e);                                                 \
        m0 = __builtin_amdgcn_readfirstlane(m0);                                               \
        m_end = __builtin_amdgcn_readfirstlane(m_end);                                         \
        n0 = nt_ * BN;                                                                         \
        pBg = KG ? p.B0 : p.B0 + (size_t)e * p.N * K;                                          \
        pBu = DUAL ? p.B1 + (size_t)e * p.N * K : pBg;                                         \
        swg_p = p.S0 + ((size_t)e * nbk + (DUAL ? n0 : n0 + wn * 128) / 128) * nk;             \
        swu_p = DUAL ? p.S1 + ((size_t)e * nbk + n0 / 128) * nk : swg_p;                       \
        int ar_[8], sr_[4];                                                                    \
        _Pragma("unroll") for (int i = 0; i < 8; ++i) ar_[i] = min(m0 + drow[i], m_end - 1);    \
        _Pragma("unroll") for (int i = 0; i < 4; ++i)                                          \
            sr_[i] = min(m0 + wm * 128 + 32 * i + (lane & 31), m_end - 1);                     \
        if (p.a_rows) { /* the row lookups issued together */                                  \
            _Pragma("unroll") for (int i = 0; i < 8; ++i) ar_[i] = p.a_rows[ar_[i]];            \
            if (!p.as_km) {                                                                    \
                _Pragma("unroll") for (int i = 0; i < 4; ++i) sr_[i] = p.a_rows[sr_[i]];        \
            }                                                                                  \
            _Pragma("unroll") for (int i = 0; i < 8; ++i) ar_[i] /= p.a_div;                    \
            if (!p.as_km) {                                                                    \
                _Pragma("unroll") for (int i = 0; i < 4; ++i) sr_[i] /= p.a_div;                \
            }                                                                                  \
        }                                                                                      \
        _Pragma("unroll") for (int i = 0; i < 8; ++i) {                                        \
            aoff[i] = (uint32_t)ar_[i] * (uint32_t)K + (uint32_t)(dcol[i] + kbase);            \
            const int r = drow[i];                                                             \
            const int br = DUAL ? n0 + (r & (BN - 1)) : n0 + r;                                \
            boff[i] = (uint32_t)br * (uint32_t)K + (uint32_t)(dcol[i] + kbase);                \
            if (m0 + r >= m_end) aoff[i] = kOobOff; /* padding rows fetch nothing */           \
        }                                                                                      \
        _Pragma("unroll") for (int i = 0; i < 4; ++i)                                          \
            soff[i] = p.as_km ? (uint32_t)sr_[i] : (uint32_t)sr_[i] * (uint32_t)nkall + (uint32_t)(kbase / LKB); \
        _Pragma("unroll") for (int j = 0; j < 4; ++j)                                          \
            bsoff[j] = (uint32_t)(n0 + wn * 128 + 32 * j + (lane & 31)) * (uint32_t)nkall +    \
                       (uint32_t)(kbase / LKB);                                                \
    }
    // Stage 0's scales, then A_0, B_0, A_1, B_1 of the tile just set up.
#define PROLOGUE_LOADS()                                                                       \
    {                                                                                          \
        LOAD_SCALES(0, sa, sw, sb);                                                            \
        B_RSRC()                                                                               \
        _Pragma("unroll") for (int i = 0; i < 8; ++i) ISSUE_A(0, i, UNIT(0));                  \
        _Pragma("unroll") for (int i = 0; i < 8; ++i) ISSUE_B(0, i, UNIT(1));                  \
        _Pragma("unroll") for (int i = 0; i < 8; ++i) ISSUE_A(1, i, UNIT(2));                  \
        _Pragma("unroll") for (int i = 0; i < 8; ++i) ISSUE_B(1, i, UNIT(3));                  \
    }

    int sa[4], sw[2], sa_n[4], sw_n[2], sb[4], sb_n[4];  // E8M0 exponents
    // Tile order: every XCD's P/8 workgroups take P/8 consecutive tiles at a
    // time (one L2 shares their operands): tiles (8i + xcd) P/8 + w in the
    // i-th pass.
    const int tlim = total, tstep = P;
    int t = (blockIdx.x & 7) * (P >> 3) + (blockIdx.x >> 3);
    if (t < tlim) {
        TILE_SETUP(t);
        PROLOGUE_LOADS();
    }
    bool first = true;
    for (; t < tlim; t += tstep) {
        f32x16 acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

#define B_ROW(j) ((DUAL ? (((j) >> 1) * 128 + wn * 64 + ((j) & 1) * 32) : (wn * 128 + (j) * 32)) + (lane & 31))
        // One 64-wide K step: 16 MFMAs on (AC, BC) with the stage's exponents
        // (EA per row block, EB0 / EB1 for the gate / up column blocks).  The
        // next step's 8 fragments (units nA / nB, piece column cn; fragments
        // 0-3 of A, 4-7 of B) are read before MFMA RD(r) (A only for the NB_
        // live row blocks, B only if any is live), HOOK(x) runs before MFMA
        // x and the slot load DMA(x) right after it; scheduling barriers
        // keep the order.
#define FRAG_READ(r, AN, BN_, nA, nB, cn)                                                      \
        if ((r) < 4)                                                                           \
            AN[(r) & 3] = frag32((nA), wm * 128 + ((r) & 3) * 32 + (lane & 31), (cn));         \
        else                                                                                   \
            BN_[(r) & 3] = frag32((nB), B_ROW((r) & 3), (cn));
#define STEP(AC, BC, AN, BN_, nA, nB, cn, RD, HOOK, DMA, NB_, EA, EB)                         \
        _Pragma("unroll") for (int x = 0; x < 16; ++x) {                                       \
            _Pragma("unroll") for (int r = 0; r < 8; ++r)                                      \
                if (RD(r) == x && ((r) < 4 ? (r) < (NB_) : (NB_) > 0)) {                       \
                    FRAG_READ(r, AN, BN_, nA, nB, cn)                                          \
                }                                                                              \
            __builtin_amdgcn_sched_barrier(0);                                                 \
            HOOK(x);                                                                           \
            __builtin_amdgcn_sched_barrier(0);                                                 \
            if ((NB_) > (x >> 2))                                                              \
                acc[x >> 2][x & 3] = mma<TRANS>(AC[x >> 2], BC[x & 3], acc[x >> 2][x & 3], EA[x >> 2], \
                                                EB[x & 3]);                                    \
            __builtin_amdgcn_sched_barrier(0);                                                 \
            DMA(x);                                                                            \
            __builtin_amdgcn_sched_barrier(0);                                                 \
        }

        // A_0, B_0 (and stage 0's scales) landed for every wave; behind them
        // this wave may have queued the previous register epilogue's stores.
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (TRANS && !first)
            wait_vmcnt_lds<(16 + kEpiStores < 63 ? 16 + kEpiStores : 63)>();
        else
            wait_vmcnt_lds<16>();
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        B_RSRC()
        const int live = m_end - m0 - wm * 128;
        i32x8 a0[4], b0[4], a1[4], b1[4];
        {
            const uint8_t *sA = UNIT(0), *sB = UNIT(1);  // A_0, B_0: step 0's fragments
#pragma unroll
            for (int i = 0; i < 4; ++i) a0[i] = frag32(sA, wm * 128 + i * 32 + (lane & 31), 2 * g);
#pragma unroll
            for (int j = 0; j < 4; ++j) b0[j] = frag32(sB, B_ROW(j), 2 * g);
        }

        // Stage kt: step 0 (K bytes 0-63 of the rows: pieces 2g, 2g+1) then
        // step 1 (pieces 4 + 2g, 5 + 2g).  The ring's five units hold A_kt,
        // B_kt, A_{kt+1}, B_{kt+1} and A_{kt+2} (in flight).  Step 0 reads
        // step 1's fragments, B's first; once every wave has them, a barrier
        // frees B_kt's unit and B_{kt+2} streams into it.  Once A_{kt+1} and
        // B_{kt+1} have landed, a second barrier makes them visible and frees
        // A_kt's unit: step 1 streams A_{kt+3} into it and reads stage kt+1's
        // first fragments.  One load per MFMA or two, eight per step, and each
        // has two steps or more to land.  (Stage 0 also issues A_2, in step 0:
        // the fifth unit serves the epilogue until the tile starts.)  Stage
        // kt+1's scales are loaded first.
#define RD_S0(r) ((r) < 4 ? 5 + (r) : (r) - 4)
#define RD_S1(r) (2 * (r))
#define HOOK_S0(x)                                                                             \
        if ((x) == 4) {                                                                        \
            __atomic_signal_fence(__ATOMIC_SEQ_CST);                                           \
            wait_vmcnt_lds<63>(); /* this wave's B_kt reads done */                            \
            __builtin_amdgcn_s_barrier();                                                      \
            __atomic_signal_fence(__ATOMIC_SEQ_CST);                                           \
        }
#define HOOK_S1(x)
#define DMA_S0(x)                                                                              \
        if ((x) < 8 && kt == 0) ISSUE_A(2, (x), UNIT(uF));                                    \
        if ((x) >= 6 && (x) < 14) ISSUE_B(kt + 2, (x) - 6, fB)
#define DMA_S1(x) if (((x) & 1) == 0) ISSUE_A(kt + 3, (x) >> 1, fA)
        // At least this many loads a wave issues after B_{kt+1}: A_{kt+2},
        // stage kt+1's A-row (and, K-grouped, B-row) scale bytes, B_{kt+2}
        // (the weight block scales may add one or two more).
        constexpr int kStageWait = 16 + (KG ? 8 : 4);
#define KLOOP(NB_)                                                                             \
        {                                                                                      \
            int uA = 0, uB = 1, uNA = 2, uNB = 3, uF = 4; /* ring units */                     \
            for (int kt = 0; kt < nk; ++kt) {                                                  \
                const uint8_t *cA = UNIT(uA), *cB = UNIT(uB);                                  \
                uint8_t *fA = UNIT(uA), *fB = UNIT(uB); /* A_{kt+3}, B_{kt+2} */               \
                int ea_[4], eb_[4];                                                            \
                _Pragma("unroll") for (int i = 0; i < 4; ++i) ea_[i] = sa[i];                  \
                /* B exponents per column block: per lane (K-grouped rows) or the block's */   \
                _Pragma("unroll") for (int j = 0; j < 4; ++j)                                  \
                    eb_[j] = KG ? sb[j] : sw[DUAL && j >= 2 ? 1 : 0];                          \
                LOAD_SCALES(kt + 1, sa_n, sw_n, sb_n);                                         \
                STEP(a0, b0, a1, b1, cA, cB, 4 + 2 * g, RD_S0, HOOK_S0, DMA_S0, NB_, ea_, eb_); \
                __atomic_signal_fence(__ATOMIC_SEQ_CST);                                       \
                wait_vmcnt_lds<kStageWait>(); /* A_{kt+1}, B_{kt+1} landed for this wave */    \
                __builtin_amdgcn_s_barrier(); /* ... for all waves; A_kt no longer read */     \
                __atomic_signal_fence(__ATOMIC_SEQ_CST);                                       \
                const uint8_t *nA = UNIT(uNA), *nB = UNIT(uNB);                                \
                STEP(a1, b1, a0, b0, nA, nB, 2 * g, RD_S1, HOOK_S1, DMA_S1, NB_, ea_, eb_);    \
                _Pragma("unroll") for (int i = 0; i < 4; ++i) sa[i] = sa_n[i];                 \
                _Pragma("unroll") for (int j = 0; j < 4; ++j) sb[j] = sb_n[j];                 \
                sw[0] = sw_n[0];                                                               \
                sw[1] = sw_n[1];                                                               \
                const int fr_ = uA;                                                            \
                uA = uNA;                                                                      \
                uNA = uF;                                                                      \
                uF = fr_;                                                                      \
                const int nb_ = uB;                                                            \
                uB = uNB;                                                                      \
                uNB = nb_;                                                                     \
            }                                                                                  \
        }
        switch (live <= 0 ? 0 : live >= 128 ? 4 : (live + 31) / 32) {
            case 4: KLOOP(4) break;
            case 3: KLOOP(3) break;
            case 2: KLOOP(2) break;
            case 1: KLOOP(1) break;
            default: KLOOP(0) break;
        }
#undef KLOOP
#undef RD_S0
#undef RD_S1
#undef HOOK_S0
#undef HOOK_S1
#undef DMA_S0
#undef DMA_S1
#undef STEP
#undef FRAG_READ
#undef B_ROW
        __syncthreads();  // every wave done with the ring (and its loads landed)
        first = false;
        const int cm0 = m0, cm_end = m_end, cn0 = n0, ce = e;  // this tile, for its epilogue
        const int c4 = 4 * g;

        if constexpr (TRANS) {
            // The ring's first four units take the next tile's first two
            // stages now, so they land while the epilogue runs.
            if (t + tstep < tlim) {
                TILE_SETUP(t + tstep);
                PROLOGUE_LOADS();
            }
            // Lane: tile rows wm*128 + 32i + (lane & 31); per 32-column block,
            // 4 runs of 4 consecutive columns.  Every lane issues every store
            // (padding rows, and lanes that do not own a scale, get an offset
            // past the end of the resource, which the hardware drops).
            if constexpr (DUAL) {
                // h = silu(g) u; the tile's 128 h columns are one quantisation
                // tile: this wave's 64 (both lane halves), then the other
                // column wave's through the free fifth unit
                // h is formed once and kept in registers (the K loop's fragment
                // registers are free here) for the quantisation pass
                float *xch = reinterpret_cast<float *>(UNIT(4));  // [2][256] row amax
                float am[4];
                float hv[4][2][16];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float m = 0.f;
#pragma unroll
                    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            hv[i][jj][r] = swiglu(acc_read(acc[i][jj][r]), acc_read(acc[i][2 + jj][r]));
                            m = fmaxf(m, fabsf(hv[i][jj][r]));
                        }
                    m = fmaxf(m, __shfl_xor(m, 32, 64));
                    am[i] = m;
                    if (g == 0) xch[wn * 256 + wm * 128 + 32 * i + lane] = m;
                }
                // LDS only: the next tile's loads (issued above) stay in flight
                __atomic_signal_fence(__ATOMIC_SEQ_CST);
                wait_vmcnt_lds<63>();
                __builtin_amdgcn_s_barrier();
                __atomic_signal_fence(__ATOMIC_SEQ_CST);
                const __amdgpu_buffer_rsrc_t rQ = buf_rsrc(p.hq, (uint32_t)p.M * (uint32_t)p.N);
                const __amdgpu_buffer_rsrc_t rS = buf_rsrc(p.hs, (uint32_t)p.M * (uint32_t)(p.N / 128));
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int tr = wm * 128 + 32 * i + (lane & 31);
                    const int row = cm0 + tr;
                    const float s = e4m3_tile_scale(fmaxf(am[i], xch[(wn ^ 1) * 256 + tr]));
                    const float inv = 1.0f / s;  // a power of two: h * inv == h / s exactly
                    const bool ok = row < cm_end;
                    const uint32_t qbase = ok ? (uint32_t)row * (uint32_t)p.N + (uint32_t)cn0 : kOobOff;
#pragma unroll
                    for (int jj = 0; jj < 2; ++jj) {
                        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const uint32_t w = e4m3x4(hv[i][jj][4 * q] * inv, hv[i][jj][4 * q + 1] * inv,
                                                      hv[i][jj][4 * q + 2] * inv, hv[i][jj][4 * q + 3] * inv);
                            const int col = wn * 64 + jj * 32 + 8 * q + c4;
                            __builtin_amdgcn_raw_buffer_store_b32((int)w, rQ, qbase + (uint32_t)col, 0, 0);
                        }
                    }
                    const uint32_t so = (ok && wn == 0 && g == 0)
                                            ? (uint32_t)(cn0 / 128) * (uint32_t)p.M + (uint32_t)row
                                            : kOobOff;
                    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)e8m0_of(s), rS, so, 0, 0);
                }
            } else if constexpr (EPI == MX_STORE) {
                const __amdgpu_buffer_rsrc_t rOut = buf_rsrc(p.out, (uint32_t)p.M * (uint32_t)p.N * 2u);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = cm0 + wm * 128 + 32 * i + (lane & 31);
                    const uint32_t obase = row < cm_end ? ((uint32_t)row * (uint32_t)p.N + (uint32_t)cn0) * 2u : kOobOff;
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        __builtin_amdgcn_sched_barrier(0);
                        // w[q]: columns 8q + c4 .. +3 of the block as bf16.
                        // Lanes l and l + 32 hold one row; swapping w[2h+1]
                        // of lanes 0-31 with w[2h] of lanes 32-63 leaves
                        // each lane 8 consecutive columns, 16h + 8g .. +7,
                        // stored as one 16 bytes.
                        uint32_t w[4][2];
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            w[q][0] = pack_bf16x2(acc_read(acc[i][jj][4 * q]), acc_read(acc[i][jj][4 * q + 1]));
                            w[q][1] = pack_bf16x2(acc_read(acc[i][jj][4 * q + 2]), acc_read(acc[i][jj][4 * q + 3]));
                        }
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
#pragma unroll
                            for (int k = 0; k < 2; ++k) {
                                const auto sw2 = __builtin_amdgcn_permlane32_swap(w[2 * h][k], w[2 * h + 1][k], false, false);
                                w[2 * h][k] = sw2[0];
                                w[2 * h + 1][k] = sw2[1];
                            }
                            const int col = wn * 128 + jj * 32 + 16 * h + 8 * g;
                            __builtin_amdgcn_raw_buffer_store_b128(
                                i32x4{(int)w[2 * h][0], (int)w[2 * h][1], (int)w[2 * h + 1][0], (int)w[2 * h + 1][1]}, rOut,
                                obase + (uint32_t)col * 2u, 0, 0);
                        }
                    }
                }
            } else {
                const __amdgpu_buffer_rsrc_t rOutF =
                    buf_rsrc(KG ? uniform_ptr(p.yout + (size_t)ce * p.cstride) : p.yout, (uint32_t)p.M * (uint32_t)p.ldo * 4u);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = cm0 + wm * 128 + 32 * i + (lane & 31);
                    const uint32_t obase = row < cm_end ? ((uint32_t)row * (uint32_t)p.ldo + (uint32_t)cn0) * 4u : kOobOff;
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const int col = wn * 128 + jj * 32 + 8 * q + c4;
                            __builtin_amdgcn_raw_buffer_store_b128(
                                i32x4{__float_as_int(acc_read(acc[i][jj][4 * q])), __float_as_int(acc_read(acc[i][jj][4 * q + 1])),
                                      __float_as_int(acc_read(acc[i][jj][4 * q + 2])),
                                      __float_as_int(acc_read(acc[i][jj][4 * q + 3]))},
                                rOutF, obase + (uint32_t)col * 4u, 0, 0);
                        }
                    }
                }
            }
        } else {
            // Combine epilogue: four 64-row chunks of the fp32 tile through
            // LDS, so every y_perm gather and y store is a 16-byte access.
            // The tile's routed-row indices and combine weights (256 rows x
            // 8) go to LDS first, one 16-byte load pair per thread, so each
            // gather depends on one global round trip instead of two; rows
            // past the group's end are clamped to its last row (every load
            // is valid, only the stores are skipped), which lets the gathers
            // of several rows be in flight at once.
            float *ch = reinterpret_cast<float *>(smem);
            int *sro = reinterpret_cast<int *>(reinterpret_cast<uint8_t *>(smem) + kChRows * kChLd * 4);  // [256][8]
            float *scw = reinterpret_cast<float *>(sro + 256 * 8);            // [256][8]
            {
                const int rr = min(cm0 + tid, cm_end - 1);
                const i32x4 *ro = reinterpret_cast<const i32x4 *>(p.row_of + (size_t)rr * 8);
                const f32x4 *wo = reinterpret_cast<const f32x4 *>(p.cw + (size_t)rr * 8);
                const i32x4 r0 = ro[0], r1 = ro[1];
                const f32x4 w0 = wo[0], w1 = wo[1];
                *reinterpret_cast<i32x4 *>(sro + tid * 8) = r0;
                *reinterpret_cast<i32x4 *>(sro + tid * 8 + 4) = r1;
                *reinterpret_cast<f32x4 *>(scw + tid * 8) = w0;
                *reinterpret_cast<f32x4 *>(scw + tid * 8 + 4) = w1;
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                if (wm == (c >> 1)) {
#pragma unroll
                    for (int ii = 0; ii < 2; ++ii) {
                        const int i = 2 * (c & 1) + ii;
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const int col = wn * 128 + j * 32 + (lane & 31);
#pragma unroll
                            for (int r = 0; r < 16; ++r)
                                ch[(ii * 32 + 8 * (r >> 2) + 4 * g + (r & 3)) * kChLd + col] = acc[i][j][r];
                        }
                    }
                }
                __syncthreads();
                const int cl = 8 * (lane & 31);
#pragma unroll 4
                for (int it = 0; it < 8; ++it) {
                    const int rl = wave * 16 + 2 * it + g;
                    const int tr = c * kChRows + rl;  // tile row
                    const int row = cm0 + tr;
                    const int trc = min(tr, cm_end - cm0 - 1);
                    int rof[8];
                    float wj[8];
                    {
                        const i32x4 a0 = *reinterpret_cast<const i32x4 *>(sro + trc * 8);
                        const i32x4 a1 = *reinterpret_cast<const i32x4 *>(sro + trc * 8 + 4);
                        const f32x4 b0 = *reinterpret_cast<const f32x4 *>(scw + trc * 8);
                        const f32x4 b1 = *reinterpret_cast<const f32x4 *>(scw + trc * 8 + 4);
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            rof[j] = a0[j];
                            rof[4 + j] = a1[j];
                            wj[j] = b0[j];
                            wj[4 + j] = b1[j];
                        }
                    }
                    i32x4 yv[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        yv[j] = *reinterpret_cast<const i32x4 *>(p.y_perm + (size_t)rof[j] * p.N + cn0 + cl);
                    const float *cr = ch + rl * kChLd + cl;
                    const f32x4 s0 = *reinterpret_cast<const f32x4 *>(cr);
                    const f32x4 s1 = *reinterpret_cast<const f32x4 *>(cr + 4);
                    float v[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
#pragma unroll
                    for (int j = 0; j < 8; ++j)
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            v[2 * u] += wj[j] * bf16_to_f32((uint32_t)yv[j][u] & 0xffffu);
                            v[2 * u + 1] += wj[j] * bf16_to_f32((uint32_t)yv[j][u] >> 16);
                        }
                    if (row < cm_end) {
                        float *yo = p.yout + (size_t)row * p.N + cn0 + cl;
                        *reinterpret_cast<f32x4 *>(yo) = f32x4{v[0], v[1], v[2], v[3]};
                        *reinterpret_cast<f32x4 *>(yo + 4) = f32x4{v[4], v[5], v[6], v[7]};
                    }
                }
                __syncthreads();
            }
            if (t + tstep < tlim) {
                TILE_SETUP(t + tstep);
                PROLOGUE_LOADS();
            }
        }
    }
#undef TILE_SETUP
#undef PROLOGUE_LOADS
#undef LOAD_SCALES
#undef B_RSRC
#undef ISSUE_A
#undef ISSUE_B
#undef UNIT
}

int cu_count_mx() {
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

bool ffn_fp8_mx_ok(const FfnArgs &a) {
    const int groups = a.offsets ? a.E : 1;
    const unsigned long long lim = kOobOff - (1ULL << 20);
    const unsigned long long arows = a.a_rows ? (unsigned long long)a.M / a.a_div : (unsigned long long)a.M;
    const bool fits = arows * a.d < lim && (unsigned long long)a.M * a.I < lim && (unsigned long long)a.I * a.d < lim &&
                      (unsigned long long)a.M * a.d * 4 < lim && (unsigned long long)a.M * a.d * 2 < lim;
    return fits && (long long)a.M >= 128LL * groups && a.I % 256 == 0 && a.d % 256 == 0;
}

// Phase 1 (gate/up, fused SwiGLU + h quantisation) and / or phase 2 (down:
// bf16 y_perm, or the shared expert's output with the weighted combine).
hipError_t launch_ffn_fp8_mx(const FfnArgs &a, hipStream_t s) {
    const int P = (cu_count_mx() / 8) * 8;
    const bool routed = a.offsets != nullptr;
    if (a.phases & 1) {
        MxParams p{};
        p.M = a.M;
        p.offsets = a.offsets;
        p.A = static_cast<const uint8_t *>(a.a);
        p.As = a.a_scale;
        p.as_km = a.a_scale_kmajor;
        p.a_rows = a.a_rows;
        p.a_div = a.a_rows ? a.a_div : 1;
        p.K = a.d;
        p.B0 = static_cast<const uint8_t *>(a.w.gate);
        p.B1 = static_cast<const uint8_t *>(a.w.up);
        p.S0 = a.w.s_gate;
        p.S1 = a.w.s_up;
        p.N = a.I;
        p.hq = static_cast<uint8_t *>(a.h);
        p.hs = a.h_scale;
        if (routed) hipLaunchKernelGGL((k_gemm_fp8_mx<MX_SWIGLU_Q, true>), dim3(P), dim3(256), 0, s, p);
        else hipLaunchKernelGGL((k_gemm_fp8_mx<MX_SWIGLU_Q, false>), dim3(P), dim3(256), 0, s, p);
    }
    if (a.phases & 2) {
        MxParams q{};
        q.M = a.M;
        q.offsets = a.offsets;
        q.A = static_cast<const uint8_t *>(a.h);
        q.As = a.h_scale;
        q.as_km = 1;  // written so by the gate/up epilogue
        q.a_div = 1;
        q.K = a.I;
        q.B0 = static_cast<const uint8_t *>(a.w.down);
        q.S0 = a.w.s_down;
        q.N = a.d;
        if (a.combine) {
            q.yout = static_cast<float *>(a.y);
            q.y_perm = static_cast<const uint16_t *>(a.y_perm);
            q.row_of = a.row_of;
            q.cw = a.cw;
            hipLaunchKernelGGL((k_gemm_fp8_mx<MX_COMBINE, false>), dim3(P), dim3(256), 0, s, q);
            return hipGetLastError();
        }
        q.out = static_cast<uint16_t *>(a.y);
        if (routed) hipLaunchKernelGGL((k_gemm_fp8_mx<MX_STORE, true>), dim3(P), dim3(256), 0, s, q);
        else hipLaunchKernelGGL((k_gemm_fp8_mx<MX_STORE, false>), dim3(P), dim3(256), 0, s, q);
    }
    return hipGetLastError();
}

bool fp8_mx_gemm_ok(const Fp8GemmArgs &g) {
    const int groups = g.offsets ? kE : 1;
    const unsigned long long lim = kOobOff - (1ULL << 20);
    const unsigned long long a_rows = g.a_rows ? (unsigned long long)g.a_src_rows : (unsigned long long)g.M;
    return (long long)g.M >= 128LL * groups && g.N % LB == 0 && g.K % LKB == 0 && a_rows * g.K < lim &&
           a_rows * (g.K / LKB) < lim && (unsigned long long)g.N * g.K < lim &&
           (unsigned long long)g.M * g.ldo * 4 < lim && g.ldo >= g.N && (!g.a_rows || g.M / g.a_div == g.a_src_rows);
}

bool fp8_mx_kg_ok(const Fp8KgArgs &g) {
    const unsigned long long lim = kOobOff - (1ULL << 20);
    return g.M > 0 && g.M % LM == 0 && g.N % LB == 0 && g.K % LKB == 0 && g.ldo >= g.N &&
           (unsigned long long)g.M * g.K < lim && (unsigned long long)g.N * g.K < lim &&
           (unsigned long long)g.M * (g.K / LKB) < lim && (unsigned long long)g.N * (g.K / LKB) < lim &&
           (unsigned long long)g.M * g.ldo * 4 < lim;
}

hipError_t launch_fp8_mx_kg(const Fp8KgArgs &g, hipStream_t s) {
    const int P = (cu_count_mx() / 8) * 8;
    MxParams p{};
    p.M = g.M;
    p.A = g.A;
    p.As = g.As;
    p.a_div = 1;
    p.K = g.K;
    p.B0 = g.B;
    p.Bs = g.Bs;
    p.N = g.N;
    p.yout = g.out;
    p.ldo = g.ldo;
    p.kseg = g.kseg;
    p.cstride = g.cstride;
    hipLaunchKernelGGL((k_gemm_fp8_mx<MX_F32, false, true>), dim3(P), dim3(256), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_fp8_mx_gemm(const Fp8GemmArgs &g, hipStream_t s) {
    const int P = (cu_count_mx() / 8) * 8;
    MxParams p{};
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
    if (g.offsets) hipLaunchKernelGGL((k_gemm_fp8_mx<MX_F32, true>), dim3(P), dim3(256), 0, s, p);
    else hipLaunchKernelGGL((k_gemm_fp8_mx<MX_F32, false>), dim3(P), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace moe
