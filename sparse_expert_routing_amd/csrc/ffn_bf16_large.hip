// Grouped SwiGLU expert GEMMs in bf16 for large groups (prefill): persistent
// workgroups, 256x256 tiles, XCD-aware grouped tile order, LDS-staged
// vectorised epilogues.
//
// Routed experts and their gather/accumulate: Scaling Efficiency: A Deep Dive
// into the DeepSeek-V3 Architecture, "Implementation: A Modular Look"; many
// small routed experts plus one shared expert: DeepSeek V3 From Scratch,
// "The idea".  Gated (SwiGLU) form: our reading (see the C ABI header).
//
// Design for gfx950:
//   - 4 waves in a 2x2 layout, each owning a 128x128 block of the 256x256
//     tile (256 fp32 accumulators per lane, in AGPRs), half the LDS traffic
//     per MFMA of a 64x64 wave tile.  The forward's SwiGLU gate/up and bf16
//     store (k_gemm_bf16_mi16) hold it as 8x8 v_mfma_f32_16x16x32_bf16
//     accumulators, which run the same work at a lower power per FLOP and
//     so at a higher clock under the chip's power limit; the backward's
//     fp32 forms and the combine (k_gemm_bf16_large) as 4x4
//     v_mfma_f32_32x32x16_bf16 accumulators, reading 8 fragments (8 KB) per
//     16 of K;
//   - K stages of 64 (each tile row a whole 128-byte line), the A and B slabs
//     of a stage (32 KB each) in a ring of five LDS units filled straight
//     from global memory by buffer_load_dwordx4 ... lds (a buffer resource
//     per operand, a fixed per-lane offset, the stage offset in an SGPR).  A
//     stage is 4 steps of 16 K; A of stage s+2 streams in during steps 0-2
//     and B of stage s+2 during step 3, after a mid-stage barrier (this
//     wave's loads of stage s+1 landed, s_waitcnt vmcnt) has freed stage s's
//     units: one barrier per stage, loads spread between the MFMAs;
//   - fragments are double-buffered in registers: the next 16-wide K step's
//     8 fragments (the next stage's first step included) are read from LDS
//     while the current step's 16 MFMAs run, pinned by scheduling barriers;
//   - LDS layout: 128-byte rows whose 16-byte pieces are XOR-swizzled with
//     (row & 7) ^ ((row >> 3) & 1), so the 32-row MFMA fragment reads hit
//     distinct banks;
//   - one persistent workgroup per CU; the 32 workgroups an XCD runs together
//     take 32 consecutive tiles.  Routed tiles run expert by expert, inside an
//     expert in groups of at most 8 row tiles with the row tile fastest, so
//     the row tiles that read one weight column slice run side by side in
//     one L2 and no group spans two experts' weights;
//   - the row tile -> (expert, first row) map is computed on the device from
//     `offsets` (a wavefront scan over the 256 experts), never on the host;
//   - register epilogues from the transposed accumulators (the next tile's
//     first two stages already in flight): SwiGLU -> bf16 h, or bf16 y_perm,
//     converted two values per v_cvt_pk_bf16_f32 and stored 16 bytes per
//     lane after a lane-half swap; the shared expert's combine
//     y = acc + sum_j w_j * y_perm[row_of[t*k + j]] in fp32 stages 64-row
//     chunks through LDS so its gathers and stores are 16-byte accesses.
#include "device.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kE = 256;
constexpr int LM = 256;      // rows per tile
constexpr int LB = 256;      // B rows per tile
constexpr int LK = 64;       // K per stage: 128-byte rows (whole L2 lines)
constexpr int NUNIT = 5;     // LDS ring units of one stage operand (5 x 32 KB)
// A buffer-load byte offset past the end of every operand (the host keeps
// operands below kOobOff - 1 MB, and a stage offset, < 1 MB, added to it
// stays below 2^32): such a load fetches nothing.
constexpr uint32_t kOobOff = 0xFFFF0000u;
constexpr int UNIT_ELEMS = LM * LK;
static_assert(LM == LB, "A and B stage slabs share the unit size");
constexpr int kGroupM = 8;   // row tiles per ordering group
constexpr int kChRows = 64;  // epilogue chunk rows
constexpr int kChLd = LB + 4;

// EPI_PRE / EPI_F32: fp32 outputs (the layer backward's GEMMs): the gate and up
// pre-activations of a SwiGLU tile, or a plain fp32 product.
enum { EPI_SWIGLU = 0, EPI_STORE = 1, EPI_COMBINE = 2, EPI_PRE = 3, EPI_F32 = 4 };

struct LargeParams {
    int M;
    const int32_t *offsets;
    const uint16_t *A;
    const int32_t *a_rows;  // optional row indirection into A: row a_rows[r] / a_div
    int a_div;
    int K;
    const uint16_t *B0, *B1;
    int N;
    uint16_t *out;
    float *yout;
    const uint16_t *y_perm;
    const int32_t *row_of;
    const float *cw;
    int k;
    float *outf;  // EPI_PRE / EPI_F32: fp32 output, row stride ldo; EPI_PRE puts up at column + up_off
    int ldo, up_off;
    // K-grouped form (weight gradients): group e reduces over K in
    // [kseg[e], kseg[e+1]) (multiples of 64) of A [M, ldk] and B [N, ldk],
    // into outf + e * cstride; groups with an empty range are skipped
    const int32_t *kseg;
    int ldk;
    int64_t cstride;
    // B stored K-major ([K, N] per group, N contiguous): K rows [0, ksplit)
    // come from B0 [G, ksplit, N] and [ksplit, K) from B1 (ksplit 0: all of
    // K from B0 [G, K, N])
    int ksplit;
};

// Row-tile map: lane owns experts 4*lane .. 4*lane+3.
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
// non-empty K range has `per` tiles.
__device__ __forceinline__ void kgmap_init(TileMap &tm, const int32_t *__restrict__ kseg, int per) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < 5; ++i) tm.off[i] = kseg[lane * 4 + i];
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

// Element offset, inside one stage operand region, of the 16-byte piece c
// (K elements 8c .. 8c+7) of tile row `row`: rows are 128 bytes; piece c is
// stored at position c ^ (row & 7) ^ ((row >> 3) & 1), so 8 consecutive rows
// (32 banks) and 16 consecutive rows (64 banks) reading one logical piece hit
// distinct banks.
__device__ __forceinline__ int lds_piece(int row, int c) {
    return row * LK + ((c ^ (row & 7) ^ ((row >> 3) & 1)) * 8);
}

// Wait until at most N of this wave's vector-memory operations are
// outstanding and all its LDS operations are done (expcnt unconstrained).
template <int N>
__device__ __forceinline__ void wait_vmcnt_lds() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef int i32x2 __attribute__((ext_vector_type(2)));

// Raw buffer resource over `bytes` bytes at p (gfx9 descriptor word 3).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}

// A pointer the caller knows to be wave-uniform, in scalar registers: a
// buffer resource built from it then needs no per-lane (waterfall) loop.
__device__ __forceinline__ const void *uniform_ptr(const void *p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<const void *>(((uint64_t)hi << 32) | lo);
}

// One 1 KB block (8 rows of 128 B) of a stage operand, global -> LDS
// (buffer_load_dwordx4 ... lds): the operand's resource and the stage's
// byte offset live in scalar registers, the lane's byte offset in a fixed
// VGPR, so a stage's loads need no vector address arithmetic.
__device__ __forceinline__ void dma_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint16_t *lds_block) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)(lds_block), 16, voff, soff, 0, 0);
}

// The same load issued from inline assembly, for the K-major B form: the
// compiler does not see these LDS writes, so it adds no wait for them before
// the transposing LDS reads (for which it cannot tell the units apart and
// would wait on every load in flight).  The kernel's own vmcnt waits and
// barriers order them, as they do the builtin's.  The LDS address goes in
// through an M0 operand, so the compiler itself writes M0 for the block
// (and knows it does); the s_nop covers the M0 write -> LDS DMA hazard.
__device__ __forceinline__ void dma_asm(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint16_t *lds_block) {
    const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t *)(lds_block));
    const uint32_t so = __builtin_amdgcn_readfirstlane(soff);
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                 :
                 : "v"(voff), "s"(r), "s"(so), "{m0}"(lds)
                 : "memory");
}

template <bool ASM>
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint16_t *lds_block) {
    if constexpr (ASM) dma_asm(r, voff, soff, lds_block);
    else dma_buf(r, voff, soff, lds_block);
}

// acc += A_frag x B_frag^T.  TRANS swaps the operands, so the accumulator
// holds the transposed 32x32 block: lane l then owns tile row l % 32 and, in
// registers 4q .. 4q+3, the 4 consecutive tile columns 8q + 4(l / 32) .. +3,
// which the epilogue stores straight from registers.
template <bool TRANS>
__device__ __forceinline__ f32x16 mma(bf16x8 a, bf16x8 b, f32x16 c) {
    if constexpr (TRANS) return __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c, 0, 0, 0);
    else return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// One accumulator element, copied from its AGPR where it is used: left to
// the compiler, every accumulator is copied to VGPRs at the loop exit,
// which needs 256 VGPRs and spills the tile loop's state.
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 *lds_v4i16_t;

// K-major B unit: 64 K rows of LB columns; the 16-byte piece c of row k sits
// at position c ^ 4 (k % 4).  B fragment (32 columns from ncol0, K values
// 16 ks + 8 (lane / 32) .. +7 of column ncol0 + lane % 32) from two
// transposing reads: within each 16 lanes, lane 4a + c receives element c of
// the 8 bytes that lanes a, a+4, a+8, a+12 point at, so lane s points at row
// 16 ks + 8 (s / 32) + (s % 16) / 4 (+ 4 for the second read), columns
// ncol0 + 16 ((s / 16) % 2) + 4 (s % 4) .. +3.
__device__ __forceinline__ int kn_off(int k, int col) { return k * LB + ((((col >> 3) ^ (4 * (k & 3))) << 3) | (col & 7)); }

__device__ __forceinline__ bf16x8 frag_kn(const uint16_t *unit, int ks, int ncol0, int lane) {
    const int h = lane >> 4, a = lane & 15;
    const int k = 16 * ks + 8 * (h >> 1) + (a >> 2);
    const int off = kn_off(k, ncol0 + 16 * (h & 1) + 4 * (a & 3));
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t)(unit + off));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t)(unit + off + 4 * LB));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ float acc_read(float x) {
    float r;
    asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(r) : "a"(x));
    return r;
}

// silu(g) * u in fp32 from the hardware exp2 and reciprocal (about 1 ulp
// each; the product is rounded to bf16 next).
__device__ __forceinline__ float swiglu(float g, float u) {
    return g * u * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * g));
}

template <int EPI, bool ROUTED, bool KG = false, bool BKN = false>
__global__ __launch_bounds__(256, 1) void k_gemm_bf16_large(LargeParams p) {
    static_assert(!BKN || (EPI == EPI_F32 && !KG), "K-major B: plain fp32 products only");
    constexpr bool DUAL = EPI == EPI_SWIGLU || EPI == EPI_PRE;
    constexpr bool TRANS = EPI != EPI_COMBINE;  // register epilogue (no LDS staging)
    constexpr int BN = DUAL ? LB / 2 : LB;  // output columns per tile
    // buffer stores per lane per register epilogue
    constexpr int kEpiStores = TRANS ? (EPI == EPI_SWIGLU ? 16 : EPI == EPI_STORE ? 32 : 64) : 0;
    __shared__ __attribute__((aligned(1024))) uint16_t smem[NUNIT * UNIT_ELEMS];  // 160 KB

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: LDS bases stay scalar
    const int wm = wave >> 1, wn = wave & 1, g = lane >> 5;
    const int K = p.K;
    const int ldk = KG ? p.ldk : K;  // row stride of A and B (elements)
    int nk = K / LK;                 // K-grouped: set per tile

    TileMap tm;
    int Mt, total;
    const int NT = p.N / BN;
    if (ROUTED) {
        tilemap_init(tm, p.offsets);
        Mt = tm.total;
        total = Mt * NT;
    } else if (KG) {
        Mt = p.M / LM;
        kgmap_init(tm, p.kseg, Mt * NT);
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
        dcol[i] = ((lane & 7) ^ (row & 7) ^ ((row >> 3) & 1)) * 8;
    }

    // State of the tile about to run (TILE_SETUP): expert, rows, columns,
    // its B matrices and the per-lane byte offsets of its DMA blocks.
    int e = 0, m0 = 0, m_end = 0, n0 = 0, kbase = 0;
    const uint32_t a_rows_total = p.a_rows ? (uint32_t)(p.M / p.a_div) : (uint32_t)p.M;
    const __amdgpu_buffer_rsrc_t rA = buf_rsrc(p.A, a_rows_total * (uint32_t)ldk * 2u);
    const int kb_rows = BKN && p.ksplit ? p.ksplit : K;           // K-major B: K rows per matrix
    const uint32_t b_bytes = (uint32_t)p.N * (uint32_t)(BKN ? kb_rows : ldk) * 2u;  // one expert's B matrix
    const uint16_t *pBg = p.B0, *pBu = p.B1;                     // the tile's expert
    uint32_t aoff[8], boff[8];

    // LDS ring of NUNIT operand units: operand j of the tile's sequence
    // A_0, B_0, A_1, B_1, ... (A_s / B_s: the A / B slab of stage s) lives
    // in unit j % NUNIT.  Loads past the last stage are clamped to it:
    // they fill units that are never read as that stage, which keeps
    // every load and read unconditional.
#define UNIT(u) (smem + (u) * UNIT_ELEMS)
#define ISSUE_A(st_, i, unit_)                                                                 \
        dma16<BKN>(rA, aoff[i], (uint32_t)min((st_), nk - 1) * (LK * 2), (unit_) + (wave + 4 * (i)) * 512)
    // ISSUE_B reads rBg_ / rBu_: the B resources of the tile whose loads are
    // being issued, built once per tile in scalar registers.
#define B_RSRC()                                                                               \
        const __amdgpu_buffer_rsrc_t rBg_ = buf_rsrc(uniform_ptr(pBg), b_bytes);               \
        const __amdgpu_buffer_rsrc_t rBu_ = (DUAL || BKN) ? buf_rsrc(uniform_ptr(pBu), b_bytes) : rBg_;
    // K-major B: stage st's 64 rows start at row st*LK of B0, or of B1 past ksplit
#define B_UP(st_) (BKN && p.ksplit && min((st_), nk - 1) * LK >= p.ksplit)
#define ISSUE_B(st_, i, unit_)                                                                 \
        dma16<BKN>((B_UP(st_) || (DUAL && (i) >= 4)) ? rBu_ : rBg_, boff[i],                    \
                BKN ? (uint32_t)(min((st_), nk - 1) * LK - (B_UP(st_) ? p.ksplit : 0)) * (uint32_t)p.N * 2u \
                    : (uint32_t)min((st_), nk - 1) * (LK * 2),                                 \
                (unit_) + (wave + 4 * (i)) * 512)
    // Tile tt -> (e, m0, m_end, n0), B matrices (DMA block i of B comes
    // from the up matrix for i >= 4 in the SwiGLU tile: rows 128..255 of its
    // B operand) and DMA offsets.
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
            kbase = __builtin_amdgcn_readfirstlane(p.kseg[e]);                                 \
            nk = __builtin_amdgcn_readfirstlane((p.kseg[e + 1] - kbase) / LK);                 \
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
        pBg = KG ? p.B0 : p.B0 + (size_t)e * p.N * (BKN ? kb_rows : K);                       \
        pBu = DUAL ? p.B1 + (size_t)e * p.N * K : (BKN && p.ksplit) ? p.B1 + (size_t)e * p.N * kb_rows : pBg; \
        int ar_[8];                                                                            \
        _Pragma("unroll") for (int i = 0; i < 8; ++i) ar_[i] = min(m0 + drow[i], m_end - 1);    \
        if (p.a_rows) { /* 8 independent lookups, issued together */                            \
            _Pragma("unroll") for (int i = 0; i < 8; ++i) ar_[i] = p.a_rows[ar_[i]];            \
            _Pragma("unroll") for (int i = 0; i < 8; ++i) ar_[i] /= p.a_div;                    \
        }                                                                                      \
        _Pragma("unroll") for (int i = 0; i < 8; ++i) {                                        \
            aoff[i] = ((uint32_t)ar_[i] * (uint32_t)ldk + (uint32_t)(dcol[i] + kbase)) * 2u;   \
            const int r = drow[i];                                                             \
            const int br = DUAL ? n0 + (r & (BN - 1)) : n0 + r;                                \
            boff[i] = ((uint32_t)br * (uint32_t)ldk + (uint32_t)(dcol[i] + kbase)) * 2u;       \
            if (BKN) { /* 1 KB block = K rows 2 blk, 2 blk + 1; lane: physical piece lane % 32 */ \
                const int kr_ = 2 * (wave + 4 * i) + (lane >> 5);                              \
                const int pc_ = (lane & 31) ^ (4 * (kr_ & 3));                                 \
                boff[i] = ((uint32_t)kr_ * (uint32_t)p.N + (uint32_t)(n0 + 8 * pc_)) * 2u;     \
            }                                                                                  \
            /* rows past the group's end: an offset past the A resource, so the */             \
            /* load fetches nothing (their outputs are dropped) */                              \
            if (m0 + r >= m_end) aoff[i] = kOobOff;                                             \
        }                                                                                      \
    }
    // A_0, B_0, A_1, B_1 of the tile just set up (32 loads per wave).
#define PROLOGUE_LOADS()                                                                       \
    {                                                                                          \
        B_RSRC()                                                                               \
        _Pragma("unroll") for (int i = 0; i < 8; ++i) ISSUE_A(0, i, UNIT(0));                  \
        _Pragma("unroll") for (int i = 0; i < 8; ++i) ISSUE_B(0, i, UNIT(1));                  \
        _Pragma("unroll") for (int i = 0; i < 8; ++i) ISSUE_A(1, i, UNIT(2));                  \
        _Pragma("unroll") for (int i = 0; i < 8; ++i) ISSUE_B(1, i, UNIT(3));                  \
    }

    int t = (blockIdx.x & 7) * (P >> 3) + (blockIdx.x >> 3);
    if (t < total) {
        TILE_SETUP(t);
        PROLOGUE_LOADS();
    }
    bool first = true;
    for (; t < total; t += P) {
        f32x16 acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

#define READ_AT(r) (2 * (r))
#define B_ROW(j) ((DUAL ? (((j) >> 1) * 128 + wn * 64 + ((j) & 1) * 32) : (wn * 128 + (j) * 32)) + (lane & 31))

        // One 16-wide K step: 16 MFMAs on (AC, BC).  The next step's 8
        // fragments (from the units nA / nB at piece column cn into AN, BN_)
        // are read at READ_AT(r) (before MFMA READ_AT(r); only those of the
        // NB_ live row blocks), the load DMA(x) (if any) right after MFMA
        // x.  The order is fixed by scheduling
        // barriers: a slot load blocks this wave's issue for up to about one
        // MFMA's duration, so loads are spread between MFMAs rather than
        // issued back to back.
#define FRAG_READ(r, AN, BN_, nA, nB, cn)                                                      \
        if ((r) < 4)                                                                           \
            AN[(r) & 3] = *reinterpret_cast<const bf16x8 *>((nA) + lds_piece(wm * 128 + ((r) & 3) * 32 + (lane & 31), (cn))); \
        else if (BKN)                                                                          \
            BN_[(r) & 3] = frag_kn((nB), (cn) >> 1, wn * 128 + ((r) & 3) * 32, lane);          \
        else                                                                                   \
            BN_[(r) & 3] = *reinterpret_cast<const bf16x8 *>((nB) + lds_piece(B_ROW((r) & 3), (cn)));
#define STEP(AC, BC, AN, BN_, nA, nB, cn, DMA, NB_)                                            \
        _Pragma("unroll") for (int x = 0; x < 16; ++x) {                                       \
            _Pragma("unroll") for (int r = 0; r < 8; ++r)                                      \
                if (READ_AT(r) == x && ((r) < 4 ? (r) < (NB_) : (NB_) > 0)) {                  \
                    FRAG_READ(r, AN, BN_, nA, nB, cn)                                          \
                }                                                                              \
            __builtin_amdgcn_sched_barrier(0);                                                 \
            if ((NB_) > (x >> 2)) /* 32-row blocks wholly past the group's end: no MFMA */       \
                acc[x >> 2][x & 3] = mma<TRANS>(AC[x >> 2], BC[x & 3], acc[x >> 2][x & 3]);     \
            __builtin_amdgcn_sched_barrier(0);                                                 \
            DMA(x);                                                                            \
            __builtin_amdgcn_sched_barrier(0);                                                 \
        }

        // A_0, B_0, A_1, B_1 are in flight (issued before the previous tile's
        // epilogue, or before the loop): wait until A_0 and B_0 landed for
        // every wave, then read the first step's fragments.  Behind those
        // loads this wave may have queued the previous register epilogue's
        // stores (kEpiStores of them, always all issued); memory operations
        // retire in order, so at most 16 + kEpiStores may remain.
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (TRANS && !first)
            wait_vmcnt_lds<(16 + kEpiStores < 63 ? 16 + kEpiStores : 63)>();
        else
            wait_vmcnt_lds<16>();
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        B_RSRC()  // this tile's B resources, for the loads of stages 2..
        // Rows of this wave's 128 that belong to the group (wave-uniform):
        // the MFMAs and A fragment reads of a 32-row block with none are
        // left out, and a wave with no rows reads no B fragments either
        // (its slot loads still run, keeping the schedule and barriers).
        const int live = m_end - m0 - wm * 128;
        bf16x8 a0[4], b0[4], a1[4], b1[4];
        {
            const uint16_t *sA = UNIT(0), *sB = UNIT(1);  // A_0, B_0
#pragma unroll
            for (int i = 0; i < 4; ++i)
                a0[i] = *reinterpret_cast<const bf16x8 *>(sA + lds_piece(wm * 128 + i * 32 + (lane & 31), g));
#pragma unroll
            for (int j = 0; j < 4; ++j)
                b0[j] = BKN ? frag_kn(sB, 0, wn * 128 + j * 32, lane)
                            : *reinterpret_cast<const bf16x8 *>(sB + lds_piece(B_ROW(j), g));
        }

        // Stage kt = 4 steps of 16 K; fragments of step s+1 are read during
        // step s.  Steps 0-2 stream A_{kt+2} into the unit B_{kt-1} left
        // (free since the previous stage's barrier), one load per 6 MFMAs.
        // After step 2 every fragment of stage kt is in registers, so the
        // mid-stage barrier (once A_{kt+1} and B_{kt+1} have landed: only
        // A_{kt+2}'s 8 loads may remain in flight) frees A_kt's and B_kt's
        // units; step 3 streams B_{kt+2} into A_kt's unit, one load per 2
        // MFMAs, and reads stage kt+1's first fragments.  A gets about 1.5
        // stages to arrive, B about one.
        // The K loop, for NB_ (compile-time) 32-row blocks of this wave that
        // hold group rows; u0 = unit of A_kt (2kt mod 5), carried.
#define DMA_S0(x) if ((x) == 2 || (x) == 8 || (x) == 14) ISSUE_A(kt + 2, ((x) - 2) / 6, fA)
#define DMA_S1(x) if ((x) == 4 || (x) == 10) ISSUE_A(kt + 2, 3 + ((x) - 4) / 6, fA)
#define DMA_S2(x) if ((x) == 0 || (x) == 6 || (x) == 12) ISSUE_A(kt + 2, 5 + (x) / 6, fA)
#define DMA_S3(x) if (((x) & 1) == 0) ISSUE_B(kt + 2, (x) >> 1, fB)
#define KLOOP(NB_)                                                                             \
        {                                                                                      \
            int u0 = 0;                                                                        \
            for (int kt = 0; kt < nk; ++kt) {                                                  \
                const int u1 = u0 + 1 - (u0 + 1 >= NUNIT ? NUNIT : 0);                         \
                const int u2 = u0 + 2 - (u0 + 2 >= NUNIT ? NUNIT : 0);                         \
                const int u3 = u0 + 3 - (u0 + 3 >= NUNIT ? NUNIT : 0);                         \
                const int u4 = u0 + 4 - (u0 + 4 >= NUNIT ? NUNIT : 0);                         \
                const uint16_t *cA = UNIT(u0), *cB = UNIT(u1);                                 \
                uint16_t *fA = UNIT(u4), *fB = UNIT(u0); /* A_{kt+2}, B_{kt+2} */              \
                STEP(a0, b0, a1, b1, cA, cB, 2 + g, DMA_S0, NB_);                              \
                STEP(a1, b1, a0, b0, cA, cB, 4 + g, DMA_S1, NB_);                              \
                STEP(a0, b0, a1, b1, cA, cB, 6 + g, DMA_S2, NB_);                              \
                __atomic_signal_fence(__ATOMIC_SEQ_CST);                                       \
                wait_vmcnt_lds<8>();          /* A_{kt+1}, B_{kt+1} landed for this wave */    \
                __builtin_amdgcn_s_barrier(); /* ... for all waves; A_kt, B_kt no longer read */ \
                __atomic_signal_fence(__ATOMIC_SEQ_CST);                                       \
                const uint16_t *nA = UNIT(u2), *nB = UNIT(u3);                                 \
                STEP(a1, b1, a0, b0, nA, nB, g, DMA_S3, NB_);                                  \
                u0 = u2;                                                                       \
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
#undef DMA_S0
#undef DMA_S1
#undef DMA_S2
#undef DMA_S3
#undef STEP
#undef FRAG_READ
#undef READ_AT
#undef B_ROW
        if (BKN) wait_vmcnt_lds<0>();  // loads the compiler does not see
        __syncthreads();  // every wave done with the ring (and its loads landed)
        first = false;
        const int cm0 = m0, cm_end = m_end, cn0 = n0, ce = e;  // this tile, for its epilogue

        if constexpr (TRANS) {
            // The ring is free and this epilogue does not use LDS: start the
            // next tile's loads first, so they land while the epilogue runs.
            if (t + P < total) {
                TILE_SETUP(t + P);
                PROLOGUE_LOADS();
            }
            // Register epilogue: lane owns tile rows wm*128 + 32i + (lane & 31)
            // and, per 32-column block, 4 runs of 4 consecutive columns (bf16
            // outputs: regrouped across the lane halves into 2 runs of 8, one
            // 16-byte buffer store each).  Values are computed for every
            // row (padding rows repeat the group's last row); a padding row's
            // stores get an offset past the end of the output resource, which
            // the hardware drops, so every lane issues every store (the wait
            // count above relies on it) and the epilogue stays one block whose
            // scheduling barriers bound how many accumulators sit in VGPRs.
            const int c4 = 4 * g;
            if constexpr (EPI == EPI_PRE || EPI == EPI_F32) {
                // fp32: one 16-byte store per run of 4 columns (and its up twin);
                // padding rows get kOobOff, which leaves room for the column offsets
                const __amdgpu_buffer_rsrc_t rOutF =
                    buf_rsrc(KG ? uniform_ptr(p.outf + (size_t)ce * p.cstride) : p.outf, (uint32_t)p.M * (uint32_t)p.ldo * 4u);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = cm0 + wm * 128 + 32 * i + (lane & 31);
                    const uint32_t obase = row < cm_end ? ((uint32_t)row * (uint32_t)p.ldo + (uint32_t)cn0) * 4u : kOobOff;
#pragma unroll
                    for (int jj = 0; jj < (DUAL ? 2 : 4); ++jj) {
                        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const int col = (DUAL ? wn * 64 : wn * 128) + jj * 32 + 8 * q + c4;
                            __builtin_amdgcn_raw_buffer_store_b128(
                                i32x4{__float_as_int(acc_read(acc[i][jj][4 * q])), __float_as_int(acc_read(acc[i][jj][4 * q + 1])),
                                      __float_as_int(acc_read(acc[i][jj][4 * q + 2])),
                                      __float_as_int(acc_read(acc[i][jj][4 * q + 3]))},
                                rOutF, obase + (uint32_t)col * 4u, 0, 0);
                            if constexpr (DUAL)
                                __builtin_amdgcn_raw_buffer_store_b128(
                                    i32x4{__float_as_int(acc_read(acc[i][2 + jj][4 * q])),
                                          __float_as_int(acc_read(acc[i][2 + jj][4 * q + 1])),
                                          __float_as_int(acc_read(acc[i][2 + jj][4 * q + 2])),
                                          __float_as_int(acc_read(acc[i][2 + jj][4 * q + 3]))},
                                    rOutF, obase + (uint32_t)(p.up_off + col) * 4u, 0, 0);
                        }
                    }
                }
            } else {
            const __amdgpu_buffer_rsrc_t rOut = buf_rsrc(p.out, (uint32_t)p.M * (uint32_t)p.N * 2u);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = cm0 + wm * 128 + 32 * i + (lane & 31);
                const uint32_t obase =
                    row < cm_end ? ((uint32_t)row * (uint32_t)p.N + (uint32_t)cn0) * 2u : 0xfffff000u;
                const bool blk = cm_end - cm0 - wm * 128 > 32 * i;  // block has rows (uniform)
#pragma unroll
                for (int jj = 0; jj < (DUAL ? 2 : 4); ++jj) {
                    __builtin_amdgcn_sched_barrier(0);
                    // w[q]: columns 8q + c4 .. +3 of the block as bf16
                    uint32_t w[4][2];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        if constexpr (DUAL) {
                            w[q][0] = w[q][1] = 0;
                            if (blk) {  // an empty block's stores are dropped: skip its math
                                float h[4];
#pragma unroll
                                for (int u = 0; u < 4; ++u)
                                    h[u] = swiglu(acc_read(acc[i][jj][4 * q + u]), acc_read(acc[i][2 + jj][4 * q + u]));
                                w[q][0] = pack_bf16x2(h[0], h[1]);
                                w[q][1] = pack_bf16x2(h[2], h[3]);
                            }
                        } else {
                            w[q][0] = pack_bf16x2(acc_read(acc[i][jj][4 * q]), acc_read(acc[i][jj][4 * q + 1]));
                            w[q][1] = pack_bf16x2(acc_read(acc[i][jj][4 * q + 2]), acc_read(acc[i][jj][4 * q + 3]));
                        }
                    }
                    // Lanes l and l + 32 hold one row: swapping w[2h+1] of
                    // lanes 0-31 with w[2h] of lanes 32-63 leaves each lane
                    // the 8 consecutive columns 16h + 8g .. +7.
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
#pragma unroll
                        for (int k = 0; k < 2; ++k) {
                            const auto sw2 = __builtin_amdgcn_permlane32_swap(w[2 * h][k], w[2 * h + 1][k], false, false);
                            w[2 * h][k] = sw2[0];
                            w[2 * h + 1][k] = sw2[1];
                        }
                        const int col = (DUAL ? wn * 64 : wn * 128) + jj * 32 + 16 * h + 8 * g;
                        __builtin_amdgcn_raw_buffer_store_b128(
                            i32x4{(int)w[2 * h][0], (int)w[2 * h][1], (int)w[2 * h + 1][0], (int)w[2 * h + 1][1]}, rOut,
                            obase + (uint32_t)col * 2u, 0, 0);
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
                // Half-wave per row: lanes 0-31 take row 2*it, lanes 32-63 row
                // 2*it+1 of this wave's 16 chunk rows, 8 columns per lane, so
                // each gather of a routed output row is one contiguous 512-byte
                // run (few lines and pages per load instruction).
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
            // LDS free again: the next tile's loads
            if (t + P < total) {
                TILE_SETUP(t + P);
                PROLOGUE_LOADS();
            }
        }
    }
#undef TILE_SETUP
#undef PROLOGUE_LOADS
#undef B_RSRC
#undef ISSUE_A
#undef ISSUE_B
#undef B_UP
#undef UNIT
}

// acc += the 16x16x32 product of two fragments.  A fragment is 16 tile rows
// (lane l: row l % 16) by 32 K (K values 8 (l / 16) .. +7); the operands are
// swapped, so the accumulator holds the transposed 16x16 block: lane l owns
// tile row l % 16 and its 4 consecutive columns 4 (l / 16) .. +3.  Issued
// from inline assembly with the accumulator tied to the destination: with
// the builtin, the register allocator does not keep 64 four-register
// accumulators in place in the 256 AGPRs and shuffles them between MFMAs.
// The compiler still waits for the fragments' LDS reads (asm inputs); the
// accumulators are read only after the tile's K loop, past the barrier.
__device__ __forceinline__ void mma16t(bf16x8 a, bf16x8 b, f32x4 &c) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(b), "v"(a));
}

// The 16-byte piece swizzle of the 16x16 kernel: piece c of tile row `row`
// sits at position c ^ s(row), s(row) = (row & 7) with its two low bits
// swapped, ^ 2 for rows 8-15 of each 16.  A fragment read covers 16 rows and
// 4 consecutive pieces (lanes 16q .. 16q+15: piece 4s + q); the lanes LDS
// serves together (8 of one 32-lane half with the 8 beside them in the
// other, and any 8 or 16 consecutive lanes) then hit distinct banks, where
// the 32x32 kernel's swizzle puts rows r and r ^ 2 with pieces c and c ^ 2
// on the same banks.
__device__ __forceinline__ int swz16(int row) {
    const int r3 = row & 7;
    return ((r3 & 4) | ((r3 & 1) << 1) | ((r3 >> 1) & 1)) ^ (((row >> 3) & 1) << 1);
}
__device__ __forceinline__ int lds_piece16(int row, int c) { return row * LK + ((c ^ swz16(row)) * 8); }

// The forward's SwiGLU gate/up (routed or shared) and routed down (bf16
// store) on the same persistent 256x256 tiles, LDS ring, tile order and
// epilogue placement as k_gemm_bf16_large, with each wave's 128x128 block
// as 8x8 v_mfma_f32_16x16x32_bf16 accumulators instead of 4x4 of
// v_mfma_f32_32x32x16_bf16.  The work per K step is the same, but the
// 16x16 instruction draws less power for the same FLOPs, so the chip holds
// a higher clock under its power limit (register-only loops on every CU:
// about 2.1 GHz against 1.8).  A stage of 64 K is 2 steps of 32.
template <int EPI, bool ROUTED>
__global__ __launch_bounds__(256, 1) void k_gemm_bf16_mi16(LargeParams p) {
    static_assert(EPI == EPI_SWIGLU || EPI == EPI_STORE, "register bf16 epilogues only");
    constexpr bool DUAL = EPI == EPI_SWIGLU;
    constexpr int BN = DUAL ? LB / 2 : LB;      // output columns per tile
    constexpr int kEpiStores = DUAL ? 16 : 32;  // buffer stores per lane per epilogue
    __shared__ __attribute__((aligned(1024))) uint16_t smem[NUNIT * UNIT_ELEMS];  // 160 KB

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int q = lane >> 4, l16 = lane & 15;
    const int K = p.K;
    const int nk = K / LK;

    TileMap tm;
    int Mt, total;
    const int NT = p.N / BN;
    if (ROUTED) {
        tilemap_init(tm, p.offsets);
        Mt = tm.total;
        total = Mt * NT;
    } else {
        Mt = (p.M + LM - 1) / LM;
        total = Mt * NT;
    }
    const int P = gridDim.x;

    int drow[8], dcol[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = 8 * (wave + 4 * i) + (lane >> 3);
        drow[i] = row;
        dcol[i] = ((lane & 7) ^ swz16(row)) * 8;
    }

    int e = 0, m0 = 0, m_end = 0, n0 = 0;
    const uint32_t a_rows_total = p.a_rows ? (uint32_t)(p.M / p.a_div) : (uint32_t)p.M;
    const __amdgpu_buffer_rsrc_t rA = buf_rsrc(p.A, a_rows_total * (uint32_t)K * 2u);
    const uint32_t b_bytes = (uint32_t)p.N * (uint32_t)K * 2u;
    const uint16_t *pBg = p.B0, *pBu = p.B1;
    uint32_t aoff[8], boff[8];

#define UNIT(u) (smem + (u) * UNIT_ELEMS)
#define ISSUE_A(st_, i, unit_) \
        dma_buf(rA, aoff[i], (uint32_t)min((st_), nk - 1) * (LK * 2), (unit_) + (wave + 4 * (i)) * 512)
#define B_RSRC()                                                                               \
        const __amdgpu_buffer_rsrc_t rBg_ = buf_rsrc(uniform_ptr(pBg), b_bytes);               \
        const __amdgpu_buffer_rsrc_t rBu_ = DUAL ? buf_rsrc(uniform_ptr(pBu), b_bytes) : rBg_;
#define ISSUE_B(st_, i, unit_)                                                                 \
        dma_buf((DUAL && (i) >= 4) ? rBu_ : rBg_, boff[i], (uint32_t)min((st_), nk - 1) * (LK * 2), \
                (unit_) + (wave + 4 * (i)) * 512)
#define TILE_SETUP(tt)                                                                         \
    {                                                                                          \
        int mt_, nt_;                                                                          \
        if (ROUTED) {                                                                          \
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
        pBg = p.B0 + (size_t)e * p.N * K;                                                      \
        pBu = DUAL ? p.B1 + (size_t)e * p.N * K : pBg;                                         \
        int ar_[8];                                                                            \
        _Pragma("unroll") for (int i = 0; i < 8; ++i) ar_[i] = min(m0 + drow[i], m_end - 1);    \
        if (p.a_rows) {                                                                        \
            _Pragma("unroll") for (int i = 0; i < 8; ++i) ar_[i] = p.a_rows[ar_[i]];            \
            _Pragma("unroll") for (int i = 0; i < 8; ++i) ar_[i] /= p.a_div;                    \
        }                                                                                      \
        _Pragma("unroll") for (int i = 0; i < 8; ++i) {                                        \
            aoff[i] = ((uint32_t)ar_[i] * (uint32_t)K + (uint32_t)dcol[i]) * 2u;               \
            const int r = drow[i];                                                             \
            const int br = DUAL ? n0 + (r & (BN - 1)) : n0 + r;                                \
            boff[i] = ((uint32_t)br * (uint32_t)K + (uint32_t)dcol[i]) * 2u;                   \
            if (m0 + r >= m_end) aoff[i] = kOobOff;                                             \
        }                                                                                      \
    }
#define PROLOGUE_LOADS()                                                                       \
    {                                                                                          \
        B_RSRC()                                                                               \
        _Pragma("unroll") for (int i = 0; i < 8; ++i) ISSUE_A(0, i, UNIT(0));                  \
        _Pragma("unroll") for (int i = 0; i < 8; ++i) ISSUE_B(0, i, UNIT(1));                  \
        _Pragma("unroll") for (int i = 0; i < 8; ++i) ISSUE_A(1, i, UNIT(2));                  \
        _Pragma("unroll") for (int i = 0; i < 8; ++i) ISSUE_B(1, i, UNIT(3));                  \
    }

    int t = (blockIdx.x & 7) * (P >> 3) + (blockIdx.x >> 3);
    if (t < total) {
        TILE_SETUP(t);
        PROLOGUE_LOADS();
    }
    bool first = true;
    for (; t < total; t += P) {
        f32x4 acc[8][8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

        // B operand rows of column block j (16 columns): the SwiGLU tile's B
        // holds 128 gate rows, then 128 up rows; a wave takes 64 of each.
#define B_ROW16(j) (DUAL ? (((j) >> 2) * 128 + wn * 64 + ((j) & 3) * 16) : (wn * 128 + (j) * 16))
#define FRAG16(unit, row0, pc) (*reinterpret_cast<const bf16x8 *>((unit) + lds_piece16((row0) + l16, (pc))))
        // One 32-wide K step: 64 MFMAs on (AC, BC), row block by row block.
        // The next step's 16 fragments (B first, then A; from the units nA /
        // nB at piece 4 s + lane / 16) are read one per 4 MFMAs; the load
        // DMA(x), if any, follows MFMA x.  Scheduling barriers fix the order.
#define STEP16(AC, BC, AN, BN_, nA, nB, pc, DMA, NB_)                                          \
        _Pragma("unroll") for (int x = 0; x < 64; ++x) {                                       \
            if (((x) & 3) == 0) {                                                              \
                if ((x) < 32) {                                                                \
                    if ((NB_) > 0) BN_[(x) >> 2] = FRAG16((nB), B_ROW16((x) >> 2), (pc));      \
                } else if ((((x) - 32) >> 2) < 2 * (NB_)) {                                    \
                    AN[((x) - 32) >> 2] = FRAG16((nA), wm * 128 + (((x) - 32) >> 2) * 16, (pc)); \
                }                                                                              \
            }                                                                                  \
            __builtin_amdgcn_sched_barrier(0);                                                 \
            if (2 * (NB_) > (x >> 3)) /* 16-row blocks past the group's end: no MFMA */         \
                mma16t(AC[x >> 3], BC[x & 7], acc[x >> 3][x & 7]);                             \
            __builtin_amdgcn_sched_barrier(0);                                                 \
            DMA(x);                                                                            \
            __builtin_amdgcn_sched_barrier(0);                                                 \
        }

        // A_0, B_0 landed for every wave (behind them: A_1, B_1 and maybe the
        // previous epilogue's stores), then step 0's fragments.
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (!first)
            wait_vmcnt_lds<16 + kEpiStores>();
        else
            wait_vmcnt_lds<16>();
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        B_RSRC()
        const int live = m_end - m0 - wm * 128;
        bf16x8 a0[8], b0[8], a1[8], b1[8];
        {
            const uint16_t *sA = UNIT(0), *sB = UNIT(1);
#pragma unroll
            for (int i = 0; i < 8; ++i) a0[i] = FRAG16(sA, wm * 128 + i * 16, q);
#pragma unroll
            for (int j = 0; j < 8; ++j) b0[j] = FRAG16(sB, B_ROW16(j), q);
        }

        // Stage kt = 2 steps of 32 K.  Step 0 streams A_{kt+2} into the free
        // unit and reads step 1's fragments; then every fragment of stage kt
        // is in registers, so the barrier (once A_{kt+1} and B_{kt+1} landed:
        // only A_{kt+2}'s 8 loads may remain in flight) frees A_kt's and
        // B_kt's units.  Step 1 streams B_{kt+2} into A_kt's unit and reads
        // stage kt+1's first fragments.
#define DMA16_S0(x) if (((x) & 7) == 2) ISSUE_A(kt + 2, (x) >> 3, fA)
#define DMA16_S1(x) if (((x) & 7) == 2) ISSUE_B(kt + 2, (x) >> 3, fB)
#define KLOOP16(NB_)                                                                           \
        {                                                                                      \
            int u0 = 0;                                                                        \
            for (int kt = 0; kt < nk; ++kt) {                                                  \
                const int u1 = u0 + 1 - (u0 + 1 >= NUNIT ? NUNIT : 0);                         \
                const int u2 = u0 + 2 - (u0 + 2 >= NUNIT ? NUNIT : 0);                         \
                const int u3 = u0 + 3 - (u0 + 3 >= NUNIT ? NUNIT : 0);                         \
                const int u4 = u0 + 4 - (u0 + 4 >= NUNIT ? NUNIT : 0);                         \
                const uint16_t *cA = UNIT(u0), *cB = UNIT(u1);                                 \
                uint16_t *fA = UNIT(u4), *fB = UNIT(u0);                                       \
                STEP16(a0, b0, a1, b1, cA, cB, 4 + q, DMA16_S0, NB_);                          \
                __atomic_signal_fence(__ATOMIC_SEQ_CST);                                       \
                wait_vmcnt_lds<8>();                                                           \
                __builtin_amdgcn_s_barrier();                                                  \
                __atomic_signal_fence(__ATOMIC_SEQ_CST);                                       \
                const uint16_t *nA = UNIT(u2), *nB = UNIT(u3);                                 \
                STEP16(a1, b1, a0, b0, nA, nB, q, DMA16_S1, NB_);                              \
                u0 = u2;                                                                       \
            }                                                                                  \
        }
        switch (live <= 0 ? 0 : live >= 128 ? 4 : (live + 31) / 32) {
            case 4: KLOOP16(4) break;
            case 3: KLOOP16(3) break;
            case 2: KLOOP16(2) break;
            case 1: KLOOP16(1) break;
            default: KLOOP16(0) break;
        }
#undef KLOOP16
        // the MFMAs are assembly the compiler does not track: give the last
        // one its result latency before any accumulator read
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#undef DMA16_S0
#undef DMA16_S1
#undef STEP16
#undef FRAG16
#undef B_ROW16
        __syncthreads();  // every wave done with the ring (and its loads landed)
        first = false;
        const int cm0 = m0, cm_end = m_end, cn0 = n0;
        // the next tile's first two stages land while the epilogue runs
        if (t + P < total) {
            TILE_SETUP(t + P);
            PROLOGUE_LOADS();
        }
        // Register epilogue: lane owns tile rows wm*128 + 16i + lane % 16 and,
        // per 16-column block, the 4 columns 4 (lane / 16) .. +3.  Two blocks'
        // values, swapped between the 16-lane rows of the wave (lanes
        // 16-31 <-> 0-15 and 48-63 <-> 32-47), leave each lane 8 consecutive
        // columns of one block: block 2jp + (lane / 16) % 2, columns
        // 8 (lane / 32) .. +7, one 16-byte store.  Padding rows' stores get an
        // offset past the end of the output, which the hardware drops, so
        // every lane issues every store (the wait count above relies on it).
        const __amdgpu_buffer_rsrc_t rOut = buf_rsrc(p.out, (uint32_t)p.M * (uint32_t)p.N * 2u);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int row = cm0 + wm * 128 + 16 * i + l16;
            const uint32_t obase =
                row < cm_end ? ((uint32_t)row * (uint32_t)p.N + (uint32_t)cn0) * 2u : 0xfffff000u;
            const bool blk = cm_end - cm0 - wm * 128 > 16 * i;  // block has rows (uniform)
#pragma unroll
            for (int jp = 0; jp < (DUAL ? 2 : 4); ++jp) {
                __builtin_amdgcn_sched_barrier(0);
                uint32_t w[2][2];  // [block 2jp + h][dword]: 4 bf16 values
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int j = 2 * jp + h;
                    if constexpr (DUAL) {
                        w[h][0] = w[h][1] = 0;
                        if (blk) {  // an empty block's stores are dropped: skip its math
                            float v[4];
#pragma unroll
                            for (int u = 0; u < 4; ++u) v[u] = swiglu(acc_read(acc[i][j][u]), acc_read(acc[i][j + 4][u]));
                            w[h][0] = pack_bf16x2(v[0], v[1]);
                            w[h][1] = pack_bf16x2(v[2], v[3]);
                        }
                    } else {
                        w[h][0] = pack_bf16x2(acc_read(acc[i][j][0]), acc_read(acc[i][j][1]));
                        w[h][1] = pack_bf16x2(acc_read(acc[i][j][2]), acc_read(acc[i][j][3]));
                    }
                }
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    const auto sw = __builtin_amdgcn_permlane16_swap(w[0][k], w[1][k], false, false);
                    w[0][k] = sw[0];
                    w[1][k] = sw[1];
                }
                const int col = (DUAL ? wn * 64 : wn * 128) + 16 * (2 * jp + (q & 1)) + 8 * (q >> 1);
                __builtin_amdgcn_raw_buffer_store_b128(i32x4{(int)w[0][0], (int)w[0][1], (int)w[1][0], (int)w[1][1]},
                                                      rOut, obase + (uint32_t)col * 2u, 0, 0);
            }
        }
    }
#undef TILE_SETUP
#undef PROLOGUE_LOADS
#undef B_RSRC
#undef ISSUE_A
#undef ISSUE_B
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

bool ffn_bf16_large_ok(const FfnArgs &a) {
    const int groups = a.offsets ? a.E : 1;
    // DMA offsets are 32-bit bytes from each operand's base (A rows, h rows,
    // one expert's weights); every operand ends below the out-of-range
    // offset kOobOff (plus a stage offset) used for padding rows
    const unsigned long long lim = kOobOff - (1ULL << 20);
    const bool fits = (unsigned long long)a.M * a.d * 2 < lim && (unsigned long long)a.M * a.I * 2 < lim &&
                      (unsigned long long)a.I * a.d * 2 < lim;
    return fits && (long long)a.M >= 128LL * groups && a.I % 128 == 0 && a.d % 256 == 0 && a.d % LK == 0 &&
           a.I % LK == 0 && a.d < (1 << 19) && a.I < (1 << 19);
}

bool bf16_large_gemm_ok(const LargeGemmArgs &g) {
    if (g.b_kn) {
        const int groups = g.offsets ? kE : 1;
        const unsigned long long lim = kOobOff - (1ULL << 20);
        const unsigned long long a_rows = g.a_rows ? (unsigned long long)g.a_src_rows : (unsigned long long)g.M;
        const int kb = g.ksplit ? g.ksplit : g.K;
        return !g.dual && !g.kseg && (long long)g.M >= 128LL * groups && g.N % LB == 0 && g.K % LK == 0 &&
               kb % LK == 0 && g.ksplit < g.K && (g.ksplit == 0 || g.K == 2 * g.ksplit) && g.K < (1 << 19) &&
               a_rows * g.K * 2 < lim && (unsigned long long)g.N * kb * 2 < lim &&
               (unsigned long long)g.M * g.ldo * 4 < lim;
    }
    if (g.kseg) {
        const unsigned long long lim = kOobOff - (1ULL << 20);
        return !g.dual && !g.offsets && !g.a_rows && g.M % LM == 0 && g.N % LB == 0 && g.ldk % 8 == 0 &&
               (unsigned long long)g.M * g.ldk * 2 < lim && (unsigned long long)g.N * g.ldk * 2 < lim &&
               (unsigned long long)g.M * g.ldo * 4 < lim && (unsigned long long)LB * 4 < 65536;
    }
    const int groups = g.offsets ? kE : 1;
    const unsigned long long lim = kOobOff - (1ULL << 20);
    const unsigned long long a_rows = g.a_rows ? (unsigned long long)g.a_src_rows : (unsigned long long)g.M;
    const int bn = g.dual ? LB / 2 : LB;
    return (long long)g.M >= 128LL * groups && g.N % bn == 0 && g.K % LK == 0 && g.K < (1 << 19) &&
           a_rows * g.K * 2 < lim && (unsigned long long)g.N * g.K * 2 < lim &&
           (unsigned long long)g.M * g.ldo * 4 < lim && (unsigned long long)(g.up_off + LB) * 4 < 65536;
}

hipError_t launch_bf16_large_gemm(const LargeGemmArgs &g, hipStream_t s) {
    const int P = (cu_count() / 8) * 8;
    LargeParams p{};
    p.M = g.M;
    p.offsets = g.offsets;
    p.A = g.A;
    p.a_rows = g.a_rows;
    p.a_div = g.a_div;
    p.K = g.K;
    p.B0 = g.B0;
    p.B1 = g.B1;
    p.N = g.N;
    p.outf = g.out;
    p.ldo = g.ldo;
    p.up_off = g.up_off;
    p.kseg = g.kseg;
    p.ldk = g.ldk;
    p.cstride = g.cstride;
    p.ksplit = g.ksplit;
    if (g.b_kn) {
        if (g.offsets) hipLaunchKernelGGL((k_gemm_bf16_large<EPI_F32, true, false, true>), dim3(P), dim3(256), 0, s, p);
        else hipLaunchKernelGGL((k_gemm_bf16_large<EPI_F32, false, false, true>), dim3(P), dim3(256), 0, s, p);
    } else if (g.kseg) {
        hipLaunchKernelGGL((k_gemm_bf16_large<EPI_F32, false, true>), dim3(P), dim3(256), 0, s, p);
    } else if (g.dual) {
        if (g.offsets) hipLaunchKernelGGL((k_gemm_bf16_large<EPI_PRE, true>), dim3(P), dim3(256), 0, s, p);
        else hipLaunchKernelGGL((k_gemm_bf16_large<EPI_PRE, false>), dim3(P), dim3(256), 0, s, p);
    } else {
        if (g.offsets) hipLaunchKernelGGL((k_gemm_bf16_large<EPI_F32, true>), dim3(P), dim3(256), 0, s, p);
        else hipLaunchKernelGGL((k_gemm_bf16_large<EPI_F32, false>), dim3(P), dim3(256), 0, s, p);
    }
    return hipGetLastError();
}

hipError_t launch_ffn_bf16_large(const FfnArgs &a, hipStream_t s) {
    const int P = (cu_count() / 8) * 8;
    const bool routed = a.offsets != nullptr;
    if (a.phases & 1) {
        LargeParams p{};
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
        if (routed)
            hipLaunchKernelGGL((k_gemm_bf16_mi16<EPI_SWIGLU, true>), dim3(P), dim3(256), 0, s, p);
        else
            hipLaunchKernelGGL((k_gemm_bf16_mi16<EPI_SWIGLU, false>), dim3(P), dim3(256), 0, s, p);
    }
    if (a.phases & 2) {
        LargeParams q{};
        q.M = a.M;
        q.offsets = a.offsets;
        q.A = static_cast<const uint16_t *>(a.h);
        q.K = a.I;
        q.B0 = static_cast<const uint16_t *>(a.w.down);
        q.N = a.d;
        if (a.combine) {
            q.yout = static_cast<float *>(a.y);
            q.y_perm = static_cast<const uint16_t *>(a.y_perm);
            q.row_of = a.row_of;
            q.cw = a.cw;
            q.k = a.k;
            hipLaunchKernelGGL((k_gemm_bf16_large<EPI_COMBINE, false>), dim3(P), dim3(256), 0, s, q);
        } else {
            q.out = static_cast<uint16_t *>(a.y);
            if (routed)
                hipLaunchKernelGGL((k_gemm_bf16_mi16<EPI_STORE, true>), dim3(P), dim3(256), 0, s, q);
            else
                hipLaunchKernelGGL((k_gemm_bf16_mi16<EPI_STORE, false>), dim3(P), dim3(256), 0, s, q);
        }
    }
    return hipGetLastError();
}

}  // namespace moe
