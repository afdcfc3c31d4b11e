// Internal launch interface between the C ABI (moe_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

enum Dtype { kF32 = 0, kBF16 = 1, kE4M3 = 2 };

struct RouteArgs {
    int T, d;
    bool x_bf16;
    const void *x;
    const float *wr, *bias;
    int32_t *idx;
    float *w, *gap;
};
hipError_t launch_route(const RouteArgs &a, hipStream_t s);
// bf16 activations: split router + bf16 MFMA logits + top-k (workspace:
// route_bf16_ws_bytes).
bool route_bf16_ok(int d);
size_t route_bf16_ws_bytes(int T, int d);
hipError_t launch_route_bf16(const RouteArgs &a, void *ws, hipStream_t s);

constexpr int kDispatchBlock = 256;  // tokens per dispatch workgroup

struct DispatchArgs {
    int T, d, E, k;
    int act, wt;
    const int32_t *idx;
    const void *x;
    int32_t *counts, *offsets, *row_src, *row_of;
    void *x_perm;         // null: no gather (counts, offsets, row_src, row_of only)
    uint8_t *x_perm_scale;  // e4m3: [T*k, d/128] E8M0
    int32_t *block_base;  // workspace [ceil(T/256), E]
};
hipError_t launch_dispatch(const DispatchArgs &a, hipStream_t s);
// The same dispatch with the block counts in the library's static device
// scratch instead of a caller workspace (a.block_base is ignored): at most
// kDispatchScratchTokens tokens (checked by the caller); the scratch
// address is looked up once per device (its HIP error is returned).
constexpr int kDispatchScratchTokens = 1 << 20;
hipError_t launch_dispatch_noalloc(DispatchArgs a, hipStream_t s);

// Quantise T rows of bf16 x to e4m3 per 1x128 tile (no permutation); E8M0 scales.
hipError_t launch_quant_rows_e4m3(int rows, int d, const uint16_t *x, uint8_t *q, uint8_t *scales,
                                  hipStream_t s);
// out[kb * M + r] = scales[(rows[r] / div) * nkb + kb] (rows == nullptr: row r):
// the per-row E8M0 tile scales of (gathered) rows laid out per 128-block in
// GEMM row order.
hipError_t launch_gather_scales_kmajor(int M, int nkb, int div, const int32_t *rows, const uint8_t *scales,
                                       uint8_t *out, hipStream_t s);

// Every e4m3 scale in the library is an E8M0 byte (OCP MX): byte e is 2^(e-127).
struct FfnWeights {
    const void *gate, *up, *down;
    const uint8_t *s_gate, *s_up, *s_down;
};

// Grouped SwiGLU FFN over permuted rows (routed: offsets != nullptr, E groups)
// or over plain rows (shared: offsets == nullptr, one group of M rows).
struct FfnArgs {
    int M;            // rows (T*k routed, T shared)
    int d, I, E;      // E groups when offsets != nullptr
    int wt;           // kF32, kBF16, kE4M3
    const int32_t *offsets;
    const void *a;    // [M, d] rows in wt type (or [*, d] rows picked by a_rows)
    const uint8_t *a_scale;  // e4m3: [M, d/128] E8M0 (row-aligned with a)
    const int32_t *a_rows;  // optional: A row r of the GEMM is row a_rows[r] / a_div of a / a_scale
    // e4m3, persistent kernel only: a_scale is instead [d/128, M], each
    // 128-block's scales in GEMM row order (no gather through a_rows)
    bool a_scale_kmajor;
    int a_div;
    FfnWeights w;
    void *h;          // workspace [M, I] in wt type
    uint8_t *h_scale;  // e4m3: [M, I/128] E8M0 ([I/128, M] on the persistent e4m3 kernel)
    // output: either y_perm (routed) or the combine (shared)
    void *y;          // routed: [M, d] f32 / bf16; shared: [M, d] f32
    // which GEMMs to run: 1 = gate/up only, 2 = down only, 3 = both
    int phases;
    // combine epilogue (shared only)
    bool combine;
    int k;
    const void *y_perm;
    const int32_t *row_of;
    const float *cw;
    // shared expert at small T: fp32 workspace for split-K partial sums
    // (ffn_shared_split_bytes; nullptr = no split)
    float *part;
};
hipError_t launch_ffn(const FfnArgs &a, hipStream_t s);
size_t ffn_shared_split_bytes(int M, int d, int I, int wt);
// y[t] += sum_{j<k} cw[t*k+j] * y_perm[row_of[t*k+j]] (bf16 rows, fp32, ascending j).
hipError_t launch_combine_add(int T, int d, int k, const uint16_t *y_perm, const int32_t *row_of, const float *cw,
                              float *y, hipStream_t s);
hipError_t launch_ffn_fp8(const FfnArgs &a, hipStream_t s);
// Tiny-group bf16 path (decode: routed groups averaging at most 4 rows):
// weights streamed from HBM into registers, K split over the 4 waves.
bool ffn_skinny_ok(const FfnArgs &a);
hipError_t launch_ffn_skinny(const FfnArgs &a, hipStream_t s);
// Large-group bf16 path (persistent 256x256 tiles): usable when every group
// averages at least 128 rows and the widths tile evenly.
bool ffn_bf16_large_ok(const FfnArgs &a);
hipError_t launch_ffn_bf16_large(const FfnArgs &a, hipStream_t s);
// The same persistent 256x256-tile kernel as a grouped NT GEMM with an fp32
// output (the layer backward), grouped over M or (kseg) over K: out[m, n] = sum_k A[m, k] B_g[n, k] with B
// per group (offsets != nullptr) or one B; dual: B0 / B1 are the gate / up
// matrices of a SwiGLU tile and their products go to columns n and
// up_off + n.  a_rows: A row m is row a_rows[m] / a_div (a_src_rows rows).
struct LargeGemmArgs {
    int M;
    const int32_t *offsets;
    const uint16_t *A;
    const int32_t *a_rows;
    int a_div;
    int a_src_rows;
    int K;
    const uint16_t *B0, *B1;
    int N;
    float *out;
    int ldo, up_off;
    bool dual;
    // K-grouped form (weight gradients): out_e = A[:, K_e] B[:, K_e]^T with
    // K_e = [kseg[e], kseg[e+1]) (multiples of 64) of A [M, ldk], B [N, ldk],
    // written to out + e * cstride; groups with empty K_e are not written
    const int32_t *kseg = nullptr;
    int ldk = 0;
    int64_t cstride = 0;
    // B stored K-major, [G, K, N] (N contiguous), instead of [G, N, K]; with
    // ksplit, K rows [0, ksplit) come from B0 [G, ksplit, N] and the rest
    // from B1 (K = 2 ksplit).  Plain fp32 products only (not dual, not
    // K-grouped).
    bool b_kn = false;
    int ksplit = 0;
};
bool bf16_large_gemm_ok(const LargeGemmArgs &g);
hipError_t launch_bf16_large_gemm(const LargeGemmArgs &g, hipStream_t s);

// An e4m3 NT product on the persistent e4m3 kernel with an fp32 output:
// out[m*ldo + n] = sum_kb s_a(m, kb) s_b(n/128, kb) sum_k A(m,k) B(n,k), A rows
// per 1x128 tile (As [rows, K/128]), B [G, N, K] with 128x128 block scales
// Bs [G, N/128, K/128]; grouped over M by offsets (B per group) or one group.
struct Fp8GemmArgs {
    int M;
    const int32_t *offsets;
    const uint8_t *A;
    const uint8_t *As;
    const int32_t *a_rows;  // optional: row m reads row a_rows[m] / a_div of A / As
    int a_div;
    int a_src_rows;         // rows of A when a_rows is given
    int K;
    const uint8_t *B;
    const uint8_t *Bs;
    int N;
    float *out;
    int ldo;
};
// K-grouped e4m3 product (weight gradients): for each group e with a
// non-empty range [kseg[e], kseg[e+1]) (multiples of 128; kseg [257], or
// nullptr for one group over [0, K)), out + e*cstride [M, ldo] =
// sum_kb As(m, kb) Bs(n, kb) sum_k A(m,k) B(n,k) over that range.  A [M, K],
// B [N, K] codes (K the row stride), As [M, K/128], Bs [N, K/128] E8M0
// scales.  Groups with an empty range are not written.
struct Fp8KgArgs {
    int M, N, K;
    const int32_t *kseg;
    const uint8_t *A;
    const uint8_t *As;
    const uint8_t *B;
    const uint8_t *Bs;
    float *out;
    int ldo;
    int64_t cstride;
};
// The e4m3 large-group path on the bf16 kernel's schedule (persistent 256x256
// tiles, 4 waves, AGPR accumulators), scales applied by the block-scaled
// MFMA (csrc/ffn_fp8_mx.hip).
bool ffn_fp8_mx_ok(const FfnArgs &a);
hipError_t launch_ffn_fp8_mx(const FfnArgs &a, hipStream_t s);
bool fp8_mx_gemm_ok(const Fp8GemmArgs &g);
hipError_t launch_fp8_mx_gemm(const Fp8GemmArgs &g, hipStream_t s);
bool fp8_mx_kg_ok(const Fp8KgArgs &g);
hipError_t launch_fp8_mx_kg(const Fp8KgArgs &g, hipStream_t s);

hipError_t launch_bias_update(int E, int k, int T, const int32_t *counts, float gamma, float *bias,
                              hipStream_t s);

// Backward of the layer (bf16 experts): gradients for the forward's routing.
struct BackwardArgs {
    int T, d, I, k;
    const void *x;            // [T, d] bf16
    const float *w_router;    // [E, d]
    const int32_t *idx;       // [T, k] chosen ids (ascending)
    const float *weights;     // [T, k] combine weights
    const int32_t *offsets, *row_src, *row_of;
    FfnWeights experts, shared;
    const void *y_perm;       // [T*k, d] bf16 routed outputs of the forward
    const float *dy;          // [T, d]
    float *dx, *dw_router, *dw_gate, *dw_up, *dw_down, *ds_gate, *ds_up, *ds_down;
    float *dg;                // [T, k] or nullptr
};
size_t backward_ws_bytes(int T, int d, int I, int k);
bool backward_ok(int d, int I);
hipError_t launch_backward(const BackwardArgs &a, void *ws, hipStream_t s);
// The same with e4m3 expert weights (128x128 block scales): every backward
// GEMM on e4m3 operands (csrc/backward_fp8.hip).
size_t backward_fp8_ws_bytes(int T, int d, int I, int k);
hipError_t launch_backward_fp8(const BackwardArgs &a, void *ws, hipStream_t s);

}  // namespace moe
