// Steps of the layer backward that the bf16 and e4m3 forms share
// (csrc/backward.hip).  All launches are asynchronous on `s`.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {
namespace bwd {

// poff = exclusive scan of the 256 group sizes (off[e+1] - off[e]) each
// rounded up to a multiple of `align` (64 or 128); poff[256] = the total.
hipError_t pad_offsets(const int32_t *off, int32_t *poff, int align, hipStream_t s);

// Per token: dg_j = dy . y_perm[row_of[t*k+j]]; the routed output gradient
// g_j dy into row row_of[t*k+j] of dyp and the shared one (dy) into row t of
// dys, both bf16, or fp32 when f32_out.
hipError_t combine(int T, int d, const float *dy, const uint16_t *y_perm, const int32_t *row_of, const float *g,
                   void *dyp, void *dys, float *dg, bool f32_out, hipStream_t s);

// From the pre-activations P [rows, 2I] (gate | up) and dh [rows, I]: h and
// (da | db) [rows, 2I], bf16, or fp32 when f32_out.
hipError_t swiglu(int64_t rows, int I, const float *P, const float *dh, void *h, void *dab, bool f32_out,
                  hipStream_t s);

// Router backward per token (dl, and dx written with the router's share),
// then the router weight gradient from dl and x (part: dwr_part_bytes(d)).
hipError_t router(int T, int d, const uint16_t *x, const float *wr, const int32_t *idx, const float *dg, float *dl,
                  float *dx, hipStream_t s);
size_t dwr_part_bytes(int d);
hipError_t dwr(int d, const int32_t *offsets, const int32_t *row_src, const float *dl, const uint16_t *x,
               float *part, float *dwr, hipStream_t s);

// Zeroes out + e*per [per floats] for every group e with no rows
// (off[e+1] == off[e]); per a multiple of 4.
hipError_t zero_empty(int64_t per, const int32_t *off, float *out, hipStream_t s);

// dx[t] += dxs[t] + sum_j dxp[row_of[t*k+j]].
hipError_t dx(int T, int d, const float *dxs, const float *dxp, const int32_t *row_of, float *dx, hipStream_t s);

}  // namespace bwd
}  // namespace moe
