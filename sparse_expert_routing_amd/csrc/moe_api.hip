// C ABI of the MoE layer (declared in include/moe.h): host-side validation,
// workspace sizing and kernel launches.  Nothing here allocates, frees,
// synchronises or reads device memory.
#include "moe.h"

#include <hip/hip_runtime.h>

#include "kernels.h"

namespace {

using moe::kBF16;
using moe::kE4M3;
using moe::kF32;

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

size_t elem_bytes(int dt) { return dt == kF32 ? 4 : dt == kBF16 ? 2 : 1; }

// Shape validation shared by every call.
moe_status_t check_desc(const moe_desc_t *d) {
    if (d == nullptr) return MOE_EINVAL;
    if (d->T <= 0 || d->d <= 0 || d->E <= 0 || d->k <= 0 || d->I <= 0) return MOE_EINVAL;
    if (d->k > d->E) return MOE_EINVAL;
    const bool pair_ok = (d->act == MOE_F32 && d->wt == MOE_F32) || (d->act == MOE_BF16 && d->wt == MOE_BF16) ||
                         (d->act == MOE_BF16 && d->wt == MOE_E4M3);
    if (d->act < 0 || d->act > 2 || d->wt < 0 || d->wt > 2) return MOE_EINVAL;
    if (d->wt == MOE_E4M3 && (d->d % 128 != 0 || d->I % 128 != 0)) return MOE_EINVAL;
    if (!pair_ok) return MOE_ENOTSUP;
    if (d->E != 256 || d->k != 8) return MOE_ENOTSUP;
    if (d->d % 64 != 0 || d->I % 64 != 0) return MOE_ENOTSUP;
    if (d->wt == MOE_BF16 && d->d % 128 != 0) return MOE_ENOTSUP;
    // 32-bit row indices and element offsets within one row block
    if ((long long)d->T * d->k >= (1LL << 31)) return MOE_ENOTSUP;
    return MOE_OK;
}

struct FfnWs {
    size_t h, h_scale, total;
};
FfnWs ffn_ws(int rows, const moe_desc_t *d) {
    FfnWs w{};
    w.h = align_up((size_t)rows * d->I * elem_bytes(d->wt));
    w.h_scale = d->wt == MOE_E4M3 ? align_up((size_t)rows * (d->I / 128)) : 0;  // E8M0 bytes
    w.total = w.h + w.h_scale;
    return w;
}

// The routed FFN stage: h (+ its scales) for T*k rows, and for e4m3 room for
// x quantised once per token (moe_expert_gate_up_rows).
size_t xq_bytes(const moe_desc_t *d) {
    return d->wt == MOE_E4M3 ? align_up((size_t)d->T * d->d) + align_up((size_t)d->T * (d->d / 128)) : 0;
}
// e4m3 gathered rows: their tile scales per 128-block in GEMM row order.
size_t xs_km_bytes(const moe_desc_t *d) {
    return d->wt == MOE_E4M3 ? align_up((size_t)d->T * d->k * (d->d / 128)) : 0;
}
size_t routed_ffn_ws(const moe_desc_t *d) { return ffn_ws(d->T * d->k, d).total + xq_bytes(d) + xs_km_bytes(d); }

size_t dispatch_ws(const moe_desc_t *d) {
    const size_t nblk = (d->T + moe::kDispatchBlock - 1) / moe::kDispatchBlock;
    return align_up(nblk * d->E * sizeof(int32_t));
}

size_t route_ws(const moe_desc_t *d) {
    return d->act == MOE_BF16 && moe::route_bf16_ok(d->d) ? align_up(moe::route_bf16_ws_bytes(d->T, d->d)) : 0;
}

// The shared expert + combine: h (+ scales), x quantised (e4m3), and fp32
// split-K partials at small T (bf16).
size_t backward_ws(const moe_desc_t *d) {
    if (d->act != MOE_BF16 || !moe::backward_ok(d->d, d->I)) return 0;
    if (d->wt == MOE_BF16) return align_up(moe::backward_ws_bytes(d->T, d->d, d->I, d->k));
    if (d->wt == MOE_E4M3) return align_up(moe::backward_fp8_ws_bytes(d->T, d->d, d->I, d->k));
    return 0;
}

size_t combine_ws(const moe_desc_t *d) {
    const size_t xs_km = d->wt == MOE_E4M3 ? align_up((size_t)d->T * (d->d / 128)) : 0;
    return ffn_ws(d->T, d).total + xq_bytes(d) + xs_km +
           align_up(moe::ffn_shared_split_bytes(d->T, d->d, d->I, d->wt));
}

moe_status_t hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_EHIP; }

bool ffn_weights_ok(const moe_ffn_weights_t *w, int wt) {
    if (w == nullptr || w->gate == nullptr || w->up == nullptr || w->down == nullptr) return false;
    if (wt == MOE_E4M3 && (w->s_gate == nullptr || w->s_up == nullptr || w->s_down == nullptr)) return false;
    return true;
}

moe::FfnWeights to_internal(const moe_ffn_weights_t *w) {
    return moe::FfnWeights{w->gate, w->up, w->down, w->s_gate, w->s_up, w->s_down};
}

}  // namespace

extern "C" {

const char *moe_status_str(moe_status_t s) {
    switch (s) {
        case MOE_OK: return "MOE_OK";
        case MOE_EINVAL: return "MOE_EINVAL: invalid argument";
        case MOE_ENOTSUP: return "MOE_ENOTSUP: shape or dtype not supported by the library";
        case MOE_EWORKSPACE: return "MOE_EWORKSPACE: workspace smaller than moe_workspace_bytes()";
        case MOE_EHIP: return "MOE_EHIP: HIP launch error";
        case MOE_ESCRATCH: return "MOE_ESCRATCH: request larger than the library's static scratch";
    }
    return "unknown moe_status_t";
}

size_t moe_workspace_bytes(const moe_desc_t *d, int32_t stage) {
    if (check_desc(d) != MOE_OK) return 0;
    switch (stage) {
        case MOE_WS_ROUTE: return route_ws(d);
        case MOE_WS_DISPATCH: return dispatch_ws(d);
        case MOE_WS_FFN: return routed_ffn_ws(d);
        case MOE_WS_COMBINE: return combine_ws(d);
        case MOE_WS_BACKWARD: return backward_ws(d);
    }
    return 0;
}

moe_status_t moe_route(const moe_desc_t *d, const void *x, const float *w_router, const float *bias,
                       int32_t *idx, float *weights, float *gap, void *workspace, size_t ws_bytes,
                       void *stream) {
    moe_status_t st = check_desc(d);
    if (st != MOE_OK) return st;
    if (!x || !w_router || !bias || !idx || !weights) return MOE_EINVAL;
    const size_t need = route_ws(d);
    if (need && (!workspace || ws_bytes < need)) return MOE_EWORKSPACE;
    moe::RouteArgs a{d->T, d->d, d->act == MOE_BF16, x, w_router, bias, idx, weights, gap};
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (need) return hip_status(moe::launch_route_bf16(a, workspace, s));
    return hip_status(moe::launch_route(a, s));
}

moe_status_t moe_dispatch(const moe_desc_t *d, const int32_t *idx, const void *x, int32_t *counts,
                          int32_t *offsets, int32_t *row_src, int32_t *row_of, void *x_perm,
                          uint8_t *x_perm_scale, void *workspace, size_t ws_bytes, void *stream) {
    moe_status_t st = check_desc(d);
    if (st != MOE_OK) return st;
    if (!idx || !counts || !offsets || !row_src || !row_of) return MOE_EINVAL;
    if (x_perm && (!x || (d->wt == MOE_E4M3 && !x_perm_scale))) return MOE_EINVAL;
    if (!workspace || ws_bytes < dispatch_ws(d)) return MOE_EWORKSPACE;
    moe::DispatchArgs a{d->T, d->d, d->E, d->k, d->act, d->wt, idx, x, counts, offsets, row_src, row_of,
                        x_perm, x_perm_scale, static_cast<int32_t *>(workspace)};
    return hip_status(moe::launch_dispatch(a, static_cast<hipStream_t>(stream)));
}

moe_status_t moe_dispatch_noalloc(const moe_desc_t *d, const int32_t *idx, const void *x, int32_t *counts,
                                  int32_t *offsets, int32_t *row_src, int32_t *row_of, void *x_perm,
                                  uint8_t *x_perm_scale, void *stream) {
    moe_status_t st = check_desc(d);
    if (st != MOE_OK) return st;
    if (!idx || !counts || !offsets || !row_src || !row_of) return MOE_EINVAL;
    if (x_perm && (!x || (d->wt == MOE_E4M3 && !x_perm_scale))) return MOE_EINVAL;
    if (d->T > moe::kDispatchScratchTokens) return MOE_ESCRATCH;
    moe::DispatchArgs a{d->T, d->d, d->E, d->k, d->act, d->wt, idx, x, counts, offsets, row_src, row_of,
                        x_perm, x_perm_scale, nullptr};
    return hip_status(moe::launch_dispatch_noalloc(a, static_cast<hipStream_t>(stream)));
}

// a_rows == nullptr: A = x_perm (+ x_perm_scale), one row per routed row.
// a_rows != nullptr: A row r is row a_rows[r] / k of x (T rows; quantised into the
// workspace first for e4m3).
static moe_status_t expert_ffn_phases(const moe_desc_t *d, const void *x_perm, const uint8_t *x_perm_scale,
                                      const int32_t *a_rows, const int32_t *offsets,
                                      const moe_ffn_weights_t *experts, void *y_perm, void *workspace,
                                      size_t ws_bytes, void *stream, int phases) {
    moe_status_t st = check_desc(d);
    if (st != MOE_OK) return st;
    if (!offsets || !ffn_weights_ok(experts, d->wt)) return MOE_EINVAL;
    if ((phases & 1) && (!x_perm || (d->wt == MOE_E4M3 && !a_rows && !x_perm_scale))) return MOE_EINVAL;
    if ((phases & 2) && !y_perm) return MOE_EINVAL;
    const FfnWs w = ffn_ws(d->T * d->k, d);
    if (!workspace || ws_bytes < routed_ffn_ws(d)) return MOE_EWORKSPACE;
    char *ws = static_cast<char *>(workspace);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (a_rows && d->wt == MOE_E4M3 && (phases & 1)) {
        char *xq = ws + w.total;
        uint8_t *xs = reinterpret_cast<uint8_t *>(xq + align_up((size_t)d->T * d->d));
        hipError_t e = moe::launch_quant_rows_e4m3(d->T, d->d, static_cast<const uint16_t *>(x_perm),
                                                   reinterpret_cast<uint8_t *>(xq), xs, s);
        if (e != hipSuccess) return MOE_EHIP;
        x_perm = xq;
        x_perm_scale = xs;
    }
    moe::FfnArgs a{};
    a.M = d->T * d->k;
    a.d = d->d;
    a.I = d->I;
    a.E = d->E;
    a.wt = d->wt;
    a.offsets = offsets;
    a.a = x_perm;
    a.a_scale = x_perm_scale;
    a.a_rows = a_rows;
    a.a_div = d->k;
    a.w = to_internal(experts);
    a.h = ws;
    a.h_scale = w.h_scale ? reinterpret_cast<uint8_t *>(ws + w.h) : nullptr;
    a.y = y_perm;
    a.phases = phases;
    a.combine = false;
    if (a_rows && d->wt == MOE_E4M3 && (phases & 1) && moe::ffn_fp8_mx_ok(a)) {
        // the persistent e4m3 kernel reads each stage's A-row scales of a
        // tile as one contiguous run: lay the gathered rows' scales out per
        // 128-block in GEMM row order (instead of one scattered byte per row)
        uint8_t *xs_km = reinterpret_cast<uint8_t *>(ws + w.total + xq_bytes(d));
        hipError_t e = moe::launch_gather_scales_kmajor(a.M, d->d / 128, d->k, a_rows, x_perm_scale, xs_km, s);
        if (e != hipSuccess) return MOE_EHIP;
        a.a_scale = xs_km;
        a.a_scale_kmajor = true;
    }
    a.k = d->k;
    return hip_status(moe::launch_ffn(a, s));
}

moe_status_t moe_expert_ffn(const moe_desc_t *d, const void *x_perm, const uint8_t *x_perm_scale,
                            const int32_t *offsets, const moe_ffn_weights_t *experts, void *y_perm,
                            void *workspace, size_t ws_bytes, void *stream) {
    return expert_ffn_phases(d, x_perm, x_perm_scale, nullptr, offsets, experts, y_perm, workspace, ws_bytes,
                             stream, 3);
}

moe_status_t moe_expert_gate_up(const moe_desc_t *d, const void *x_perm, const uint8_t *x_perm_scale,
                                const int32_t *offsets, const moe_ffn_weights_t *experts, void *workspace,
                                size_t ws_bytes, void *stream) {
    return expert_ffn_phases(d, x_perm, x_perm_scale, nullptr, offsets, experts, nullptr, workspace, ws_bytes,
                             stream, 1);
}

moe_status_t moe_expert_gate_up_rows(const moe_desc_t *d, const void *x, const int32_t *row_src,
                                     const int32_t *offsets, const moe_ffn_weights_t *experts, void *workspace,
                                     size_t ws_bytes, void *stream) {
    if (!row_src) return MOE_EINVAL;
    return expert_ffn_phases(d, x, nullptr, row_src, offsets, experts, nullptr, workspace, ws_bytes, stream, 1);
}

moe_status_t moe_expert_down(const moe_desc_t *d, const int32_t *offsets, const moe_ffn_weights_t *experts,
                             void *y_perm, void *workspace, size_t ws_bytes, void *stream) {
    return expert_ffn_phases(d, nullptr, nullptr, nullptr, offsets, experts, y_perm, workspace, ws_bytes, stream,
                             2);
}

moe_status_t moe_combine(const moe_desc_t *d, const void *x, const moe_ffn_weights_t *shared,
                         const void *y_perm, const int32_t *row_of, const float *weights, float *y,
                         void *workspace, size_t ws_bytes, void *stream) {
    moe_status_t st = check_desc(d);
    if (st != MOE_OK) return st;
    if (!x || !y_perm || !row_of || !weights || !y || !ffn_weights_ok(shared, d->wt)) return MOE_EINVAL;
    if (!workspace || ws_bytes < combine_ws(d)) return MOE_EWORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    char *ws = static_cast<char *>(workspace);
    const FfnWs w = ffn_ws(d->T, d);
    moe::FfnArgs a{};
    a.M = d->T;
    a.d = d->d;
    a.I = d->I;
    a.E = 1;
    a.wt = d->wt;
    a.offsets = nullptr;
    a.a = x;
    a.a_scale = nullptr;
    if (d->wt == MOE_E4M3) {
        char *xq = ws + w.total;
        uint8_t *xs = reinterpret_cast<uint8_t *>(xq + align_up((size_t)d->T * d->d));
        hipError_t e = moe::launch_quant_rows_e4m3(d->T, d->d, static_cast<const uint16_t *>(x),
                                                   reinterpret_cast<uint8_t *>(xq), xs, s);
        if (e != hipSuccess) return MOE_EHIP;
        a.a = xq;
        a.a_scale = xs;
    }
    a.w = to_internal(shared);
    a.h = ws;
    a.h_scale = w.h_scale ? reinterpret_cast<uint8_t *>(ws + w.h) : nullptr;
    a.y = y;
    a.phases = 3;
    a.combine = true;
    a.k = d->k;
    a.y_perm = y_perm;
    a.row_of = row_of;
    a.cw = weights;
    if (d->wt == MOE_E4M3 && moe::ffn_fp8_mx_ok(a)) {
        // the persistent e4m3 kernel reads each stage's A-row scales of a
        // tile as one contiguous run: lay them out per 128-block
        uint8_t *xs_km = reinterpret_cast<uint8_t *>(ws + w.total + xq_bytes(d));
        hipError_t e = moe::launch_gather_scales_kmajor(d->T, d->d / 128, 1, nullptr, a.a_scale, xs_km, s);
        if (e != hipSuccess) return MOE_EHIP;
        a.a_scale = xs_km;
        a.a_scale_kmajor = true;
    }
    if (moe::ffn_shared_split_bytes(d->T, d->d, d->I, d->wt))
        a.part = reinterpret_cast<float *>(
            ws + w.total + xq_bytes(d) + (d->wt == MOE_E4M3 ? align_up((size_t)d->T * (d->d / 128)) : 0));
    return hip_status(moe::launch_ffn(a, s));
}

moe_status_t moe_bias_update(const moe_desc_t *d, const int32_t *counts, float gamma, float *bias,
                             void *stream) {
    moe_status_t st = check_desc(d);
    if (st != MOE_OK) return st;
    if (!counts || !bias) return MOE_EINVAL;
    return hip_status(moe::launch_bias_update(d->E, d->k, d->T, counts, gamma, bias,
                                              static_cast<hipStream_t>(stream)));
}

moe_status_t moe_backward(const moe_desc_t *d, const void *x, const float *w_router, const int32_t *idx,
                          const float *weights, const int32_t *offsets, const int32_t *row_src,
                          const int32_t *row_of, const moe_ffn_weights_t *experts,
                          const moe_ffn_weights_t *shared, const void *y_perm, const float *dy, float *dx,
                          float *dw_router, float *dw_gate, float *dw_up, float *dw_down, float *ds_gate,
                          float *ds_up, float *ds_down, float *dg, void *workspace, size_t ws_bytes,
                          void *stream) {
    moe_status_t st = check_desc(d);
    if (st != MOE_OK) return st;
    if (d->act != MOE_BF16 || (d->wt != MOE_BF16 && d->wt != MOE_E4M3) || !moe::backward_ok(d->d, d->I))
        return MOE_ENOTSUP;
    if (!x || !w_router || !idx || !weights || !offsets || !row_src || !row_of || !y_perm || !dy || !dx ||
        !dw_router || !dw_gate || !dw_up || !dw_down || !ds_gate || !ds_up || !ds_down ||
        !ffn_weights_ok(experts, d->wt) || !ffn_weights_ok(shared, d->wt))
        return MOE_EINVAL;
    if (!workspace || ws_bytes < backward_ws(d)) return MOE_EWORKSPACE;
    moe::BackwardArgs a{};
    a.T = d->T;
    a.d = d->d;
    a.I = d->I;
    a.k = d->k;
    a.x = x;
    a.w_router = w_router;
    a.idx = idx;
    a.weights = weights;
    a.offsets = offsets;
    a.row_src = row_src;
    a.row_of = row_of;
    a.experts = to_internal(experts);
    a.shared = to_internal(shared);
    a.y_perm = y_perm;
    a.dy = dy;
    a.dx = dx;
    a.dw_router = dw_router;
    a.dw_gate = dw_gate;
    a.dw_up = dw_up;
    a.dw_down = dw_down;
    a.ds_gate = ds_gate;
    a.ds_up = ds_up;
    a.ds_down = ds_down;
    a.dg = dg;
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    return hip_status(d->wt == MOE_E4M3 ? moe::launch_backward_fp8(a, workspace, hs)
                                        : moe::launch_backward(a, workspace, hs));
}

}  // extern "C"
