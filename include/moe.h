/*
 * moe.h -- C ABI of the MI355X (gfx950) DeepSeekMoE layer forward with
 * auxiliary-loss-free (bias) routing.
 *
 * The layer, as the pages state it:
 *   - DeepSeek V3 From Scratch, "The idea": 256 routed experts plus one shared
 *     expert that every token uses; each token goes to its top 8 routed
 *     experts; a per-expert bias, added to the router affinity, steers which
 *     experts are chosen, while the combine weights come from the unbiased
 *     affinities; the bias is a control loop, not a loss term.
 *   - DeepSeek V3 From Scratch, "Worked example" (routing, concretely) and
 *     "In code" (route, update_bias): sigmoid affinities, top-k of affinity
 *     plus bias, the chosen k unbiased affinities renormalised to sum to 1,
 *     and bias <- bias + step * sign(target - load).
 *   - kbwen.com DeepSeek feed, "A bias term for each expert": the bias moves
 *     once per step, from the load over the whole batch, by the same fixed
 *     amount (0.001) up or down; no token is dropped.
 *   - Scaling Efficiency: A Deep Dive into the DeepSeek-V3 Architecture,
 *     "Implementation: A Modular Look": the output is the shared expert's
 *     output plus, for each routed expert, its output on the tokens that
 *     chose it scaled by their weight.
 *   - crackai.dev DeepSeek-V3 summary, "How It Works": the routed work is
 *     split into a dispatch and a combine around the expert computation; FP8
 *     expert matmuls with a scale per tile and FP32 accumulation.
 * Our readings where the pages are silent: each expert is a bias-free SwiGLU
 * FFN y = W_down (silu(W_gate a) * (W_up a)); equal biased scores go to the
 * lower expert id; the k chosen ids are reported in ascending order.
 *
 * Conventions for every call:
 *   - Tensors are row-major and contiguous, in device memory owned by the
 *     caller.  The library never allocates, frees or synchronises, and never
 *     reads device memory on the host.  Work is enqueued on `stream` (a
 *     hipStream_t; NULL is the default stream) and the call returns.
 *   - Arguments are validated on the host before anything is launched:
 *     MOE_EINVAL for a null required pointer, non-positive sizes, k > E, or
 *     d / I not multiples of 128 with e4m3; MOE_ENOTSUP for shapes the library
 *     does not cover (E != 256, k != 8, d or I not a multiple of 64, d not a
 *     multiple of 128 with bf16 weights, T * k >= 2^31 routed rows (their
 *     indices are int32), an unsupported dtype pair); MOE_EWORKSPACE when
 *     ws_bytes is below
 *     moe_workspace_bytes(); MOE_ESCRATCH when moe_dispatch_noalloc gets
 *     more tokens than its static scratch holds; MOE_EHIP when a launch
 *     reports an error.
 *     Device faults surface at the caller's next synchronisation.
 *   - No C++ exception crosses the ABI; the library never aborts.
 *   - Calls are stateless and re-entrant (moe_dispatch_noalloc aside: its
 *     calls share one static scratch per GPU); calls on different streams
 *     that share output buffers race, as with any kernel launch.
 *
 * Storage types (moe_dtype_t): fp32; bf16 as 16-bit patterns (upper half of
 * binary32); e4m3 as OCP FP8 E4M3FN bytes, each 1x128 activation tile and
 * 128x128 weight block with one scale stored as an OCP MX E8M0 byte: byte e
 * stands for 2^(e-127) (e = 0 .. 254), so a scale is a power of two by
 * construction; 255 is the format's NaN, and every output that a tile or
 * block with that byte feeds comes out NaN.  The block-scaled MFMA of gfx950
 * takes these bytes as they are.  Supported
 * (act, wt) pairs: (F32, F32), (BF16, BF16), (BF16, E4M3).  The router is
 * always fp32.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_EINVAL = 1,
    MOE_ENOTSUP = 2,
    MOE_EWORKSPACE = 3,
    MOE_EHIP = 4,
    MOE_ESCRATCH = 5  /* moe_dispatch_noalloc: more tokens than its static scratch holds */
} moe_status_t;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_E4M3 = 2 } moe_dtype_t;

/* Shape of one layer call.  T tokens, model width d, E routed experts, top-k,
 * expert intermediate width I.  act: storage type of x.  wt: storage type of
 * the expert weights, which is also the type the expert GEMMs read their
 * activations in (x_perm and the intermediate h). */
typedef struct {
    int32_t T, d, E, k, I;
    int32_t act;
    int32_t wt;
} moe_desc_t;

/* Weights of a stack of G SwiGLU experts (G = E routed, or G = 1 shared):
 * gate, up: [G, I, d]; down: [G, d, I] (each row contiguous along the reduced
 * dimension).  For e4m3 the scales hold one E8M0 byte per 128x128 block:
 * s_gate, s_up: [G, I/128, d/128]; s_down: [G, d/128, I/128]; the value of an
 * element is code * 2^(s - 127).  Scales are NULL for fp32 and bf16. */
typedef struct {
    const void *gate, *up, *down;
    const uint8_t *s_gate, *s_up, *s_down;
} moe_ffn_weights_t;

/* Workspace stages for moe_workspace_bytes. */
enum { MOE_WS_DISPATCH = 0, MOE_WS_FFN = 1, MOE_WS_COMBINE = 2, MOE_WS_ROUTE = 3, MOE_WS_BACKWARD = 4 };

/*
 * Router, biased top-k choice and combine weights (DeepSeek V3 From Scratch,
 * "In code": route; "Worked example").
 *   x        [T, d]  act type
 *   w_router [E, d]  fp32; logit of expert e = x_t . w_router[e]
 *   bias     [E]     fp32 balancing bias (read only)
 *   idx      [T, k]  int32 out: the k experts with the largest
 *                    fl32(sigmoid(logit)) + bias, ascending id order; equal
 *                    scores go to the lower id
 *   weights  [T, k]  fp32 out: sigmoid(logit) of each chosen expert divided by
 *                    the sum over the k chosen (bias not included)
 *   gap      [T]     fp32 out or NULL: k-th minus (k+1)-th largest biased
 *                    score, as the kernel computed it
 *   workspace >= moe_workspace_bytes(desc, MOE_WS_ROUTE) bytes of device memory
 *                    (0 for fp32 activations; NULL allowed then)
 * All scores are computed in fp32: the logit is an fp32 accumulation of
 * exact products (bf16 x times the fp32 router split exactly into three bf16
 * terms, or fp32 x times fp32 w).
 */
moe_status_t moe_route(const moe_desc_t *desc, const void *x, const float *w_router,
                       const float *bias, int32_t *idx, float *weights, float *gap,
                       void *workspace, size_t ws_bytes, void *stream);

/*
 * Dispatch: per-expert load, its prefix sum and a stable grouping of the T*k
 * (token, slot) assignments by expert, with the token rows gathered into that
 * order (crackai.dev DeepSeek-V3 summary, "How It Works": dispatch; Scaling
 * Efficiency ..., "Implementation: A Modular Look": each expert sees the
 * tokens that chose it).  Every assignment is kept: no capacity, no drops
 * (kbwen.com DeepSeek feed, "A bias term for each expert").
 *   idx          [T, k]   int32 from moe_route (ids in [0, E), distinct per token; an id
 *                         outside [0, E) is not dispatched: it takes no row, its row_of
 *                         entry is -1 and offsets[E] falls short of T*k by the number
 *                         of such ids; the later calls need a complete dispatch)
 *   x            [T, d]   act type
 *   counts       [E]      int32 out: assignments per expert (the load)
 *   offsets      [E+1]    int32 out: exclusive prefix sum of counts; offsets[E] = T*k
 *   row_src      [T*k]    int32 out: flat assignment id t*k + j of permuted row r;
 *                         within an expert rows are in ascending t*k + j order
 *   row_of       [T*k]    int32 out: the inverse, permuted row of assignment t*k + j
 *   x_perm       [T*k, d] out, in the expert GEMM input type: row r = x[row_src[r] / k];
 *                         for e4m3 the row is quantised per 1x128 tile:
 *   x_perm_scale [T*k, d/128] E8M0 bytes out (e4m3 only, else NULL): scale = the
 *                         smallest power of two at or above amax/448 (the fp32
 *                         quotient; 1 for an all-zero tile), code =
 *                         e4m3_rne_sat(v / scale)
 *   workspace    >= moe_workspace_bytes(desc, MOE_WS_DISPATCH) bytes of device memory
 * x_perm may be NULL: then only counts, offsets, row_src and row_of are
 * written (x and x_perm_scale are not read), for moe_expert_gate_up_rows,
 * which gathers the rows itself.
 * Integer outputs are bit-exact and deterministic (no atomics decide order).
 */
moe_status_t moe_dispatch(const moe_desc_t *desc, const int32_t *idx, const void *x,
                          int32_t *counts, int32_t *offsets, int32_t *row_src, int32_t *row_of,
                          void *x_perm, uint8_t *x_perm_scale, void *workspace, size_t ws_bytes,
                          void *stream);

/*
 * moe_dispatch for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments (minus the workspace) and the same outputs, bit for bit;
 * the per-block count table lives in a static device array of the library
 * instead (4 MiB on each GPU the library runs on, held until the process
 * ends), so T is limited to 1048576 tokens: MOE_ESCRATCH above that, checked
 * before anything is launched.  The array's device address is looked up on
 * the first call on each device (MOE_EHIP if that fails).  No allocation or
 * free happens in any call.  Every call on one GPU uses the same array:
 * calls that overlap in time on one GPU (several streams or host threads)
 * race and must be serialised by the caller.  Each call overwrites every
 * entry it reads, so nothing carries over from an earlier call.
 */
moe_status_t moe_dispatch_noalloc(const moe_desc_t *desc, const int32_t *idx, const void *x,
                                  int32_t *counts, int32_t *offsets, int32_t *row_src, int32_t *row_of,
                                  void *x_perm, uint8_t *x_perm_scale, void *stream);

/*
 * Routed expert FFNs, grouped: rows [offsets[e], offsets[e+1]) of x_perm go
 * through expert e (DeepSeek V3 From Scratch, "The idea": fine-grained routed
 * experts; crackai.dev DeepSeek-V3 summary, "How It Works": FP8 matmuls with
 * per-tile scales and FP32 accumulation).
 *   h = silu(x_perm W_gate[e]^T) * (x_perm W_up[e]^T), fp32 accumulation,
 *       rounded to the wt type (bf16; or e4m3 per 1x128 tile with an E8M0
 *       scale, as in moe_dispatch; or fp32), kept in the workspace;
 *   y_perm = h W_down[e]^T, fp32 accumulation, stored as fp32 (wt = F32) or
 *       bf16 (otherwise).
 *   x_perm, x_perm_scale, offsets: from moe_dispatch; offsets are read on the
 *       device only (no host synchronisation).
 *   experts   E routed experts (see moe_ffn_weights_t)
 *   y_perm    [T*k, d] out
 *   workspace >= moe_workspace_bytes(desc, MOE_WS_FFN) bytes of device memory
 */
moe_status_t moe_expert_ffn(const moe_desc_t *desc, const void *x_perm, const uint8_t *x_perm_scale,
                            const int32_t *offsets, const moe_ffn_weights_t *experts,
                            void *y_perm, void *workspace, size_t ws_bytes, void *stream);

/*
 * The two halves of moe_expert_ffn, for callers that schedule or time them
 * separately.  moe_expert_gate_up computes h (kept in `workspace`);
 * moe_expert_down reads h from the same workspace and writes y_perm.  Called
 * in that order on one stream with one workspace they are exactly
 * moe_expert_ffn.  Arguments as for moe_expert_ffn.
 */
moe_status_t moe_expert_gate_up(const moe_desc_t *desc, const void *x_perm, const uint8_t *x_perm_scale,
                                const int32_t *offsets, const moe_ffn_weights_t *experts,
                                void *workspace, size_t ws_bytes, void *stream);
moe_status_t moe_expert_down(const moe_desc_t *desc, const int32_t *offsets,
                             const moe_ffn_weights_t *experts, void *y_perm, void *workspace,
                             size_t ws_bytes, void *stream);

/*
 * moe_expert_gate_up with the dispatch gather folded into the GEMM: row r of
 * the grouped GEMM's input is token row_src[r] / k of x, read in place, so no
 * x_perm is materialised (the same rows in the same order as moe_dispatch's
 * x_perm, hence the same h bit for bit).  With wt = e4m3, x is first
 * quantised once per token (T rows, 1x128 tiles, as in moe_dispatch) into the
 * workspace.
 *   x         [T, d] act type (the layer input given to moe_dispatch)
 *   row_src   [T*k]  int32 from moe_dispatch (flat assignment ids t*k + j;
 *             row r of the GEMM reads token row_src[r] / k)
 *   offsets, experts, workspace: as for moe_expert_gate_up
 * Then moe_expert_down as usual.
 */
moe_status_t moe_expert_gate_up_rows(const moe_desc_t *desc, const void *x, const int32_t *row_src,
                                     const int32_t *offsets, const moe_ffn_weights_t *experts,
                                     void *workspace, size_t ws_bytes, void *stream);

/*
 * Shared expert plus weighted combine (Scaling Efficiency ..., "Implementation:
 * A Modular Look": shared output plus the routed outputs scaled by their
 * weights; DeepSeek V3 From Scratch, "The idea": one shared expert for every
 * token).
 *   y[t] = shared(x[t]) + sum_{j<k} weights[t, j] * y_perm[row_of[t*k + j]]
 * with the j-sum in ascending expert-id order, in fp32; the shared expert's
 * fp32 accumulator is not rounded before the sum (at small T with bf16
 * weights its K range is split over workgroups and the fp32 partial sums are
 * added in a fixed order, so the result is still deterministic).  The shared expert has the
 * SwiGLU form of the routed ones; with wt = e4m3 its input is x quantised per
 * 1x128 tile (as in moe_dispatch) inside the workspace.
 *   x        [T, d] act type
 *   shared   one expert (G = 1)
 *   y_perm, row_of, weights: from moe_expert_ffn, moe_dispatch, moe_route
 *   y        [T, d] fp32 out
 *   workspace >= moe_workspace_bytes(desc, MOE_WS_COMBINE) bytes of device memory
 */
moe_status_t moe_combine(const moe_desc_t *desc, const void *x, const moe_ffn_weights_t *shared,
                         const void *y_perm, const int32_t *row_of, const float *weights,
                         float *y, void *workspace, size_t ws_bytes, void *stream);

/*
 * Sign-step bias update, once per step after the forward (DeepSeek V3 From
 * Scratch, "In code": update_bias; kbwen.com DeepSeek feed, "A bias term for
 * each expert"):  with load_e = counts[e] / T and target = k / E,
 *   bias[e] <- fl32(bias[e] + gamma * sign(target - load_e)),
 * sign(0) = 0.  The sign is evaluated exactly as sign(k*T - E*counts[e]).
 *   counts [E] int32 (from moe_dispatch); bias [E] fp32, updated in place.
 */
moe_status_t moe_bias_update(const moe_desc_t *desc, const int32_t *counts, float gamma,
                             float *bias, void *stream);

/* Device workspace, in bytes, that a call of the given stage needs for this
 * shape (0 when the shape is invalid). */
size_t moe_workspace_bytes(const moe_desc_t *desc, int32_t stage);

/*
 * Backward of the layer: the gradients of the layer output y for the
 * routing the forward chose, given dy = dL/dy (act = bf16 with wt = bf16 or
 * e4m3; other types give MOE_ENOTSUP).  What is differentiated is the forward above
 * (DeepSeek V3 From Scratch, "The idea", "In code"; Scaling Efficiency ...,
 * "Implementation: A Modular Look"):
 *   y = shared(x) + sum_j g_j * y_perm_j,  g_j = s_j / sum_i s_i over the
 *   chosen experts,  s_e = sigmoid(x . w_router[e]).
 * The choice is piecewise constant and carries no gradient; the bias is used
 * only for the choice and gets no gradient (kbwen.com DeepSeek feed, "A bias
 * term for each expert").  Inside: the routed and shared output gradients
 * (g_j dy and dy) and the SwiGLU input gradients are rounded to bf16 as GEMM
 * inputs, like h in the forward; the expert pre-activations are recomputed;
 * accumulation is fp32.  Deterministic (no atomics).
 * With e4m3 weights (crackai.dev DeepSeek-V3 summary, "How It Works": FP8
 * in the backward pass too, a scale per tile) every backward GEMM takes e4m3
 * operands quantised per 1x128 tile along its reduction: row tiles for the
 * data gradients (against the weight blocks, transposed as blocks); for the
 * weight gradients, each column of a group of 128 of an expert's rows
 * (dispatch order; the shared expert: 128 consecutive tokens) is one tile,
 * quantised from the fp32 values and the bf16 x.
 *   x          [T, d] bf16, the forward's input
 *   w_router   [E, d] fp32
 *   idx, weights [T, k]: from moe_route
 *   offsets, row_src, row_of: from moe_dispatch
 *   experts, shared: as for the forward (bf16, or e4m3 with block scales)
 *   y_perm     [T*k, d] bf16: the forward's routed outputs (moe_expert_ffn)
 *   dy         [T, d] fp32
 * Outputs (fp32, written, not accumulated):
 *   dx [T, d]; dw_router [E, d]; dw_gate, dw_up [E, I, d]; dw_down [E, d, I];
 *   ds_gate, ds_up [I, d]; ds_down [d, I] (the shared expert);
 *   dg [T, k] the combine-weight gradients dy . y_perm_j (NULL: not returned).
 *   workspace >= moe_workspace_bytes(desc, MOE_WS_BACKWARD) bytes of device
 *   memory: about (T*k + T)(6d + 18I) for the per-row intermediates, plus
 *   (T*k + 64E + T)(4d + 6I) for their K-contiguous transposes, 64*E*d
 *   for the router partials, and, only where the data-gradient products
 *   cannot read the weights as stored (fewer than 128 rows per expert on
 *   average, or d or I not a multiple of 256), 6(E + 1)*I*d for transposed
 *   weights
 *   (about 17 GiB at T=16384, d=7168, I=2048, E=256, k=8; with e4m3 weights,
 *   which are always transposed as blocks, about 31 GiB).
 * Requires d % 128 == 0 and I % 128 == 0.
 */
moe_status_t moe_backward(const moe_desc_t *desc, const void *x, const float *w_router, const int32_t *idx,
                          const float *weights, const int32_t *offsets, const int32_t *row_src,
                          const int32_t *row_of, const moe_ffn_weights_t *experts,
                          const moe_ffn_weights_t *shared, const void *y_perm, const float *dy, float *dx,
                          float *dw_router, float *dw_gate, float *dw_up, float *dw_down, float *ds_gate,
                          float *ds_up, float *ds_down, float *dg, void *workspace, size_t ws_bytes,
                          void *stream);

/* Static, human-readable name of a status code. */
const char *moe_status_str(moe_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
