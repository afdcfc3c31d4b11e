/*
 * CPU oracle for the DeepSeekMoE layer forward with auxiliary-loss-free
 * (bias) routing, and its backward (gradients of the layer output).  TEST INFRASTRUCTURE: only the tests, the smoke check and
 * the bench's CPU-baseline leg may load this library.  It shares no code,
 * header or table with the HIP path.
 *
 * Plain loops, fp64 accumulation, one token at a time, written from the
 * pages' statement of the method:
 *   - DeepSeek V3 From Scratch, "The idea", "Worked example" (routing,
 *     concretely) and "In code" (route, update_bias): sigmoid affinities,
 *     the per-expert bias added for the top-8 choice only, combine weights
 *     from the unbiased affinities of the chosen 8 renormalised to sum to 1,
 *     and the sign-step bias update.
 *   - kbwen.com DeepSeek feed, "A bias term for each expert": the bias moves
 *     once per step, over the whole batch, by a fixed 0.001 up or down; no
 *     token is dropped.
 *   - Scaling Efficiency: A Deep Dive into the DeepSeek-V3 Architecture,
 *     "Implementation: A Modular Look": shared expert added to the routed
 *     sum; each routed expert applied to the tokens that chose it and its
 *     output accumulated with that token's weight.
 *   - crackai.dev DeepSeek-V3 summary, "How It Works": 256 routed + 1 shared
 *     expert, top-8; FP8 matmuls with a scale per tile and FP32 accumulation.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - expert FFN is a bias-free SwiGLU: y = Wd (silu(Wg a) * (Wu a));
 *   - ties among equal biased scores go to the lower expert id; the k chosen
 *     ids are reported in ascending id order;
 *   - the selection is decided on fp32 biased scores fl32(fl32(s) + b), the
 *     precision the kernel decides in; the fp64 gap between the k-th and
 *     (k+1)-th largest fp64 biased score is reported so that near-ties
 *     (gap < 1e-6) can be told apart;
 *   - load_i = c_i / T, target = k / E, so sign(target - load_i) =
 *     sign(k*T - E*c_i), evaluated exactly in integers;
 *   - rounding points: h and y_perm are rounded to the storage type the
 *     kernel keeps them in (fp32, bf16, or e4m3 per 1x128 tile for h), the
 *     shared expert's output and y stay unrounded until the fp32 output;
 *   - e4m3 (OCP E4M3FN) tile/block scale = the smallest power of two at or
 *     above amax / 448 (fp32 quotient; 1 if amax = 0), code =
 *     round-to-nearest-even(v / scale), saturating; every scale that crosses
 *     the interface is stored as an OCP MX E8M0 byte (byte e stands for
 *     2^(e - 127), 255 for NaN).
 *
 * Build: gcc -O2 -fopenmp -fno-fast-math -ffp-contract=off -shared -fPIC
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F32 = 0, OR_BF16 = 1, OR_E4M3 = 2 };

typedef struct {
    int32_t T, d, E, k, I;
    int32_t act; /* storage type of x: OR_F32 or OR_BF16 */
    int32_t wt;  /* storage type of expert weights = expert GEMM input type */
} or_shape;

typedef struct {
    const void *gate, *up, *down;           /* [G,I,d], [G,I,d], [G,d,I] */
    const uint8_t *s_gate, *s_up, *s_down;  /* e4m3 only: 128x128 block scales, E8M0 */
} or_ffn;

/* ------------------------------------------------------------------ codecs */

/* bf16: the upper 16 bits of an IEEE binary32. */
static double bf16_dec(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Round a binary32 to the nearest bf16, ties to the even bf16. */
static uint16_t bf16_enc(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t lower = u & 0xFFFFu;
    uint32_t upper = u >> 16;
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1u;
    return (uint16_t)upper;
}

static double bf16_round(double v) { return bf16_dec(bf16_enc((float)v)); }

/* OCP E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent field 0
 * is subnormal (m/8 * 2^-6); S.1111.111 is NaN; no infinities; max 448. */
static double e4m3_formula(uint8_t c) {
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m / 8.0, -6);
    else v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -v : v;
}

/* The formula, evaluated for each of the 256 codes when the library loads
 * (codec_tables below). */
static double e4m3_table[256];

static double e4m3_dec(uint8_t c) { return e4m3_table[c]; }

/* Nearest E4M3FN code to v (finite), ties to the code with even mantissa,
 * magnitudes beyond 448 saturate to 448.  Written as a search over the 127
 * non-negative finite codes, which increase in value with the code. */
static uint8_t e4m3_enc(float vf) {
    double v = (double)vf;
    double a = fabs(v);
    uint8_t sign = (v < 0.0 || (v == 0.0 && signbit(v))) ? 0x80 : 0x00;
    if (a >= 448.0) return sign | 0x7E;
    int lo = 0, hi = 0x7E; /* value(lo) <= a < value(hi) after the search */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (e4m3_dec((uint8_t)mid) <= a) lo = mid; else hi = mid;
    }
    double dlo = a - e4m3_dec((uint8_t)lo), dhi = e4m3_dec((uint8_t)hi) - a;
    int c;
    if (dlo < dhi) c = lo;
    else if (dhi < dlo) c = hi;
    else c = (lo & 1) ? hi : lo;
    return sign | (uint8_t)c;
}

/* OCP MX E8M0 scale byte: an 8-bit biased exponent with no sign and no
 * mantissa, bias 127; 255 encodes NaN. */
static double e8m0_formula(uint8_t e) { return e == 255 ? NAN : ldexp(1.0, (int)e - 127); }

/* The formula, evaluated for each of the 256 bytes when the library loads
 * (the weight loops decode a block scale per element). */
static double e8m0_table[256];

static double e8m0_dec(uint8_t e) { return e8m0_table[e]; }

/* Both decode tables, filled from their formulas before any exported
 * function can run. */
__attribute__((constructor)) static void codec_tables(void) {
    for (int i = 0; i < 256; ++i) {
        e4m3_table[i] = e4m3_formula((uint8_t)i);
        e8m0_table[i] = e8m0_formula((uint8_t)i);
    }
}

/* The E8M0 byte of a power of two s (2^-127 <= s <= 2^127): s = 0.5 * 2^ex
 * by frexp, so its exponent is ex - 1. */
static uint8_t e8m0_enc(double s) {
    int ex = 0;
    frexp(s, &ex);
    return (uint8_t)(ex - 1 + 127);
}

/* Exposed for the codec pins. */
double oracle_e8m0_decode(uint8_t e) { return e8m0_dec(e); }
double oracle_bf16_decode(uint16_t b) { return bf16_dec(b); }
uint16_t oracle_bf16_encode(float f) { return bf16_enc(f); }
double oracle_e4m3_decode(uint8_t c) { return e4m3_dec(c); }
uint8_t oracle_e4m3_encode(float f) { return e4m3_enc(f); }

/* The scale of a tile whose largest magnitude is amax: the smallest power of
 * two at or above amax / 448 (the fp32 quotient), 1 when amax = 0. */
static float tile_scale(float amax) {
    if (!(amax > 0.0f)) return 1.0f;
    float t = amax / 448.0f;
    uint32_t b;
    memcpy(&b, &t, 4);
    if (b & 0x7FFFFFu) b = (b & 0xFF800000u) + 0x800000u; /* next power of two */
    float s;
    memcpy(&s, &b, 4);
    return s;
}

/* One 1x128 tile: scale from tile_scale, codes of v / scale (fp32 division,
 * exact for a power of two).  Fine-grained fp8 tiles: crackai.dev
 * DeepSeek-V3 summary, "How It Works" (a scale per tile, FP32 accumulation);
 * DeepSeek V3 From Scratch, "The idea". */
static float quant_tile(const float *v, int n, uint8_t *q) {
    float amax = 0.0f;
    for (int i = 0; i < n; ++i) {
        float a = fabsf(v[i]);
        if (a > amax) amax = a;
    }
    float s = tile_scale(amax);
    for (int i = 0; i < n; ++i) q[i] = e4m3_enc(v[i] / s);
    return s;
}

/* Quantise rows of `cols` values (cols % 128 == 0) per 1x128 tile.
 * in_dtype OR_F32 or OR_BF16.  q: [rows, cols], scales: [rows, cols/128] E8M0. */
void oracle_quant_e4m3_rows(int64_t rows, int32_t cols, int32_t in_dtype, const void *in,
                            uint8_t *q, uint8_t *scales) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        float v[128];
        for (int tb = 0; tb < cols / 128; ++tb) {
            for (int i = 0; i < 128; ++i) {
                int64_t j = r * cols + tb * 128 + i;
                v[i] = in_dtype == OR_BF16 ? (float)bf16_dec(((const uint16_t *)in)[j])
                                           : ((const float *)in)[j];
            }
            scales[r * (cols / 128) + tb] = e8m0_enc(quant_tile(v, 128, q + r * cols + tb * 128));
        }
    }
}

/* ----------------------------------------------------------- element access */

static double x_at(const or_shape *sh, const void *x, int64_t t, int64_t j) {
    int64_t i = t * sh->d + j;
    return sh->act == OR_BF16 ? bf16_dec(((const uint16_t *)x)[i]) : (double)((const float *)x)[i];
}

/* Weight element [g, n, j] of a [G, N, K] stack (with [G, N/128, K/128]
 * block scales for e4m3). */
static double w_at(int dtype, const void *w, const uint8_t *s, int64_t N, int64_t K, int64_t g,
                   int64_t n, int64_t j) {
    int64_t i = (g * N + n) * K + j;
    if (dtype == OR_F32) return (double)((const float *)w)[i];
    if (dtype == OR_BF16) return bf16_dec(((const uint16_t *)w)[i]);
    double sc = e8m0_dec(s[(g * (N / 128) + n / 128) * (K / 128) + j / 128]);
    return e4m3_dec(((const uint8_t *)w)[i]) * sc;
}

/* The expert FFN input for token t: x itself, or x quantised per 1x128 tile
 * when the expert GEMMs run in e4m3 (dequantised values q * s). */
static void gemm_input_row(const or_shape *sh, const void *x, int64_t t, double *a) {
    if (sh->wt != OR_E4M3) {
        for (int j = 0; j < sh->d; ++j) a[j] = x_at(sh, x, t, j);
        return;
    }
    float v[128];
    uint8_t q[128];
    for (int tb = 0; tb < sh->d / 128; ++tb) {
        for (int i = 0; i < 128; ++i) v[i] = (float)x_at(sh, x, t, tb * 128 + i);
        double s = (double)quant_tile(v, 128, q);
        for (int i = 0; i < 128; ++i) a[tb * 128 + i] = e4m3_dec(q[i]) * s;
    }
}

/* Round an intermediate vector to the storage type the GEMM consumes it in. */
static void round_to_gemm_input(int wt, double *h, int n) {
    if (wt == OR_F32) {
        for (int i = 0; i < n; ++i) h[i] = (double)(float)h[i];
    } else if (wt == OR_BF16) {
        for (int i = 0; i < n; ++i) h[i] = bf16_round(h[i]);
    } else {
        float v[128];
        uint8_t q[128];
        for (int tb = 0; tb < n / 128; ++tb) {
            for (int i = 0; i < 128; ++i) v[i] = (float)h[tb * 128 + i];
            double s = (double)quant_tile(v, 128, q);
            for (int i = 0; i < 128; ++i) h[tb * 128 + i] = e4m3_dec(q[i]) * s;
        }
    }
}

/* ---------------------------------------------------------------- the FFN */

/* One SwiGLU expert (index g of the stack) on one input row a[d]:
 *   u_g = Wg a, u_u = Wu a, h = silu(u_g) * u_u with silu(z) = z / (1 + e^-z),
 *   h rounded to the GEMM input type, y = Wd h.  fp64 throughout.
 * Expert structure: Scaling Efficiency ..., "Implementation: A Modular Look"
 * (one MLP per routed expert plus one shared MLP); gated form: our reading. */
static void ffn_row(const or_shape *sh, const or_ffn *w, int64_t g, const double *a, double *y,
                    double *hbuf) {
    const int64_t d = sh->d, I = sh->I;
    for (int64_t n = 0; n < I; ++n) {
        double ug = 0.0, uu = 0.0;
        for (int64_t j = 0; j < d; ++j) {
            ug += w_at(sh->wt, w->gate, w->s_gate, I, d, g, n, j) * a[j];
            uu += w_at(sh->wt, w->up, w->s_up, I, d, g, n, j) * a[j];
        }
        hbuf[n] = ug / (1.0 + exp(-ug)) * uu;
    }
    round_to_gemm_input(sh->wt, hbuf, (int)I);
    for (int64_t n = 0; n < d; ++n) {
        double acc = 0.0;
        for (int64_t i = 0; i < I; ++i) acc += w_at(sh->wt, w->down, w->s_down, d, I, g, n, i) * hbuf[i];
        y[n] = acc;
    }
}

/* y_perm storage: fp32 when the layer is fp32, else bf16. */
static double round_yperm(const or_shape *sh, double v) {
    return sh->wt == OR_F32 ? (double)(float)v : bf16_round(v);
}

/* ------------------------------------------------------------- the router */

/* The choice for one token from its fp64 affinities s[E] (DeepSeek V3 From
 * Scratch, "In code" (route) and "Worked example"; kbwen.com DeepSeek feed,
 * "A bias term for each expert"): the k experts with the largest biased score
 * s + b are chosen; their unbiased s, divided by the sum over the chosen k,
 * are the combine weights.  The score is formed as the kernel forms it,
 * fl32(fl32(s) + b), and equal scores go to the lower id.
 *   idx[k]: chosen ids, ascending; wgt[k]: weights in that order;
 *   *gap: (k-th largest) - ((k+1)-th largest) fp64 biased score s + b. */
static void choose_token(int E, int k, const double *s, const float *bias, int32_t *idx, double *wgt,
                         double *gap) {
    float *v32 = (float *)malloc(sizeof(float) * E);
    char *taken = (char *)calloc((size_t)(E > 0 ? E : 1), 1);
    for (int e = 0; e < E; ++e) v32[e] = (float)s[e] + bias[e]; /* fp32 add */
    /* k rounds of "largest remaining biased score; equal scores -> lower id" */
    for (int r = 0; r < k; ++r) {
        int best = -1;
        for (int e = 0; e < E; ++e)
            if (!taken[e] && (best < 0 || v32[e] > v32[best])) best = e;
        taken[best] = 1;
    }
    int n = 0;
    for (int e = 0; e < E; ++e)
        if (taken[e]) idx[n++] = e;
    double sum = 0.0;
    for (int j = 0; j < k; ++j) sum += s[idx[j]];
    for (int j = 0; j < k; ++j) wgt[j] = s[idx[j]] / sum;
    if (gap) {
        double *v = (double *)malloc(sizeof(double) * E);
        for (int e = 0; e < E; ++e) v[e] = s[e] + (double)bias[e];
        double kth = 0.0, k1th = 0.0;
        memset(taken, 0, (size_t)E);
        for (int r = 0; r <= k && r < E; ++r) {
            int best = -1;
            for (int e = 0; e < E; ++e)
                if (!taken[e] && (best < 0 || v[e] > v[best])) best = e;
            taken[best] = 1;
            if (r == k - 1) kth = v[best];
            if (r == k) k1th = v[best];
        }
        *gap = (k < E) ? kth - k1th : INFINITY;
        free(v);
    }
    free(v32);
    free(taken);
}

/* Affinities of one token: s_e = sigmoid(x_t . w_e) = 1 / (1 + e^-l), fp64
 * (DeepSeek V3 From Scratch, "In code": route).  No router bias term. */
static void affinity_token(const or_shape *sh, const void *x, const float *wr, int64_t t, double *s) {
    const int E = sh->E, d = sh->d;
    for (int e = 0; e < E; ++e) {
        double l = 0.0;
        for (int j = 0; j < d; ++j) l += x_at(sh, x, t, j) * (double)wr[(int64_t)e * d + j];
        s[e] = 1.0 / (1.0 + exp(-l));
    }
}

static void route_token(const or_shape *sh, const void *x, const float *wr, const float *bias,
                        int64_t t, int32_t *idx, double *wgt, double *gap, double *s_out) {
    double *s = (double *)malloc(sizeof(double) * sh->E);
    affinity_token(sh, x, wr, t, s);
    choose_token(sh->E, sh->k, s, bias, idx, wgt, gap);
    if (s_out) memcpy(s_out, s, sizeof(double) * sh->E);
    free(s);
}

/* The choice alone for ntok tokens whose fp64 affinities are given ([ntok, E]). */
void oracle_choose(int64_t ntok, int32_t E, int32_t k, const double *s, const float *bias, int32_t *idx,
                   float *g, double *gap) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < ntok; ++i) {
        double w[64];
        choose_token(E, k, s + i * E, bias, idx + i * k, w, gap ? gap + i : NULL);
        for (int j = 0; j < k; ++j) g[i * k + j] = (float)w[j];
    }
}

/* Route a list of tokens (tok == NULL: tokens 0..ntok-1).
 * idx, g: [ntok, k]; gap: [ntok] or NULL; s_out: [ntok, E] or NULL. */
void oracle_route(const or_shape *sh, const void *x, const float *wr, const float *bias,
                  int64_t ntok, const int32_t *tok, int32_t *idx, float *g, double *gap,
                  double *s_out) {
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t i = 0; i < ntok; ++i) {
        int64_t t = tok ? tok[i] : i;
        double w[64];
        route_token(sh, x, wr, bias, t, idx + i * sh->k, w, gap ? gap + i : NULL,
                    s_out ? s_out + i * sh->E : NULL);
        for (int j = 0; j < sh->k; ++j) g[i * sh->k + j] = (float)w[j];
    }
}

/* ----------------------------------------------------------- the dispatch */

/* Load per expert, its exclusive prefix sum, and the stable grouping of the
 * T*k assignments by expert (flat id f = t*k + j kept in ascending order
 * within an expert).  Load: DeepSeek V3 From Scratch, "In code"
 * (update_bias: fraction of tokens per expert); the per-expert gather:
 * Scaling Efficiency ..., "Implementation: A Modular Look".
 *   counts[E], offsets[E+1], row_src[T*k] (row -> flat id), row_of[T*k]. */
void oracle_dispatch(int32_t T, int32_t E, int32_t k, const int32_t *idx, int32_t *counts,
                     int32_t *offsets, int32_t *row_src, int32_t *row_of) {
    int64_t A = (int64_t)T * k;
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (int64_t f = 0; f < A; ++f) counts[idx[f]]++;
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int32_t *fill = (int32_t *)calloc((size_t)(E > 0 ? E : 1), sizeof(int32_t));
    for (int64_t f = 0; f < A; ++f) {
        int e = idx[f];
        int32_t r = offsets[e] + fill[e]++;
        row_src[r] = (int32_t)f;
        row_of[f] = r;
    }
    free(fill);
}

/* -------------------------------------------------------- the bias update */

/* DeepSeek V3 From Scratch, "In code" (update_bias): b <- b + step *
 * sign(target - load); kbwen.com DeepSeek feed, "A bias term for each
 * expert": once per step over the whole batch, the same fixed amount up or
 * down (0.001).  With load = c/T and target = k/E, sign(target - load) =
 * sign(k*T - E*c).  b is fp32 state: b <- fl32(b + fl32(gamma) * sign). */
void oracle_bias_update(int32_t E, int32_t k, int32_t T, const int32_t *counts, float gamma,
                        float *bias) {
    for (int e = 0; e < E; ++e) {
        int64_t diff = (int64_t)k * T - (int64_t)E * counts[e];
        float sg = diff > 0 ? 1.0f : (diff < 0 ? -1.0f : 0.0f);
        bias[e] = bias[e] + gamma * sg;
    }
}

/* -------------------------------------------------- expert FFN and combine */

/* Routed expert FFN on permuted rows (the expert FFN stage on its own):
 * row r in [offsets[e], offsets[e+1]) goes through expert e.
 * a_rows: [A, d] in the GEMM input type (f32, bf16 bits, or e4m3 codes with
 * a_scales [A, d/128]).  Rows computed: `rows` (nrows of them) or 0..nrows-1.
 * y_perm: [nrows, d] fp32 or bf16 bits (see round_yperm), in list order. */
void oracle_expert_ffn(const or_shape *sh, const or_ffn *w, const int32_t *offsets,
                       const void *a_rows, const uint8_t *a_scales, int64_t nrows, const int32_t *rows,
                       void *y_perm) {
    const int64_t d = sh->d;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t ri = 0; ri < nrows; ++ri) {
        const int64_t r = rows ? rows[ri] : ri;
        int e = 0;
        while (offsets[e + 1] <= r) ++e;
        double *a = (double *)malloc(sizeof(double) * d);
        double *y = (double *)malloc(sizeof(double) * d);
        double *h = (double *)malloc(sizeof(double) * sh->I);
        for (int64_t j = 0; j < d; ++j) {
            int64_t i = r * d + j;
            if (sh->wt == OR_F32) a[j] = ((const float *)a_rows)[i];
            else if (sh->wt == OR_BF16) a[j] = bf16_dec(((const uint16_t *)a_rows)[i]);
            else a[j] = e4m3_dec(((const uint8_t *)a_rows)[i]) * e8m0_dec(a_scales[r * (d / 128) + j / 128]);
        }
        ffn_row(sh, w, e, a, y, h);
        for (int64_t j = 0; j < d; ++j) {
            double v = round_yperm(sh, y[j]);
            if (sh->wt == OR_F32) ((float *)y_perm)[ri * d + j] = (float)v;
            else ((uint16_t *)y_perm)[ri * d + j] = bf16_enc((float)v);
        }
        free(a);
        free(y);
        free(h);
    }
}

/* Shared expert plus the weighted sum of each token's k routed rows:
 * y[t] = shared(x[t]) + sum_j g[t,j] * y_perm[row_of[t*k + j]], j ascending
 * (= ascending expert id).  Scaling Efficiency ..., "Implementation: A
 * Modular Look" (shared output + routed output, routed rows scaled by their
 * weight); DeepSeek V3 From Scratch, "The idea" (one shared expert every
 * token uses).  y: [ntok, d] fp32. */
void oracle_combine(const or_shape *sh, const or_ffn *shared, const void *x, const void *y_perm,
                    const int32_t *row_of, const float *g, int64_t ntok, const int32_t *tok,
                    float *y) {
    const int64_t d = sh->d, k = sh->k;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < ntok; ++i) {
        int64_t t = tok ? tok[i] : i;
        double *a = (double *)malloc(sizeof(double) * d);
        double *ys = (double *)malloc(sizeof(double) * d);
        double *h = (double *)malloc(sizeof(double) * sh->I);
        gemm_input_row(sh, x, t, a);
        ffn_row(sh, shared, 0, a, ys, h);
        for (int64_t j = 0; j < d; ++j) {
            double acc = ys[j];
            for (int64_t q = 0; q < k; ++q) {
                int64_t r = row_of[t * k + q];
                double v = sh->wt == OR_F32 ? (double)((const float *)y_perm)[r * d + j]
                                            : bf16_dec(((const uint16_t *)y_perm)[r * d + j]);
                acc += (double)g[t * k + q] * v;
            }
            y[i * d + j] = (float)acc;
        }
        free(a);
        free(ys);
        free(h);
    }
}

/* ------------------------------------------------------ the whole forward */

/* The layer forward for a list of tokens (tok == NULL: 0..ntok-1).  Each
 * token is independent of the others given the bias: route, run its k
 * experts and the shared expert, combine.  idx, g: [ntok, k]; gap: [ntok]
 * or NULL; y: [ntok, d] fp32. */
void oracle_forward(const or_shape *sh, const void *x, const float *wr, const float *bias,
                    const or_ffn *experts, const or_ffn *shared, int64_t ntok, const int32_t *tok,
                    int32_t *idx, float *g, double *gap, float *y) {
    const int64_t d = sh->d, k = sh->k;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < ntok; ++i) {
        int64_t t = tok ? tok[i] : i;
        double w[64];
        route_token(sh, x, wr, bias, t, idx + i * k, w, gap ? gap + i : NULL, NULL);
        for (int64_t j = 0; j < k; ++j) g[i * k + j] = (float)w[j];
        double *a = (double *)malloc(sizeof(double) * d);
        double *yr = (double *)malloc(sizeof(double) * d);
        double *acc = (double *)malloc(sizeof(double) * d);
        double *h = (double *)malloc(sizeof(double) * sh->I);
        gemm_input_row(sh, x, t, a);
        ffn_row(sh, shared, 0, a, acc, h);
        for (int64_t j = 0; j < k; ++j) {
            ffn_row(sh, experts, idx[i * k + j], a, yr, h);
            for (int64_t n = 0; n < d; ++n) acc[n] += w[j] * round_yperm(sh, yr[n]);
        }
        for (int64_t n = 0; n < d; ++n) y[i * d + n] = (float)acc[n];
        free(a);
        free(yr);
        free(acc);
        free(h);
    }
}

/* ------------------------------------------------------ the backward pass */

/* One SwiGLU expert's forward intermediates and backward on one row, fp64:
 *   ug = Wg a, uu = Wu a, h = round(silu(ug) * uu) as the forward stores it;
 *   given the output gradient dyr (already in the GEMM input type):
 *   dh = Wd^T dyr;  d silu(z)/dz = sig(z) (1 + z (1 - sig(z)));
 *   dug = round(dh * uu * silu'(ug)), duu = round(dh * silu(ug)) (the GEMM
 *   inputs of the backward GEMMs, rounded like h);
 *   da = Wg^T dug + Wu^T duu.
 * The rounding of h and of the routed output is taken as the identity in
 * the derivative.  raw (optional, [3][I]): h, dug, duu before rounding. */
static void ffn_row_backward(const or_shape *sh, const or_ffn *w, int64_t g, const double *a,
                             const double *dyr, double *h, double *dug, double *duu, double *da,
                             double *raw) {
    const int64_t d = sh->d, I = sh->I;
    for (int64_t i = 0; i < I; ++i) {
        double ug = 0.0, uu = 0.0;
        for (int64_t j = 0; j < d; ++j) {
            ug += w_at(sh->wt, w->gate, w->s_gate, I, d, g, i, j) * a[j];
            uu += w_at(sh->wt, w->up, w->s_up, I, d, g, i, j) * a[j];
        }
        const double sg = 1.0 / (1.0 + exp(-ug));
        double dh = 0.0;
        for (int64_t n = 0; n < d; ++n) dh += w_at(sh->wt, w->down, w->s_down, d, I, g, n, i) * dyr[n];
        h[i] = ug * sg * uu;
        dug[i] = dh * uu * sg * (1.0 + ug * (1.0 - sg));
        duu[i] = dh * ug * sg;
        if (raw) {
            raw[i] = h[i];
            raw[I + i] = dug[i];
            raw[2 * I + i] = duu[i];
        }
    }
    round_to_gemm_input(sh->wt, h, (int)I);
    round_to_gemm_input(sh->wt, dug, (int)I);
    round_to_gemm_input(sh->wt, duu, (int)I);
    for (int64_t j = 0; j < d; ++j) {
        double acc = 0.0;
        for (int64_t i = 0; i < I; ++i)
            acc += w_at(sh->wt, w->gate, w->s_gate, I, d, g, i, j) * dug[i] +
                   w_at(sh->wt, w->up, w->s_up, I, d, g, i, j) * duu[i];
        da[j] = acc;
    }
}

/* Gradients of the layer's output y (given dy = dL/dy, [T, d] fp32) for the
 * routing idx [T, k] (ascending ids; the choice itself is piecewise constant
 * and carries no gradient, and the bias, used only for the choice, gets none:
 * kbwen.com DeepSeek feed, "A bias term for each expert").  Weights and
 * activations as in the forward (f32 or bf16; the GEMM inputs of the
 * backward -- the routed and shared output gradients, the SwiGLU input
 * gradients -- are rounded to that type like h):
 *   y = shared(x) + sum_j g_j * yperm_j,  g_j = s_j / sum_i s_i (chosen i),
 *   s_e = sigmoid(x . wr_e);
 *   dg_j = dy . yperm_j (yperm_j recomputed as the forward stores it);
 *   the routed output gradient of (t, j) is round(g_j dy); the shared one
 *   round(dy);
 *   ds_j = (dg_j - sum_i g_i dg_i) / sum_i s_i,  dl_j = ds_j s_j (1 - s_j);
 *   dx = sum_j (routed input gradient) + (shared input gradient)
 *        + sum_j dl_j wr_{e_j};
 *   dwr_e = sum over (t, j) with idx = e of dl_j x_t;
 *   dWg_e = sum over e's rows of dug (x) a, dWu_e likewise with duu,
 *   dWd_e = sum of (routed output gradient) (x) h; the shared expert's over
 *   all tokens.
 * e4m3 weights (fp8 GEMMs in the backward too: crackai.dev DeepSeek-V3
 * summary, "How It Works"; our reading of where the tiles lie): every
 * backward GEMM takes e4m3 operands, each quantised per 1x128 tile along
 * that GEMM's reduction.  The data-gradient GEMMs reduce along a row: the
 * output gradients (g_j dy, dy) per 1x128 tile of d, the SwiGLU input
 * gradients per 1x128 tile of I (round_to_gemm_input), against the stored
 * weight blocks.  The weight-gradient GEMMs reduce over an expert's rows:
 * the rows in dispatch order (ascending t*k + j; the shared expert: tokens
 * in order) form groups of 128 (the last one short, as if padded with
 * zeros), and every column of a group is one tile, quantised from the
 * unrounded fp32 values -- dug, duu, h = silu(ug) uu and the output
 * gradient -- and from the bf16 x.  The router stays fp32.
 * Outputs fp32: dx [T, d], dwr [E, d], dwg, dwu [E, I, d], dwd [E, d, I],
 * dsg, dsu [I, d], dsd [d, I], dg [T, k].
 * wsel selects the weight gradients: -1 all of them; -2 none (dx and dg
 * only); e >= 0 routed expert e's alone (dwg, dwu, dwd and dwr hold one
 * expert's slice, [1, I, d], [1, d, I] and [1, d]; the shared expert's are
 * not computed). */
/* Quantise each of the ncols columns of g [nr, ncols] (nr <= 128 rows of one
 * group) as one 128-value tile, the rows past nr counting as zeros; g is
 * replaced by the dequantised values. */
static void quant_cols(double *g, int nr, int64_t ncols) {
    float v[128];
    uint8_t q[128];
    for (int64_t c = 0; c < ncols; ++c) {
        for (int i = 0; i < 128; ++i) v[i] = i < nr ? (float)g[i * ncols + c] : 0.0f;
        const double sc = (double)quant_tile(v, 128, q);
        for (int i = 0; i < nr; ++i) g[i * ncols + c] = e4m3_dec(q[i]) * sc;
    }
}

/* e4m3 weight gradients of one FFN over the rows rows[0..n) (dispatch
 * order), in groups of 128: gw, uw [I, d] += Q(dug)^T Q(x), Q(duu)^T Q(x);
 * dw [d, I] += Q(dy)^T Q(h), each operand quantised per column of a group.
 * xrow(r): the token of row r; draw: [rows, 3I] raw (h, dug, duu); dyraw:
 * [rows, d] the unrounded output gradient. */
static void wgrad_e4m3(const or_shape *sh, const void *x, const int64_t *rows, int64_t n, int64_t kdiv,
                       const double *draw, const double *dyraw, double *gw, double *uw, double *dw) {
    const int64_t d = sh->d, I = sh->I;
    double *gx = (double *)malloc(sizeof(double) * 128 * d);
    double *gy = (double *)malloc(sizeof(double) * 128 * d);
    double *gg = (double *)malloc(sizeof(double) * 128 * I);
    double *gu = (double *)malloc(sizeof(double) * 128 * I);
    double *gh = (double *)malloc(sizeof(double) * 128 * I);
    for (int64_t g0 = 0; g0 < n; g0 += 128) {
        const int nr = (int)(n - g0 < 128 ? n - g0 : 128);
        for (int i = 0; i < nr; ++i) {
            const int64_t f = rows[g0 + i];
            for (int64_t c = 0; c < d; ++c) {
                gx[i * d + c] = x_at(sh, x, f / kdiv, c);
                gy[i * d + c] = dyraw[f * d + c];
            }
            for (int64_t c = 0; c < I; ++c) {
                gh[i * I + c] = draw[f * 3 * I + c];
                gg[i * I + c] = draw[f * 3 * I + I + c];
                gu[i * I + c] = draw[f * 3 * I + 2 * I + c];
            }
        }
        quant_cols(gx, nr, d);
        quant_cols(gy, nr, d);
        quant_cols(gh, nr, I);
        quant_cols(gg, nr, I);
        quant_cols(gu, nr, I);
        for (int i = 0; i < nr; ++i) {
            for (int64_t c = 0; c < I; ++c) {
                const double cg = gg[i * I + c], cu = gu[i * I + c];
                for (int64_t m = 0; m < d; ++m) {
                    gw[c * d + m] += cg * gx[i * d + m];
                    uw[c * d + m] += cu * gx[i * d + m];
                }
            }
            for (int64_t m = 0; m < d; ++m)
                for (int64_t c = 0; c < I; ++c) dw[m * I + c] += gy[i * d + m] * gh[i * I + c];
        }
    }
    free(gx);
    free(gy);
    free(gg);
    free(gu);
    free(gh);
}

void oracle_backward(const or_shape *sh, const void *x, const float *wr, const int32_t *idx,
                     const or_ffn *experts, const or_ffn *shared, const float *dy, float *dx,
                     float *dwr, float *dwg, float *dwu, float *dwd, float *dsg, float *dsu, float *dsd,
                     float *dg_out, int32_t wsel) {
    const int64_t T = sh->T, d = sh->d, I = sh->I, E = sh->E, k = sh->k;
    const int fp8 = sh->wt == OR_E4M3;
    /* per (t, j) and per token intermediates for the weight gradients */
    double *ry = (double *)malloc(sizeof(double) * T * k * d);  /* routed output gradient */
    double *rh = (double *)malloc(sizeof(double) * T * k * I);
    double *rug = (double *)malloc(sizeof(double) * T * k * I);
    double *ruu = (double *)malloc(sizeof(double) * T * k * I);
    double *sy = (double *)malloc(sizeof(double) * T * d);      /* shared output gradient */
    double *sh_h = (double *)malloc(sizeof(double) * T * I);
    double *sug = (double *)malloc(sizeof(double) * T * I);
    double *suu = (double *)malloc(sizeof(double) * T * I);
    double *dl = (double *)malloc(sizeof(double) * T * k);
    double *xa = (double *)malloc(sizeof(double) * T * d);      /* x as the GEMMs read it */
    /* e4m3: unrounded values for the weight-gradient tiles */
    double *ryr = fp8 ? (double *)malloc(sizeof(double) * T * k * d) : NULL;
    double *rraw = fp8 ? (double *)malloc(sizeof(double) * T * k * 3 * I) : NULL;
    double *syr = fp8 ? (double *)malloc(sizeof(double) * T * d) : NULL;
    double *sraw = fp8 ? (double *)malloc(sizeof(double) * T * 3 * I) : NULL;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < T; ++t) {
        double *a = xa + t * d;
        double *yr = (double *)malloc(sizeof(double) * d);
        double *da = (double *)malloc(sizeof(double) * d);
        double *acc = (double *)malloc(sizeof(double) * d);
        double *hb = (double *)malloc(sizeof(double) * I);
        double s[64], dgv[64];
        gemm_input_row(sh, x, t, a);
        for (int64_t n = 0; n < d; ++n) acc[n] = 0.0;
        /* routed experts */
        double ssum = 0.0;
        for (int64_t j = 0; j < k; ++j) {
            const int e = idx[t * k + j];
            double l = 0.0;
            for (int64_t n = 0; n < d; ++n) l += x_at(sh, x, t, n) * (double)wr[(int64_t)e * d + n];
            s[j] = 1.0 / (1.0 + exp(-l));
            ssum += s[j];
        }
        for (int64_t j = 0; j < k; ++j) {
            const int e = idx[t * k + j];
            const int64_t f = t * k + j;
            const double gj = s[j] / ssum;
            ffn_row(sh, experts, e, a, yr, hb);
            double dgj = 0.0;
            for (int64_t n = 0; n < d; ++n) dgj += (double)dy[t * d + n] * round_yperm(sh, yr[n]);
            dgv[j] = dgj;
            double *dyr = ry + f * d;
            for (int64_t n = 0; n < d; ++n) dyr[n] = gj * (double)dy[t * d + n];
            if (fp8)
                for (int64_t n = 0; n < d; ++n) ryr[f * d + n] = dyr[n];
            round_to_gemm_input(sh->wt, dyr, (int)d);
            ffn_row_backward(sh, experts, e, a, dyr, rh + f * I, rug + f * I, ruu + f * I, da,
                             fp8 ? rraw + f * 3 * I : NULL);
            for (int64_t n = 0; n < d; ++n) acc[n] += da[n];
        }
        /* shared expert */
        double *dys = sy + t * d;
        for (int64_t n = 0; n < d; ++n) dys[n] = (double)dy[t * d + n];
        if (fp8)
            for (int64_t n = 0; n < d; ++n) syr[t * d + n] = dys[n];
        round_to_gemm_input(sh->wt, dys, (int)d);
        ffn_row_backward(sh, shared, 0, a, dys, sh_h + t * I, sug + t * I, suu + t * I, da,
                         fp8 ? sraw + t * 3 * I : NULL);
        for (int64_t n = 0; n < d; ++n) acc[n] += da[n];
        /* router: through the renormalised weights only */
        double gdg = 0.0;
        for (int64_t j = 0; j < k; ++j) gdg += s[j] / ssum * dgv[j];
        for (int64_t j = 0; j < k; ++j) {
            const double ds = (dgv[j] - gdg) / ssum;
            dl[t * k + j] = ds * s[j] * (1.0 - s[j]);
            const int e = idx[t * k + j];
            for (int64_t n = 0; n < d; ++n) acc[n] += dl[t * k + j] * (double)wr[(int64_t)e * d + n];
            dg_out[t * k + j] = (float)dgv[j];
        }
        for (int64_t n = 0; n < d; ++n) dx[t * d + n] = (float)acc[n];
        free(yr);
        free(da);
        free(acc);
        free(hb);
    }
    /* weight gradients: routed experts and router, one expert at a time */
    const int64_t e_lo = wsel >= 0 ? wsel : 0, e_hi = wsel >= 0 ? wsel + 1 : (wsel == -1 ? E : 0);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t e = e_lo; e < e_hi; ++e) {
        const int64_t eo = e - e_lo;  /* output slot */
        double *gw = (double *)calloc((size_t)(I * d), sizeof(double));
        double *uw = (double *)calloc((size_t)(I * d), sizeof(double));
        double *dw = (double *)calloc((size_t)(d * I), sizeof(double));
        double *rw = (double *)calloc((size_t)d, sizeof(double));
        int64_t *rows = (int64_t *)malloc(sizeof(int64_t) * (size_t)(T * k));
        int64_t n_e = 0;
        for (int64_t f = 0; f < T * k; ++f)
            if (idx[f] == e) rows[n_e++] = f;
        if (fp8) {
            wgrad_e4m3(sh, x, rows, n_e, k, rraw, ryr, gw, uw, dw);
        } else {
            for (int64_t q = 0; q < n_e; ++q) {
                const int64_t f = rows[q];
                const double *a = xa + (f / k) * d;
                for (int64_t i = 0; i < I; ++i) {
                    const double cg = rug[f * I + i], cu = ruu[f * I + i];
                    for (int64_t n = 0; n < d; ++n) {
                        gw[i * d + n] += cg * a[n];
                        uw[i * d + n] += cu * a[n];
                    }
                }
                for (int64_t n = 0; n < d; ++n)
                    for (int64_t i = 0; i < I; ++i) dw[n * I + i] += ry[f * d + n] * rh[f * I + i];
            }
        }
        for (int64_t q = 0; q < n_e; ++q) {
            const int64_t f = rows[q];
            for (int64_t n = 0; n < d; ++n) rw[n] += dl[f] * x_at(sh, x, f / k, n);
        }
        for (int64_t q = 0; q < I * d; ++q) {
            dwg[eo * I * d + q] = (float)gw[q];
            dwu[eo * I * d + q] = (float)uw[q];
            dwd[eo * d * I + q] = (float)dw[q];
        }
        for (int64_t n = 0; n < d; ++n) dwr[eo * d + n] = (float)rw[n];
        free(gw);
        free(uw);
        free(dw);
        free(rw);
        free(rows);
    }
    /* the shared expert's weight gradients: over all tokens */
    if (wsel == -1 && fp8) {
        /* groups of 128 tokens; the groups are independent partial sums,
         * added in group order */
        const int64_t ng = (T + 127) / 128;
        double *gw = (double *)calloc((size_t)(ng * I * d), sizeof(double));
        double *uw = (double *)calloc((size_t)(ng * I * d), sizeof(double));
        double *dw = (double *)calloc((size_t)(ng * d * I), sizeof(double));
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t gi = 0; gi < ng; ++gi) {
            int64_t rows[128];
            const int64_t n = T - gi * 128 < 128 ? T - gi * 128 : 128;
            for (int64_t i = 0; i < n; ++i) rows[i] = gi * 128 + i;
            wgrad_e4m3(sh, x, rows, n, 1, sraw, syr, gw + gi * I * d, uw + gi * I * d, dw + gi * d * I);
        }
        for (int64_t q = 0; q < I * d; ++q) {
            double a = 0.0, b = 0.0, c = 0.0;
            for (int64_t gi = 0; gi < ng; ++gi) {
                a += gw[gi * I * d + q];
                b += uw[gi * I * d + q];
                c += dw[gi * d * I + q];
            }
            dsg[q] = (float)a;
            dsu[q] = (float)b;
            dsd[q] = (float)c;
        }
        free(gw);
        free(uw);
        free(dw);
    } else if (wsel == -1) {
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < I; ++i)
            for (int64_t n = 0; n < d; ++n) {
                double cg = 0.0, cu = 0.0;
                for (int64_t t = 0; t < T; ++t) {
                    cg += sug[t * I + i] * xa[t * d + n];
                    cu += suu[t * I + i] * xa[t * d + n];
                }
                dsg[i * d + n] = (float)cg;
                dsu[i * d + n] = (float)cu;
            }
#pragma omp parallel for schedule(static)
        for (int64_t n = 0; n < d; ++n)
            for (int64_t i = 0; i < I; ++i) {
                double c = 0.0;
                for (int64_t t = 0; t < T; ++t) c += sy[t * d + n] * sh_h[t * I + i];
                dsd[n * I + i] = (float)c;
            }
    }
    free(ry);
    free(rh);
    free(rug);
    free(ruu);
    free(sy);
    free(sh_h);
    free(sug);
    free(suu);
    free(dl);
    free(xa);
    free(ryr);
    free(rraw);
    free(syr);
    free(sraw);
}

/* The shared expert's weight gradients restricted to columns cols[0..nc) of
 * its SwiGLU width: dsg, dsu [nc, d] hold rows cols[c] of oracle_backward's
 * [I, d] dsg, dsu and dsd [d, nc] columns cols[c] of its [d, I] dsd, over all
 * T tokens, with the same arithmetic in the same order.  (Column i of these
 * gradients needs only column i of the shared expert's hidden layer: its
 * gate and up rows, its down column, the whole output gradient and x; with
 * e4m3 weights every weight-gradient operand is quantised per column of a
 * 128-token group, so the restriction changes no tile.)  This is the same
 * computation as the shared part of oracle_backward, cut to a few columns so
 * that it finishes in seconds at the full layer size. */
void oracle_backward_shared_cols(const or_shape *sh, const void *x, const or_ffn *shared, const float *dy,
                                 int32_t nc, const int32_t *cols, float *dsg, float *dsu, float *dsd) {
    const int64_t T = sh->T, d = sh->d, I = sh->I;
    const int fp8 = sh->wt == OR_E4M3;
    double *xa = (double *)malloc(sizeof(double) * T * d);   /* x as the GEMMs read it */
    double *dyw = (double *)malloc(sizeof(double) * T * d);  /* weight-gradient operand: dy rounded (raw for e4m3) */
    double *hc = (double *)malloc(sizeof(double) * T * nc); /* h, dug, duu of the chosen columns */
    double *gc = (double *)malloc(sizeof(double) * T * nc);
    double *uc = (double *)malloc(sizeof(double) * T * nc);
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t t = 0; t < T; ++t) {
        double *a = xa + t * d;
        double *r = (double *)malloc(sizeof(double) * d);
        gemm_input_row(sh, x, t, a);
        for (int64_t n = 0; n < d; ++n) r[n] = (double)dy[t * d + n];
        for (int64_t n = 0; n < d; ++n) dyw[t * d + n] = r[n];
        round_to_gemm_input(sh->wt, r, (int)d);  /* the data-gradient operand */
        if (!fp8)
            for (int64_t n = 0; n < d; ++n) dyw[t * d + n] = r[n];
        for (int32_t c = 0; c < nc; ++c) {
            const int64_t i = cols[c];
            double ug = 0.0, uu = 0.0, dh = 0.0;
            for (int64_t j = 0; j < d; ++j) {
                ug += w_at(sh->wt, shared->gate, shared->s_gate, I, d, 0, i, j) * a[j];
                uu += w_at(sh->wt, shared->up, shared->s_up, I, d, 0, i, j) * a[j];
            }
            const double sg = 1.0 / (1.0 + exp(-ug));
            for (int64_t n = 0; n < d; ++n) dh += w_at(sh->wt, shared->down, shared->s_down, d, I, 0, n, i) * r[n];
            double v[3] = {ug * sg * uu, dh * uu * sg * (1.0 + ug * (1.0 - sg)), dh * ug * sg};
            if (!fp8)  /* fp32 and bf16 round each value on its own */
                for (int q = 0; q < 3; ++q) round_to_gemm_input(sh->wt, v + q, 1);
            hc[t * nc + c] = v[0];
            gc[t * nc + c] = v[1];
            uc[t * nc + c] = v[2];
        }
        free(r);
    }
    if (fp8) {
        const int64_t ng = (T + 127) / 128;
        double *gw = (double *)calloc((size_t)(ng * nc * d), sizeof(double));
        double *uw = (double *)calloc((size_t)(ng * nc * d), sizeof(double));
        double *dw = (double *)calloc((size_t)(ng * d * nc), sizeof(double));
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t gi = 0; gi < ng; ++gi) {
            const int nr = (int)(T - gi * 128 < 128 ? T - gi * 128 : 128);
            double *gx = (double *)malloc(sizeof(double) * 128 * d);
            double *gy = (double *)malloc(sizeof(double) * 128 * d);
            double *gh = (double *)malloc(sizeof(double) * 128 * nc);
            double *gg = (double *)malloc(sizeof(double) * 128 * nc);
            double *gu = (double *)malloc(sizeof(double) * 128 * nc);
            for (int i = 0; i < nr; ++i) {
                const int64_t t = gi * 128 + i;
                for (int64_t m = 0; m < d; ++m) {
                    gx[i * d + m] = x_at(sh, x, t, m);
                    gy[i * d + m] = dyw[t * d + m];
                }
                for (int32_t c = 0; c < nc; ++c) {
                    gh[i * nc + c] = hc[t * nc + c];
                    gg[i * nc + c] = gc[t * nc + c];
                    gu[i * nc + c] = uc[t * nc + c];
                }
            }
            quant_cols(gx, nr, d);
            quant_cols(gy, nr, d);
            quant_cols(gh, nr, nc);
            quant_cols(gg, nr, nc);
            quant_cols(gu, nr, nc);
            double *pg = gw + gi * nc * d, *pu = uw + gi * nc * d, *pd = dw + gi * d * nc;
            for (int i = 0; i < nr; ++i) {
                for (int32_t c = 0; c < nc; ++c)
                    for (int64_t m = 0; m < d; ++m) {
                        pg[c * d + m] += gg[i * nc + c] * gx[i * d + m];
                        pu[c * d + m] += gu[i * nc + c] * gx[i * d + m];
                    }
                for (int64_t m = 0; m < d; ++m)
                    for (int32_t c = 0; c < nc; ++c) pd[m * nc + c] += gy[i * d + m] * gh[i * nc + c];
            }
            free(gx);
            free(gy);
            free(gh);
            free(gg);
            free(gu);
        }
        for (int64_t q = 0; q < nc * d; ++q) {
            double a = 0.0, b = 0.0, c = 0.0;
            for (int64_t gi = 0; gi < ng; ++gi) {
                a += gw[gi * nc * d + q];
                b += uw[gi * nc * d + q];
                c += dw[gi * d * nc + q];
            }
            dsg[q] = (float)a;
            dsu[q] = (float)b;
            dsd[q] = (float)c;
        }
        free(gw);
        free(uw);
        free(dw);
    } else {
#pragma omp parallel for schedule(static)
        for (int64_t n = 0; n < d; ++n) {
            for (int32_t c = 0; c < nc; ++c) {
                double cg = 0.0, cu = 0.0, cd = 0.0;
                for (int64_t t = 0; t < T; ++t) {
                    cg += gc[t * nc + c] * xa[t * d + n];
                    cu += uc[t * nc + c] * xa[t * d + n];
                    cd += dyw[t * d + n] * hc[t * nc + c];
                }
                dsg[c * d + n] = (float)cg;
                dsu[c * d + n] = (float)cu;
                dsd[n * nc + c] = (float)cd;
            }
        }
    }
    free(xa);
    free(dyw);
    free(hc);
    free(gc);
    free(uc);
}

/* Threads later OpenMP regions of this library use (from the calling thread). */
void oracle_set_threads(int32_t n) { omp_set_num_threads(n > 0 ? n : 1); }

/* Threads an OpenMP region of this library uses (for reporting). */
int oracle_num_threads(void) {
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        n = omp_get_num_threads();
    }
    return n;
}
