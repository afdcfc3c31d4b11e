/*
 * Seeded synthetic inputs for the MoE layer: the one module that both the
 * CPU oracle (tests) and the HIP path (tests, bench) take their inputs from.
 *
 * It holds none of the layer's arithmetic.  It only draws numbers and puts
 * them into the storage format a tensor is kept in:
 *   - normals N(0, std) and uniforms U(lo, hi), element by element from a
 *     counter-based generator, so every value depends only on
 *     (seed, tensor id, element index) and never on the thread count;
 *   - rounding of those draws to fp32, bf16, or OCP fp8 e4m3 with one fp32
 *     scale per 128x128 block (the offline weight preparation that an fp8
 *     deployment does once, before any forward pass);
 *   - a per-row power-law factor (Zipf skew) for a router matrix;
 *   - random sets of k distinct ids per token, used to feed the dispatch
 *     stage on its own.
 *
 * Generator: Philox4x64-10 from Salmon, Moraes, Dror and Shaw, "Parallel
 * random numbers: as easy as 1, 2, 3" (SC 2011).  Key = (seed, tensor id),
 * counter = (element index / 4, 0, 0, 0); one call gives four 64-bit words.
 * Normals: Box-Muller on pairs of 53-bit uniforms, in double precision, for
 * fp32 tensors; an inverse-transform table for bf16 and e4m3 tensors (below).
 *
 * Build: gcc -O3 -fopenmp -shared -fPIC gen.c -o libsynth.so -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define SYNTH_F32 0
#define SYNTH_BF16 1

/* Philox4x64 round constants as published (multipliers and Weyl increments). */
#define PH_M0 0xD2E7470EE14C6C93ULL
#define PH_M1 0xCA5A826395121157ULL
#define PH_W0 0x9E3779B97F4A7C15ULL
#define PH_W1 0xBB67AE8584CAA73BULL

static inline void mulhilo64(uint64_t a, uint64_t b, uint64_t *hi, uint64_t *lo) {
    __uint128_t p = (__uint128_t)a * (__uint128_t)b;
    *hi = (uint64_t)(p >> 64);
    *lo = (uint64_t)p;
}

static inline void philox4x64_10(const uint64_t in[4], const uint64_t key_in[2], uint64_t out[4]) {
    uint64_t c0 = in[0], c1 = in[1], c2 = in[2], c3 = in[3];
    uint64_t k0 = key_in[0], k1 = key_in[1];
    for (int r = 0; r < 10; ++r) {
        if (r > 0) { k0 += PH_W0; k1 += PH_W1; }
        uint64_t hi0, lo0, hi1, lo1;
        mulhilo64(PH_M0, c0, &hi0, &lo0);
        mulhilo64(PH_M1, c2, &hi1, &lo1);
        uint64_t n0 = hi1 ^ c1 ^ k0;
        uint64_t n2 = hi0 ^ c3 ^ k1;
        c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* Exported for the known-answer test against numpy's Philox bit generator. */
void synth_philox4x64_10(const uint64_t ctr[4], const uint64_t key[2], uint64_t out[4]) {
    philox4x64_10(ctr, key, out);
}

static inline void draw4(uint64_t seed, uint32_t tensor, uint64_t block, uint64_t w[4]) {
    uint64_t ctr[4] = {block, 0, 0, 0};
    uint64_t key[2] = {seed, (uint64_t)tensor};
    philox4x64_10(ctr, key, w);
}

/* 53-bit uniform in (0, 1] and [0, 1). */
static inline double u01_open0(uint64_t w) { return ((double)(w >> 11) + 1.0) * 0x1.0p-53; }
static inline double u01(uint64_t w) { return (double)(w >> 11) * 0x1.0p-53; }

/* Four standard normals from one Philox block (two Box-Muller pairs). */
static inline void normals4(uint64_t seed, uint32_t tensor, uint64_t block, double z[4]) {
    uint64_t w[4];
    draw4(seed, tensor, block, w);
    const double two_pi = 6.283185307179586476925286766559;
    for (int p = 0; p < 2; ++p) {
        double r = sqrt(-2.0 * log(u01_open0(w[2 * p])));
        double th = two_pi * u01(w[2 * p + 1]);
        z[2 * p] = r * cos(th);
        z[2 * p + 1] = r * sin(th);
    }
}

static inline double normal_at(uint64_t seed, uint32_t tensor, uint64_t n) {
    double z[4];
    normals4(seed, tensor, n >> 2, z);
    return z[n & 3];
}

/*
 * Tensors stored in bf16 (and the bf16 values that e4m3 weights are quantised
 * from) are drawn by inverse transform: a 20-bit uniform bin i maps to
 * z_i = Phi^-1((i + 0.5) / 2^20), the standard normal quantile at the bin
 * midpoint (|z| <= 4.9).  One Philox call gives 12 such draws (three 20-bit
 * fields per 64-bit word).  At bf16 resolution (8 significant bits) this is
 * indistinguishable from an exact normal draw except beyond 4.9 sigma.
 * The table is computed once by Newton iteration on Phi(z) = erfc(-z/sqrt2)/2.
 */
#define QBITS 20
#define QN (1u << QBITS)
static double *qtable;

static double phi_cdf(double z) { return 0.5 * erfc(-z * 0.70710678118654752440); }

static void build_qtable(void) {
    if (qtable) return;
    double *t = (double *)malloc(sizeof(double) * QN);
    const double inv_sqrt_2pi = 0.39894228040143267794;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < (int64_t)QN; ++i) {
        double p = ((double)i + 0.5) / (double)QN;
        /* Newton on Phi(z) = p, kept inside a shrinking bracket (bisection
         * whenever a Newton step would leave it). */
        double lo = -12.0, hi = 12.0, z = 0.0;
        for (int it = 0; it < 200; ++it) {
            double f = phi_cdf(z) - p;
            if (f < 0.0) lo = z; else hi = z;
            double dens = inv_sqrt_2pi * exp(-0.5 * z * z);
            double zn = dens > 0.0 ? z - f / dens : 0.5 * (lo + hi);
            if (!(zn > lo && zn < hi)) zn = 0.5 * (lo + hi);
            if (fabs(zn - z) < 1e-15 * (1.0 + fabs(z))) { z = zn; break; }
            z = zn;
        }
        t[i] = z;
    }
    qtable = t;
}

/* bf16 = upper half of binary32, round to nearest even (finite inputs). */
static inline uint16_t bf16_bits_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

static inline float bf16_value(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* bf16 bits of fl32(std * z_i) for every quantile bin (2 MB, caller frees). */
static uint16_t *bf16_quantile_table(double std) {
    build_qtable();
    uint16_t *t = (uint16_t *)malloc(sizeof(uint16_t) * QN);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < (int64_t)QN; ++i) t[i] = bf16_bits_rne((float)(std * qtable[i]));
    return t;
}

static inline uint32_t qbin(const uint64_t w[4], unsigned slot) {
    return (uint32_t)((w[slot / 3] >> (20 * (slot % 3))) & (QN - 1));
}

/* OCP fp8 E4M3FN encode of a finite float, round to nearest even,
 * saturating to +-448 (bias 7, no infinities, S.1111.111 is NaN). */
static uint8_t e4m3_encode_sat(float v) {
    uint32_t u;
    memcpy(&u, &v, 4);
    uint8_t sign = (uint8_t)((u >> 24) & 0x80u);
    float a = fabsf(v);
    if (!(a < 464.0f)) return sign | 0x7E;          /* >= 464 (or NaN) -> 448 */
    if (a < 0x1.0p-6f) {                             /* subnormal: multiples of 2^-9 */
        float q = rintf(a * 512.0f);                 /* exact scaling, RNE */
        return sign | (uint8_t)q;                    /* q == 8 is the smallest normal */
    }
    memcpy(&u, &a, 4);
    int e = (int)(u >> 23) - 127;                    /* -6 .. 8 */
    uint32_t m = u & 0x7FFFFFu;
    uint32_t keep = m >> 20, rem = m & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (keep & 1u))) keep++;
    if (keep == 8) { keep = 0; e++; }
    if (e > 8 || (e == 8 && keep > 6)) return sign | 0x7E;
    return sign | (uint8_t)(((e + 7) << 3) | keep);
}

void synth_e4m3_encode(int64_t n, const float *in, uint8_t *out) {
    for (int64_t i = 0; i < n; ++i) out[i] = e4m3_encode_sat(in[i]);
}

/* out[i] = round_dtype(std * N(0,1)), i in [0, n).
 * dtype 0: f32 via Box-Muller; dtype 1: bf16 bits via the quantile table. */
void synth_normal(uint64_t seed, uint32_t tensor, int64_t n, double std, int dtype, void *out) {
    if (dtype == SYNTH_BF16) {
        uint16_t *tbl = bf16_quantile_table(std);
        int64_t nblk = (n + 11) / 12;
        uint16_t *o = (uint16_t *)out;
#pragma omp parallel for schedule(static)
        for (int64_t b = 0; b < nblk; ++b) {
            uint64_t w[4];
            draw4(seed, tensor, (uint64_t)b, w);
            for (unsigned l = 0; l < 12; ++l) {
                int64_t i = b * 12 + l;
                if (i >= n) break;
                o[i] = tbl[qbin(w, l)];
            }
        }
        free(tbl);
        return;
    }
    int64_t nblk = (n + 3) / 4;
    float *o = (float *)out;
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < nblk; ++b) {
        double z[4];
        normals4(seed, tensor, (uint64_t)b, z);
        for (int l = 0; l < 4; ++l) {
            int64_t i = b * 4 + l;
            if (i >= n) break;
            o[i] = (float)(std * z[l]);
        }
    }
}

/* Router matrix with a power-law skew: out[r, c] = fl32(std * N(0,1) * (r+1)^-s). */
void synth_normal_rowpow(uint64_t seed, uint32_t tensor, int64_t rows, int64_t cols, double std,
                         double s, float *out) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double f = pow((double)(r + 1), -s);
        for (int64_t c = 0; c < cols; ++c)
            out[r * cols + c] = (float)(std * normal_at(seed, tensor, (uint64_t)(r * cols + c)) * f);
    }
}

/* out[i] = fl32(lo + (hi - lo) * U[0,1)). */
void synth_uniform(uint64_t seed, uint32_t tensor, int64_t n, double lo, double hi, float *out) {
    int64_t nblk = (n + 3) / 4;
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < nblk; ++b) {
        uint64_t w[4];
        draw4(seed, tensor, (uint64_t)b, w);
        for (int l = 0; l < 4; ++l) {
            int64_t i = b * 4 + l;
            if (i >= n) break;
            out[i] = (float)(lo + (hi - lo) * u01(w[l]));
        }
    }
}

/*
 * fp8 weight preparation for a stack of G matrices [R, C] (R, C multiples of
 * 128): the same bf16 values synth_normal gives for this seed and tensor
 * (element index (g*R + r)*C + c), then per 128x128 block: amax = max |v|, scale = the smallest
 * power of two at or above amax / 448 (the fp32 quotient; 1 when amax = 0), q = e4m3(v / scale).
 * q: [G, R, C] codes; scales: [G, R/128, C/128] as OCP MX E8M0 bytes (the
 * biased exponent of the power of two: byte e stands for 2^(e-127)).
 */
void synth_normal_e4m3_blocks(uint64_t seed, uint32_t tensor, int64_t G, int64_t R, int64_t C,
                              double std, uint8_t *q, uint8_t *scales) {
    uint16_t *tbl = bf16_quantile_table(std);
    int64_t RB = R / 128, CB = C / 128;
    int64_t nb = G * RB * CB;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t blk = 0; blk < nb; ++blk) {
        int64_t g = blk / (RB * CB), rb = (blk / CB) % RB, cb = blk % CB;
        float v[128 * 128];
        float amax = 0.0f;
        for (int r = 0; r < 128; ++r) {
            uint64_t base = (uint64_t)((g * R + rb * 128 + r) * C + cb * 128);
            uint64_t b0 = base / 12, b1 = (base + 127) / 12;
            uint64_t w[12][4];
            for (uint64_t b = b0; b <= b1; ++b) draw4(seed, tensor, b, w[b - b0]);
            for (int c = 0; c < 128; ++c) {
                uint64_t n = base + (uint64_t)c;
                float f = bf16_value(tbl[qbin(w[n / 12 - b0], (unsigned)(n % 12))]);
                v[r * 128 + c] = f;
                float a = fabsf(f);
                if (a > amax) amax = a;
            }
        }
        float s = 1.0f;
        if (amax > 0.0f) {
            float t = amax / 448.0f;
            uint32_t b;
            memcpy(&b, &t, 4);
            if (b & 0x7FFFFFu) b = (b & 0xFF800000u) + 0x800000u; /* next power of two */
            memcpy(&s, &b, 4);
        }
        {
            uint32_t sb;
            memcpy(&sb, &s, 4);
            scales[blk] = (uint8_t)(sb >> 23); /* s is a positive normal power of two */
        }
        for (int r = 0; r < 128; ++r) {
            uint8_t *dst = q + (g * R + rb * 128 + r) * C + cb * 128;
            for (int c = 0; c < 128; ++c) dst[c] = e4m3_encode_sat(v[r * 128 + c] / s);
        }
    }
    free(tbl);
}

/* k distinct ids in [0, E) per token, ascending: a partial Fisher-Yates shuffle
 * driven by one Philox stream per token (counter = token * 64 + draw / 4). */
void synth_random_ids(uint64_t seed, uint32_t tensor, int64_t T, int E, int k, int32_t *idx) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        int32_t perm[1024];
        for (int i = 0; i < E; ++i) perm[i] = i;
        uint64_t w[4];
        for (int j = 0; j < k; ++j) {
            if ((j & 3) == 0) draw4(seed, tensor, (uint64_t)t * 64u + (uint64_t)(j >> 2), w);
            uint64_t span = (uint64_t)(E - j);
            int pick = j + (int)(((w[j & 3] >> 11) * span) >> 53);
            int32_t tmp = perm[j]; perm[j] = perm[pick]; perm[pick] = tmp;
        }
        /* insertion sort of the k picks */
        for (int a = 1; a < k; ++a) {
            int32_t v = perm[a]; int b = a - 1;
            while (b >= 0 && perm[b] > v) { perm[b + 1] = perm[b]; --b; }
            perm[b + 1] = v;
        }
        for (int j = 0; j < k; ++j) idx[t * k + j] = perm[j];
    }
}
