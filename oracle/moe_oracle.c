/*
 * moe_oracle.c -- plain CPU oracle of the routed-experts decode step of a
 * bit-quantized mixture-of-experts layer.
 *
 * TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and bench.py's
 * cpu_baseline leg may load, call or link this library. The GPU library never
 * does, and shares no code, header, table or helper with it.
 *
 * What is computed (the plain definition, written out, in fp64):
 *   route    top-k experts per token by raw logit (ties: lower expert id),
 *            weights = softmax over the k selected logits;
 *   bucket   per-expert row lists, experts ascending, rows ascending by token;
 *   rotate   x~ = R_H x with R = (1/sqrt(128)) blockdiag(H_128 diag(s)),
 *            H_128[i][j] = (-1)^popcount(i & j) (codebook format only);
 *   expert   g = Wg x~, u = Wu x~, h = silu(g) * u, h~ = R_I h, y = Wd h~;
 *   combine  out[t] = sum_j w[t][j] * y[t][j], slot order.
 * Sources: the routed-experts decode kernel "lna2" of page "LNA-CANON.md",
 * section "lna2 とは" (top-k routed rows per expert, R_e in {1,2,4,8} at
 * m <= 24, bitwise reproducible combine) and page "lna-lab/README.md",
 * section "2026-09-04 -- house kernel lna2" (small-R inner loops, rows per
 * expert 1-8). The pages name the EXL3 trellis code ("What is in the pack":
 * EXL3 2/3 bit mixed) but never define it; this oracle follows the stand-in
 * codebook format whose stored layout is defined at orc_codebook_code().
 * The NVFP4 format follows page "V100 換引擎", section 4.0 (NVFP4 for the
 * MLP weights) and 7.1 (e2m1 values expand to fp16).
 *
 * Readings where the pages are silent (router math, SwiGLU expert, which
 * inputs are rotated, Hadamard order/normalisation) are listed with the
 * design notes of this repository.
 *
 * Precision: every stored value is decoded exactly into a double; products
 * of a codebook entry and a group scale (fp16 x fp16) and of e2m1 x e4m3 x
 * fp32 are exact in double; all sums are accumulated in double.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_FMT_CODEBOOK 1
#define ORC_FMT_NVFP4 2

/* ------------------------------------------------------------------ */
/* Scalar number formats                                               */
/* ------------------------------------------------------------------ */

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 mantissa bits. */
double orc_f16_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int ex = (h >> 10) & 0x1F;
    int man = h & 0x3FF;
    double v;
    if (ex == 0)
        v = ldexp((double)man, -24); /* subnormal: man * 2^-24 */
    else if (ex == 31)
        v = man ? NAN : INFINITY;
    else
        v = ldexp(1.0 + man / 1024.0, ex - 15);
    return sign ? -v : v;
}

/* bfloat16 is the upper half of an IEEE binary32. */
double orc_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* OCP e2m1 (fp4): 1 sign, 2 exponent (bias 1), 1 mantissa; no inf/nan. */
double orc_e2m1_to_double(uint8_t nib)
{
    int sign = (nib >> 3) & 1;
    int ex = (nib >> 1) & 3;
    int man = nib & 1;
    double v = ex == 0 ? 0.5 * man : ldexp(1.0 + 0.5 * man, ex - 1);
    return sign ? -v : v;
}

/* OCP e4m3fn: 1 sign, 4 exponent (bias 7), 3 mantissa; S.1111.111 is NaN,
 * no infinities. */
double orc_e4m3fn_to_double(uint8_t b)
{
    int sign = (b >> 7) & 1;
    int ex = (b >> 3) & 0xF;
    int man = b & 7;
    double v;
    if (ex == 15 && man == 7)
        return NAN;
    if (ex == 0)
        v = ldexp(man / 8.0, -6);
    else
        v = ldexp(1.0 + man / 8.0, ex - 7);
    return sign ? -v : v;
}

/* ------------------------------------------------------------------ */
/* Block Hadamard rotation                                             */
/* ------------------------------------------------------------------ */

/* In place v <- H_128 v, H_128[i][j] = (-1)^popcount(i & j) (Sylvester,
 * natural order), by the standard fast Walsh-Hadamard butterflies. */
void orc_fwht128(double *v)
{
    for (int h = 1; h < 128; h <<= 1)
        for (int i = 0; i < 128; i += 2 * h)
            for (int j = i; j < i + h; ++j) {
                double a = v[j], b = v[j + h];
                v[j] = a + b;
                v[j + h] = a - b;
            }
}

/* out = R in, R = (1/sqrt(128)) blockdiag over 128-blocks of H_128 diag(s).
 * n must be a multiple of 128. */
void orc_rotate(int n, const int8_t *signs, const double *in, double *out)
{
    const double norm = 1.0 / sqrt(128.0);
    for (int b = 0; b < n; b += 128) {
        double t[128];
        for (int i = 0; i < 128; ++i)
            t[i] = (double)signs[b + i] * in[b + i];
        orc_fwht128(t);
        for (int i = 0; i < 128; ++i)
            out[b + i] = t[i] * norm;
    }
}

/* The inverse: R^-1 = R^T = (1/sqrt(128)) blockdiag(diag(s) H_128). */
void orc_unrotate(int n, const int8_t *signs, const double *in, double *out)
{
    const double norm = 1.0 / sqrt(128.0);
    for (int b = 0; b < n; b += 128) {
        double t[128];
        for (int i = 0; i < 128; ++i)
            t[i] = in[b + i];
        orc_fwht128(t);
        for (int i = 0; i < 128; ++i)
            out[b + i] = (double)signs[b + i] * t[i] * norm;
    }
}

/* ------------------------------------------------------------------ */
/* Stored weight layouts                                               */
/* ------------------------------------------------------------------ */
/*
 * Both formats store a matrix W of N rows (outputs) x C columns (inputs),
 * N % 16 == 0, C % 128 == 0, as tiles of 16 rows x 128 columns.
 * Tile (rb, g) holds rows 16rb..16rb+15, columns 128g..128g+127; its index
 * is tau = rb * (C / 128) + g and tiles are stored in index order. A tile
 * has 64 slots; slot l covers row 16rb + (l mod 16) and the 32 columns
 * 128g + 32 (l div 16) + jj, jj = 0..31; slots are stored in order.
 */

/* Codebook, K = bits in {2,3,6}: each slot is K little-endian uint32 words
 * w0..w(K-1). Column jj (0..31) of the slot takes its code bits, least
 * significant first, from these (word, bit) positions:
 *   K = 3, jj < 24:  d = jj div 8, i = jj mod 8: word d, bits
 *                    8 (i mod 4) + 3 (i div 4) + {0, 1, 2};
 *   K = 3, 24..31:   i = jj - 24: bits 0 and 1 at word i div 4, bits
 *                    8 (i mod 4) + 6 + {0, 1}; bit 2 at word 2, bit 8 (i mod 4) + 6 + i div 4;
 *   K = 2:           d = jj div 16, kk = jj mod 16: word d, bits
 *                    8 (kk mod 4) + 2 (kk div 4) + {0, 1};
 *   K = 6:           the slot read as one 192-bit little-endian string:
 *                    bits 6 jj .. 6 jj + 5 (word q div 32, bit q mod 32 for
 *                    string bit q).
 * Every bit of the K words holds exactly one code bit.
 * Word d of slot l of tile tau lies at word tau*64*K + l*K + d, except for
 * K = 6, whose tiles hold words 0..2 of the 64 slots, then words 3..5:
 * tau*384 + (d div 3)*192 + l*3 + d mod 3. */
static void codebook_bit_positions(int bits, int jj, int word[6], int bit[6])
{
    int k;
    if (bits == 6) {
        for (k = 0; k < 6; ++k) {
            word[k] = (6 * jj + k) / 32;
            bit[k] = (6 * jj + k) % 32;
        }
        return;
    }
    if (bits == 3 && jj < 24) {
        int i = jj % 8;
        for (k = 0; k < 3; ++k) {
            word[k] = jj / 8;
            bit[k] = 8 * (i % 4) + 3 * (i / 4) + k;
        }
    } else if (bits == 3) {
        int i = jj - 24;
        for (k = 0; k < 2; ++k) {
            word[k] = i / 4;
            bit[k] = 8 * (i % 4) + 6 + k;
        }
        word[2] = 2;
        bit[2] = 8 * (i % 4) + 6 + i / 4;
    } else {
        int kk = jj % 16;
        for (k = 0; k < 2; ++k) {
            word[k] = jj / 16;
            bit[k] = 8 * (kk % 4) + 2 * (kk / 4) + k;
        }
    }
}

uint32_t orc_codebook_code(int bits, int N, int C, const uint32_t *codes, int n, int c)
{
    (void)N;
    int G = C / 128;
    int rb = n / 16, r = n % 16, g = c / 128, cc = c % 128;
    int q = cc / 32, jj = cc % 32;
    int slot = q * 16 + r;
    long tau = (long)rb * G + g;
    int word[6], bit[6], k;
    uint32_t code = 0;
    codebook_bit_positions(bits, jj, word, bit);
    for (k = 0; k < bits; ++k) {
        long at = bits == 6 ? tau * 384 + (word[k] / 3) * 192 + slot * 3 + word[k] % 3
                            : (tau * 64 + slot) * bits + word[k];
        code |= ((codes[at] >> bit[k]) & 1u) << k;
    }
    return code;
}

/* Group scales: fp16, one per (row, 128-column group), stored per 16 x 128
 * tile in the tiles' order: the 16 scales of tile (n / 16, c / 128) in row
 * order, i.e. scales[((n / 16) * (C / 128) + c / 128) * 16 + n % 16]. */
double orc_codebook_weight(int bits, int N, int C, const uint32_t *codes, const uint16_t *scales,
                           const uint16_t *lut, int n, int c)
{
    uint32_t code = orc_codebook_code(bits, N, C, codes, n, c);
    return orc_f16_to_double(lut[code]) *
           orc_f16_to_double(scales[((long)(n / 16) * (C / 128) + c / 128) * 16 + n % 16]);
}

/* NVFP4: each slot is 16 bytes; column jj of the slot is the nibble of byte
 * jj div 2, the low nibble for even jj (the lower column in the low nibble). */
uint8_t orc_nvfp4_code(int N, int C, const uint8_t *codes, int n, int c)
{
    (void)N;
    int G = C / 128;
    int rb = n / 16, r = n % 16, g = c / 128, cc = c % 128;
    int q = cc / 32, jj = cc % 32;
    long tau = (long)rb * G + g;
    uint8_t byte = codes[(tau * 64 + q * 16 + r) * 16 + jj / 2];
    return (jj % 2) ? (byte >> 4) : (byte & 0xF);
}

/* NVFP4 block scales: e4m3fn, one per (row, 16-column block), stored per
 * 16 x 128 tile in the tiles' order, each tile's 16 x 8 scales row-major:
 * scales[((n / 16) * (C / 128) + c / 128) * 128 + (n % 16) * 8 + (c % 128) / 16].
 * W = e2m1(code) * e4m3(scale) * tensor_scale. */
double orc_nvfp4_weight(int N, int C, const uint8_t *codes, const uint8_t *scales, float ts, int n,
                        int c)
{
    double s = orc_e4m3fn_to_double(
        scales[((long)(n / 16) * (C / 128) + c / 128) * 128 + (n % 16) * 8 + (c % 128) / 16]);
    return orc_e2m1_to_double(orc_nvfp4_code(N, C, codes, n, c)) * s * (double)ts;
}

/* ------------------------------------------------------------------ */
/* Router and buckets                                                  */
/* ------------------------------------------------------------------ */

/* Per token: the k experts with the largest raw logits, in selection order
 * (largest first; equal logits: lower expert id first). Weights: softmax over
 * the k selected logits, which equals the full softmax renormalised over the
 * selected set (the full denominator cancels). */
void orc_route(int m, int E, int k, const float *logits, int32_t *ids, double *w)
{
    char *taken = (char *)malloc((size_t)E);
    for (int t = 0; t < m; ++t) {
        const float *l = logits + (size_t)t * E;
        memset(taken, 0, (size_t)E);
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e])
                    continue;
                if (best < 0 || l[e] > l[best])
                    best = e; /* strict '>' keeps the lower id on ties */
            }
            taken[best] = 1;
            ids[t * k + j] = best;
        }
        double l0 = (double)l[ids[t * k]];
        double den = 0.0;
        for (int j = 0; j < k; ++j)
            den += exp((double)l[ids[t * k + j]] - l0);
        for (int j = 0; j < k; ++j)
            w[t * k + j] = exp((double)l[ids[t * k + j]] - l0) / den;
    }
    free(taken);
}

/* counts[e] = rows routed to expert e; offsets = exclusive prefix sum
 * (offsets[E] = m*k); the row list holds entries (t, j) grouped by expert
 * (ascending e) and, within an expert, ascending token t. pos[t*k+j] is the
 * position of entry (t, j) in the row list. */
void orc_bucket(int m, int E, int k, const int32_t *ids, int32_t *counts, int32_t *offsets,
                int32_t *rows_t, int32_t *rows_j, int32_t *pos)
{
    for (int e = 0; e < E; ++e)
        counts[e] = 0;
    for (int i = 0; i < m * k; ++i)
        counts[ids[i]]++;
    offsets[0] = 0;
    for (int e = 0; e < E; ++e)
        offsets[e + 1] = offsets[e] + counts[e];
    int p = 0;
    for (int e = 0; e < E; ++e)
        for (int t = 0; t < m; ++t)
            for (int j = 0; j < k; ++j)
                if (ids[t * k + j] == e) {
                    rows_t[p] = t;
                    rows_j[p] = j;
                    pos[t * k + j] = p;
                    ++p;
                }
}

/* ------------------------------------------------------------------ */
/* The layer                                                           */
/* ------------------------------------------------------------------ */

typedef struct {
    int32_t format; /* ORC_FMT_* */
    int32_t num_experts, top_k, hidden, inter;
    const int32_t *bits;      /* [E] */
    const void *const *codes; /* [E*3]: gate, up, down */
    const void *const *scales;/* [E*3] */
    const void *const *luts;  /* [E*3] fp16 codebooks (codebook format) */
    const float *tscales;     /* [E*3] tensor scales (NVFP4) */
    const int8_t *signs_hidden; /* [hidden] (codebook) */
    const int8_t *signs_inter;  /* [inter] (codebook) */
    int32_t has_shared;         /* 1: expert E is a shared expert (codebook format):
                                 * bits[E], tensors 3E..3E+2, same H and I */
} orc_layer;

static double weight_at(const orc_layer *L, int e, int p, int N, int C, int n, int c)
{
    int idx = e * 3 + p;
    if (L->format == ORC_FMT_CODEBOOK)
        return orc_codebook_weight(L->bits[e], N, C, (const uint32_t *)L->codes[idx],
                                   (const uint16_t *)L->scales[idx],
                                   (const uint16_t *)L->luts[idx], n, c);
    return orc_nvfp4_weight(N, C, (const uint8_t *)L->codes[idx], (const uint8_t *)L->scales[idx],
                            L->tscales[idx], n, c);
}

/* y = W v for projection p of expert e (N x C matrix), fp64 accumulation. */
static void gemv(const orc_layer *L, int e, int p, int N, int C, const double *v, double *y)
{
    for (int n = 0; n < N; ++n) {
        double acc = 0.0;
        for (int c = 0; c < C; ++c)
            acc += weight_at(L, e, p, N, C, n, c) * v[c];
        y[n] = acc;
    }
}

/* One routed expert applied to one token: y = Wd R_I (silu(Wg x~) * (Wu x~))
 * where x~ is the token's (rotated, for the codebook format) activation.
 * The SwiGLU expert shape (gate, up, SiLU(gate) * up, down) is the routed
 * expert of the DeepSeek MoE block served on the pages. */
void orc_expert(const orc_layer *L, int e, const double *xr, double *y)
{
    int H = L->hidden, I = L->inter;
    double *g = (double *)malloc(sizeof(double) * I);
    double *u = (double *)malloc(sizeof(double) * I);
    double *h = (double *)malloc(sizeof(double) * I);
    double *hr = (double *)malloc(sizeof(double) * I);
    gemv(L, e, 0, I, H, xr, g);
    gemv(L, e, 1, I, H, xr, u);
    for (int n = 0; n < I; ++n)
        h[n] = g[n] / (1.0 + exp(-g[n])) * u[n];
    if (L->format == ORC_FMT_CODEBOOK)
        orc_rotate(I, L->signs_inter, h, hr);
    else
        memcpy(hr, h, sizeof(double) * I);
    gemv(L, e, 2, H, I, hr, y);
    free(g);
    free(u);
    free(h);
    free(hr);
}

/* The whole step for m tokens. token_mask (may be NULL = all) selects the
 * tokens whose expert FFNs are evaluated; routing and buckets always cover
 * all m tokens. out [m*H] (rows of unselected tokens are left untouched),
 * ids [m*k], w [m*k], y_pairs [m*k*H] (optional: per (t, j) expert output).
 * With a shared expert (has_shared), every selected token also runs expert
 * E, and its output is added with weight 1 after the k routed terms: the
 * always-on shared expert of the DeepSeek MoE block ("lna-lab/README.md",
 * "What is in the pack": shared experts among the dense linears).
 * Returns the number of OpenMP threads used. */
int orc_moe_layer(const orc_layer *L, int m, const uint16_t *x_bf16, const float *logits,
                  const uint8_t *token_mask, double *out, int32_t *ids, double *w,
                  double *y_pairs)
{
    int E = L->num_experts, k = L->top_k, H = L->hidden;
    orc_route(m, E, k, logits, ids, w);

    int npairs = 0;
    int *pair_t = (int *)malloc(sizeof(int) * m * k);
    int *pair_j = (int *)malloc(sizeof(int) * m * k);
    for (int t = 0; t < m; ++t)
        if (!token_mask || token_mask[t])
            for (int j = 0; j < k; ++j) {
                pair_t[npairs] = t;
                pair_j[npairs] = j;
                ++npairs;
            }

    /* Activations: bf16 -> double, rotated by R_H for the codebook format. */
    double *xr = (double *)malloc(sizeof(double) * (size_t)m * H);
    for (int t = 0; t < m; ++t) {
        double *xt = (double *)malloc(sizeof(double) * H);
        for (int c = 0; c < H; ++c)
            xt[c] = orc_bf16_to_double(x_bf16[(size_t)t * H + c]);
        if (L->format == ORC_FMT_CODEBOOK)
            orc_rotate(H, L->signs_hidden, xt, xr + (size_t)t * H);
        else
            memcpy(xr + (size_t)t * H, xt, sizeof(double) * H);
        free(xt);
    }

    double *ys = (double *)malloc(sizeof(double) * (size_t)(npairs ? npairs : 1) * H);
    double *ysh = NULL;  /* shared expert output per token */
    if (L->has_shared)
        ysh = (double *)malloc(sizeof(double) * (size_t)(m ? m : 1) * H);
    int used = 1;
#pragma omp parallel
    {
#ifdef _OPENMP
#pragma omp single
        used = omp_get_num_threads();
#endif
#pragma omp for schedule(dynamic, 1)
        for (int p = 0; p < npairs + (L->has_shared ? npairs / (k ? k : 1) : 0); ++p) {
            if (p < npairs) {
                int t = pair_t[p], j = pair_j[p];
                orc_expert(L, ids[t * k + j], xr + (size_t)t * H, ys + (size_t)p * H);
            } else {
                int t = pair_t[(p - npairs) * k];
                orc_expert(L, E, xr + (size_t)t * H, ysh + (size_t)t * H);
            }
        }
    }

    /* Combine in slot order j = 0..k-1. */
    for (int p0 = 0; p0 < npairs; p0 += k) {
        int t = pair_t[p0];
        for (int i = 0; i < H; ++i) {
            double acc = 0.0;
            for (int j = 0; j < k; ++j)
                acc += w[t * k + j] * ys[(size_t)(p0 + j) * H + i];
            if (ysh)
                acc += ysh[(size_t)t * H + i];
            out[(size_t)t * H + i] = acc;
        }
        if (y_pairs)
            for (int j = 0; j < k; ++j)
                memcpy(y_pairs + ((size_t)t * k + j) * H, ys + (size_t)(p0 + j) * H,
                       sizeof(double) * H);
    }
    free(ys);
    free(ysh);
    free(xr);
    free(pair_t);
    free(pair_j);
    return used;
}

/* Threads of the OpenMP regions that follow on the calling thread (timing
 * the baseline on one core); n < 1 leaves the setting alone. */
void orc_set_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Dense dequantisation of one stored matrix (for small checks). */
void orc_dequant(const orc_layer *L, int e, int p, int N, int C, double *W)
{
    for (int n = 0; n < N; ++n)
        for (int c = 0; c < C; ++c)
            W[(size_t)n * C + c] = weight_at(L, e, p, N, C, n, c);
}
