/*
 * loki_oracle.c -- plain, slow, fp64 CPU oracle for one Loki decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product (the HIP library or its
 * Python binding) may include, link, load or call this file.  Only the test
 * suite, the smoke check and the CPU-baseline leg of the benchmark use it.
 * It shares no code with the GPU path: its own dtype decoding, its own
 * rounding, its own loops.
 *
 * What it follows ("Loki: Low-Rank Keys for Efficient Sparse Attention",
 * Singhania et al., NeurIPS 2024):
 *   - deep-diver.github.io NeurIPS-2024 poster page, "Visual Insights",
 *     Figure 1 (right) and its repeated descriptions under "More on figures":
 *     keys are projected offline by PCA; at inference approximate attention
 *     scores are computed in the low-dimensional space, the top-k tokens are
 *     kept, and the final attention scores of those tokens use the
 *     full-dimensional keys.
 *   - same page, "TL;DR": the exact attention scores are computed just for
 *     the tokens that the low-dimensional ranking keeps.
 *   - briefgpt.xyz keyword page (the paper's abstract): tokens in the KV-cache
 *     are ranked and selected by attention scores computed in low-dimensional
 *     space.
 *
 * Readings taken where the pages are silent (each one is listed with its
 * reason in the design notes of the repository):
 *   - the cache stores the keys already rotated into the PCA basis, at full
 *     dimension D: krot = k . P, P a D x D orthonormal matrix whose columns are
 *     principal directions in descending variance;
 *   - the query is rotated the same way: qr = q . P;
 *   - the approximate score of token t is the plain dot product over the
 *     leading d rotated coordinates, no rescaling;
 *   - top-k order is (score descending, index ascending); the selected index
 *     set is reported in ascending order;
 *   - the final logits are scale * (qr . krot_t) over all D coordinates with
 *     scale = 1/sqrt(D) unless given; softmax runs over the k selected tokens
 *     only;
 *   - grouped-query attention maps query head h to KV head h / (Hq / Hkv);
 *   - a newly appended key is rotated in exact arithmetic and rounded once,
 *     to nearest with ties to even, to the storage dtype.
 *
 * Parity pins (which tests tie each function to something other than itself)
 * are listed in the header of oracle/loki_oracle.py.
 *
 * All arithmetic is fp64.  Storage dtypes are decoded exactly to fp64.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2, OR_F64 = 3 };

/* ------------------------------------------------------------------ */
/* storage dtype decoding (exact)                                      */
/* ------------------------------------------------------------------ */

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
static double half_bits_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);                 /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m + 1024), e - 25);     /* (1 + m/2^10) 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16: 1 sign, 8 exponent (bias 127), 7 fraction bits. */
static double bf16_bits_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 7) & 0xff;
    int m = h & 0x7f;
    double v;
    if (e == 0)
        v = ldexp((double)m, -133);                /* subnormal: m * 2^-133 */
    else if (e == 255)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m + 128), e - 134);     /* (1 + m/2^7) 2^(e-127) */
    return sign ? -v : v;
}

static double load_elem(const void *base, int dtype, size_t i)
{
    switch (dtype) {
    case OR_F32: {
        float f;
        memcpy(&f, (const char *)base + 4 * i, 4);
        return (double)f;
    }
    case OR_F16: {
        uint16_t h;
        memcpy(&h, (const char *)base + 2 * i, 2);
        return half_bits_to_double(h);
    }
    case OR_BF16: {
        uint16_t h;
        memcpy(&h, (const char *)base + 2 * i, 2);
        return bf16_bits_to_double(h);
    }
    default: {
        double x;
        memcpy(&x, (const char *)base + 8 * i, 8);
        return x;
    }
    }
}

/* ------------------------------------------------------------------ */
/* rounding fp64 -> storage dtype, to nearest, ties to even            */
/* ------------------------------------------------------------------ */

/* x >= 0; quantum is a power of two, so x / quantum is exact. */
static double round_to_quantum(double x, double quantum)
{
    double n = x / quantum;
    double f = floor(n);
    double frac = n - f;
    if (frac > 0.5 || (frac == 0.5 && fmod(f, 2.0) != 0.0))
        f += 1.0;
    return f * quantum;
}

/*
 * Generic binary format with `mant` fraction bits, smallest normal exponent
 * `emin`, overflow threshold `ovf` (values >= ovf round to infinity).
 * Returns the magnitude bits (no sign).
 */
static uint32_t encode_small_float(double x, int mant, int emin, int bias, double ovf,
                                   uint32_t inf_bits)
{
    if (x >= ovf)
        return inf_bits;
    int E;
    (void)frexp(x, &E);            /* x = m 2^E, m in [0.5, 1): leading bit 2^(E-1) */
    int lead = (x == 0.0) ? emin : E - 1;
    if (lead < emin)
        lead = emin;               /* subnormals share the smallest binade's quantum */
    double r = round_to_quantum(x, ldexp(1.0, lead - mant));
    if (r < ldexp(1.0, emin))      /* subnormal (or the smallest normal, reached by rounding) */
        return (uint32_t)(r / ldexp(1.0, emin - mant));
    int E2;
    double m2 = frexp(r, &E2);
    uint32_t biased = (uint32_t)(E2 - 1 + bias);
    uint32_t frac = (uint32_t)((m2 * 2.0 - 1.0) * ldexp(1.0, mant));
    return (biased << mant) | frac;
}

static uint16_t double_to_half_bits(double v)
{
    if (isnan(v))
        return 0x7e00;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    /* largest finite 65504; the midpoint to 2^16 is 65520 and rounds up */
    return sign | (uint16_t)encode_small_float(fabs(v), 10, -14, 15, 65520.0, 0x7c00);
}

static uint16_t double_to_bf16_bits(double v)
{
    if (isnan(v))
        return 0x7fc0;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double ovf = ldexp(2.0 - ldexp(1.0, -8), 127);
    return sign | (uint16_t)encode_small_float(fabs(v), 7, -126, 127, ovf, 0x7f80);
}

static void store_elem(void *base, int dtype, size_t i, double x)
{
    switch (dtype) {
    case OR_F32: {
        float f = (float)x;        /* C conversion: round to nearest even */
        memcpy((char *)base + 4 * i, &f, 4);
        break;
    }
    case OR_F16: {
        uint16_t h = double_to_half_bits(x);
        memcpy((char *)base + 2 * i, &h, 2);
        break;
    }
    case OR_BF16: {
        uint16_t h = double_to_bf16_bits(x);
        memcpy((char *)base + 2 * i, &h, 2);
        break;
    }
    default:
        memcpy((char *)base + 8 * i, &x, 8);
    }
}

/* Exposed so tests can pin the rounding against library conversions. */
void oracle_round_to_dtype(const double *x, size_t n, int dtype, void *dst)
{
    for (size_t i = 0; i < n; i++)
        store_elem(dst, dtype, i, x[i]);
}

void oracle_decode_dtype(const void *src, size_t n, int dtype, double *x)
{
    for (size_t i = 0; i < n; i++)
        x[i] = load_elem(src, dtype, i);
}

/* ------------------------------------------------------------------ */
/* the steps of one decode step                                        */
/* ------------------------------------------------------------------ */

/* Rotation into the PCA basis: y[j] = sum_i x[i] P[i][j]  (row vector times P). */
static void rotate_row(const void *x, int dtype, size_t x_off, const double *P, int D, double *y)
{
    for (int j = 0; j < D; j++) {
        double acc = 0.0;
        for (int i = 0; i < D; i++)
            acc += load_elem(x, dtype, x_off + i) * P[(size_t)i * D + j];
        y[j] = acc;
    }
}

typedef struct {
    double s;
    int32_t t;
} scored_t;

/* (score descending, index ascending) */
static int cmp_rank(const void *a, const void *b)
{
    const scored_t *x = (const scored_t *)a, *y = (const scored_t *)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->t > y->t) - (x->t < y->t);
}

static int cmp_i32(const void *a, const void *b)
{
    int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

/*
 * Top-k selection: the k tokens that rank first by (s descending, t ascending),
 * returned as an ascending index list.  A full library sort is the step.
 */
static void topk_ascending(const double *s, int S, int k, int32_t *idx, scored_t *tmp)
{
    for (int t = 0; t < S; t++) {
        tmp[t].s = (s[t] == 0.0) ? 0.0 : s[t];    /* -0 ranks as +0 */
        tmp[t].t = t;
    }
    qsort(tmp, (size_t)S, sizeof(scored_t), cmp_rank);
    for (int i = 0; i < k; i++)
        idx[i] = tmp[i].t;
    qsort(idx, (size_t)k, sizeof(int32_t), cmp_i32);
}

void oracle_topk_rows(const double *s, int n_rows, int S, int k, int32_t *idx)
{
    scored_t *tmp = (scored_t *)malloc(sizeof(scored_t) * (size_t)S);
    for (int r = 0; r < n_rows; r++)
        topk_ascending(s + (size_t)r * S, S, k, idx + (size_t)r * k, tmp);
    free(tmp);
}

/*
 * Exact attention over a given index set: logits scale * (qr . krot_t) over all
 * D rotated coordinates, softmax over the set, weighted sum of the V rows.
 */
static void attend_selected(const double *qr, const void *krot, const void *v, int dtype,
                            size_t head_off, int D, const int32_t *idx, int k, double scale,
                            double *out, double *z)
{
    double m = -INFINITY;
    for (int i = 0; i < k; i++) {
        size_t row = head_off + (size_t)idx[i] * D;
        double acc = 0.0;
        for (int j = 0; j < D; j++)
            acc += qr[j] * load_elem(krot, dtype, row + j);
        z[i] = scale * acc;
        if (z[i] > m)
            m = z[i];
    }
    double L = 0.0;
    for (int i = 0; i < k; i++) {
        z[i] = exp(z[i] - m);
        L += z[i];
    }
    for (int j = 0; j < D; j++)
        out[j] = 0.0;
    for (int i = 0; i < k; i++) {
        size_t row = head_off + (size_t)idx[i] * D;
        for (int j = 0; j < D; j++)
            out[j] += z[i] * load_elem(v, dtype, row + j);
    }
    for (int j = 0; j < D; j++)
        out[j] /= L;
}

/*
 * One decode step for a list of (batch, query-head) units.
 *
 *   q     [B, Hq, D]        storage dtype
 *   krot  [B, Hkv, S, D]    rotated keys (logical row-major), storage dtype
 *   v     [B, Hkv, S, D]    values, storage dtype
 *   P     [Hkv, D, D]       fp64 (exact copy of whatever the caller stores)
 *   heads flattened b*Hq + h; NULL means every unit
 * Outputs (indexed by the full (b, h) position; only listed units written):
 *   out [B,Hq,D], idx [B,Hq,k] ascending, scores [B,Hq,S] (nullable),
 *   qr_out [B,Hq,D] (nullable).
 * Returns 0, or -1 on an argument outside the method's domain.
 */
int oracle_decode(int B, int Hq, int Hkv, int S, int D, int d, int k, double scale, int dtype,
                  const void *q, const void *krot, const void *v, const double *P,
                  const int32_t *heads, int n_heads, double *out, int32_t *idx,
                  double *scores, double *qr_out)
{
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || S < 1 || D < 1 || d < 1 || d > D ||
        k < 1 || k > S)
        return -1;
    if (!(scale > 0.0))
        scale = 1.0 / sqrt((double)D);
    int g = Hq / Hkv;
    int n_units = heads ? n_heads : B * Hq;

#pragma omp parallel for schedule(dynamic, 1)
    for (int u = 0; u < n_units; u++) {
        int unit = heads ? heads[u] : u;
        int b = unit / Hq, h = unit % Hq;
        int kv = h / g;
        double *qr = (double *)malloc(sizeof(double) * (size_t)D);
        double *s = (double *)malloc(sizeof(double) * (size_t)S);
        double *z = (double *)malloc(sizeof(double) * (size_t)k);
        scored_t *tmp = (scored_t *)malloc(sizeof(scored_t) * (size_t)S);
        size_t head_off = ((size_t)b * Hkv + kv) * (size_t)S * D;

        /* 1. rotate the query into the PCA basis */
        rotate_row(q, dtype, (size_t)unit * D, P + (size_t)kv * D * D, D, qr);

        /* 2. approximate scores from the leading d rotated coordinates */
        for (int t = 0; t < S; t++) {
            double acc = 0.0;
            for (int j = 0; j < d; j++)
                acc += qr[j] * load_elem(krot, dtype, head_off + (size_t)t * D + j);
            s[t] = acc;
        }

        /* 3. top-k by approximate score */
        int32_t *my_idx = idx + (size_t)unit * k;
        topk_ascending(s, S, k, my_idx, tmp);

        /* 4. exact full-dimensional attention over the selected tokens */
        attend_selected(qr, krot, v, dtype, head_off, D, my_idx, k, scale,
                        out + (size_t)unit * D, z);

        if (scores)
            memcpy(scores + (size_t)unit * S, s, sizeof(double) * (size_t)S);
        if (qr_out)
            memcpy(qr_out + (size_t)unit * D, qr, sizeof(double) * (size_t)D);
        free(qr);
        free(s);
        free(z);
        free(tmp);
    }
    return 0;
}

/*
 * Exact attention over caller-given index sets (used to compare outputs
 * "given identical index sets").  qr comes from this oracle's own rotation.
 */
int oracle_attend_given(int B, int Hq, int Hkv, int S, int D, int k, double scale, int dtype,
                        const void *q, const void *krot, const void *v, const double *P,
                        const int32_t *idx, const int32_t *heads, int n_heads, double *out)
{
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || S < 1 || D < 1 || k < 1 || k > S)
        return -1;
    if (!(scale > 0.0))
        scale = 1.0 / sqrt((double)D);
    int g = Hq / Hkv;
    int n_units = heads ? n_heads : B * Hq;
    int bad = 0;

#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int u = 0; u < n_units; u++) {
        int unit = heads ? heads[u] : u;
        int b = unit / Hq, h = unit % Hq;
        int kv = h / g;
        const int32_t *my_idx = idx + (size_t)unit * k;
        for (int i = 0; i < k; i++)
            if (my_idx[i] < 0 || my_idx[i] >= S)
                bad = 1;
        if (bad)
            continue;
        double *qr = (double *)malloc(sizeof(double) * (size_t)D);
        double *z = (double *)malloc(sizeof(double) * (size_t)k);
        size_t head_off = ((size_t)b * Hkv + kv) * (size_t)S * D;
        rotate_row(q, dtype, (size_t)unit * D, P + (size_t)kv * D * D, D, qr);
        attend_selected(qr, krot, v, dtype, head_off, D, my_idx, k, scale,
                        out + (size_t)unit * D, z);
        free(qr);
        free(z);
    }
    return bad ? -1 : 0;
}

/*
 * PCAAttn, the variant of Loki that uses the low-dimensional attention scores
 * directly (poster page, "More on tables", the PCAAttn table, which describes
 * it as a Loki variant working with the reduced-dimensional scores).  Reading:
 * no top-k; each cached token's logit is scale times its low-dimensional score
 * (the dot product over the leading d rotated coordinates, as in the decode
 * step), softmax runs over all S tokens and the output is the weighted sum of
 * all S value rows.  Arguments as oracle_decode (out [B,Hq,D] only).
 */
int oracle_pca_attention(int B, int Hq, int Hkv, int S, int D, int d, double scale, int dtype,
                         const void *q, const void *krot, const void *v, const double *P,
                         const int32_t *heads, int n_heads, double *out)
{
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || S < 1 || D < 1 || d < 1 || d > D)
        return -1;
    if (!(scale > 0.0))
        scale = 1.0 / sqrt((double)D);
    const int g = Hq / Hkv;
    const int n_units = heads ? n_heads : B * Hq;

#pragma omp parallel for schedule(dynamic, 1)
    for (int u = 0; u < n_units; u++) {
        const int unit = heads ? heads[u] : u;
        const int b = unit / Hq, h = unit % Hq;
        const int kv = h / g;
        const size_t base = ((size_t)b * Hkv + kv) * (size_t)S * D;
        double *qr = (double *)malloc(sizeof(double) * (size_t)D);
        double *w = (double *)malloc(sizeof(double) * (size_t)S);

        /* the query in the PCA basis */
        rotate_row(q, dtype, (size_t)unit * D, P + (size_t)kv * D * D, D, qr);

        /* logits of every token from its leading d rotated coordinates */
        double zmax = -INFINITY;
        for (int t = 0; t < S; t++) {
            double dot = 0.0;
            for (int c = 0; c < d; c++)
                dot += qr[c] * load_elem(krot, dtype, base + (size_t)t * D + c);
            w[t] = scale * dot;
            if (w[t] > zmax)
                zmax = w[t];
        }
        /* softmax over all S tokens, then the weighted sum of the value rows */
        double denom = 0.0;
        for (int t = 0; t < S; t++) {
            w[t] = exp(w[t] - zmax);
            denom += w[t];
        }
        double *o = out + (size_t)unit * D;
        for (int c = 0; c < D; c++) {
            double acc = 0.0;
            for (int t = 0; t < S; t++)
                acc += w[t] * load_elem(v, dtype, base + (size_t)t * D + c);
            o[c] = acc / denom;
        }
        free(qr);
        free(w);
    }
    return 0;
}

/*
 * Calibration covariance (poster page, "Visual Insights", Figure 1 right, and
 * "More on figures": principal component analysis of the keys of a
 * calibration set, done offline).  For each KV head, with the n calibration
 * keys x_t (storage dtype, [Hkv, n, D]): mu = (1/n) sum_t x_t and
 * C = (1/n) sum_t (x_t - mu)(x_t - mu)^T, in fp64.  cov [Hkv, D, D].
 */
int oracle_covariance(int Hkv, int n, int D, int dtype, const void *keys, double *cov)
{
    if (Hkv < 1 || n < 1 || D < 1)
        return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int kv = 0; kv < Hkv; kv++) {
        const size_t kbase = (size_t)kv * n * D;
        double *mean = (double *)calloc((size_t)D, sizeof(double));
        double *xc = (double *)malloc(sizeof(double) * (size_t)D);
        double *C = cov + (size_t)kv * D * D;
        for (int t = 0; t < n; t++)
            for (int i = 0; i < D; i++)
                mean[i] += load_elem(keys, dtype, kbase + (size_t)t * D + i);
        for (int i = 0; i < D; i++)
            mean[i] /= (double)n;
        for (size_t e = 0; e < (size_t)D * D; e++)
            C[e] = 0.0;
        for (int t = 0; t < n; t++) {
            for (int i = 0; i < D; i++)
                xc[i] = load_elem(keys, dtype, kbase + (size_t)t * D + i) - mean[i];
            for (int i = 0; i < D; i++)
                for (int jj = 0; jj < D; jj++)
                    C[(size_t)i * D + jj] += xc[i] * xc[jj];
        }
        for (size_t e = 0; e < (size_t)D * D; e++)
            C[e] /= (double)n;
        free(mean);
        free(xc);
    }
    return 0;
}

/*
 * Append of one new token per (batch, KV head): the new key is rotated into
 * the PCA basis in fp64 and rounded once to the storage dtype; the value row
 * is stored unchanged.  (Poster page, "Loki's Computational Cost": the KV-cache
 * append is part of every decode step.)
 *
 *   k_new, v_new [B, Hkv, D] storage dtype;  P [Hkv, D, D] fp64
 *   krot_new_out, v_new_out [B, Hkv, D] storage dtype
 */
int oracle_append_rows(int B, int Hkv, int D, int dtype, const void *k_new, const void *v_new,
                       const double *P, void *krot_new_out, void *v_new_out)
{
    if (B < 1 || Hkv < 1 || D < 1)
        return -1;
    double *y = (double *)malloc(sizeof(double) * (size_t)D);
    for (int b = 0; b < B; b++)
        for (int kv = 0; kv < Hkv; kv++) {
            size_t off = ((size_t)b * Hkv + kv) * D;
            rotate_row(k_new, dtype, off, P + (size_t)kv * D * D, D, y);
            for (int j = 0; j < D; j++) {
                store_elem(krot_new_out, dtype, off + j, y[j]);
                store_elem(v_new_out, dtype, off + j, load_elem(v_new, dtype, off + j));
            }
        }
    free(y);
    return 0;
}

/* Query rotation alone: qr[b,h,:] = q[b,h,:] . P[h / g]. */
int oracle_rotate_queries(int B, int Hq, int Hkv, int D, int dtype, const void *q,
                          const double *P, double *qr)
{
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || D < 1)
        return -1;
    int g = Hq / Hkv;
    for (int b = 0; b < B; b++)
        for (int h = 0; h < Hq; h++) {
            size_t unit = (size_t)b * Hq + h;
            rotate_row(q, dtype, unit * D, P + (size_t)(h / g) * D * D, D, qr + unit * D);
        }
    return 0;
}
