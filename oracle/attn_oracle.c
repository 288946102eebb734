/*
 * attn_oracle.c -- plain fp64 CPU oracle for the attention forward.
 *
 * TEST INFRASTRUCTURE ONLY. The product library never links, loads or calls
 * this file. Only the tests, the smoke check and the benchmark's CPU-baseline
 * leg use it. It shares no code, header, table or constant with the GPU path.
 *
 * What it computes is the plain definition of softmax attention, not the
 * tiled method. All four pages state that the tiled method reaches exactly
 * this result (up to rounding order), so the oracle is that definition written
 * out:
 *   - Ascend C FlashAttention-2 tile-fusion page (ascendai.csdn.net),
 *     section 1.1 (scores, row softmax, product with V) and section 1.2
 *     (the tiled rewrite is mathematically the same result);
 *   - ops-transformer FlashAttention walkthrough (hwcomputing.csdn.net,
 *     6a0ef689), "core idea: tiling + online softmax" (S = QK^T, P =
 *     softmax(S), O = PV over [B,H,S,D] tensors);
 *   - catlass FlashAttention article (lnwmold.com/news/1200460), section
 *     "background" (same result as standard attention) and section "usage"
 *     (full / causal / (window_left, window_right) masks);
 *   - "FlashAttention on Ascend NPU: from principle to practice" page
 *     (hwcomputing.csdn.net, 6a0fe629), section "core idea: IO-aware"
 *     (standard attention divides QK^T by sqrt(head_dim) before softmax).
 *
 * For every batch b, head h and query row i:
 *   s_ij = scale * sum_d q[b,h,i,d] * k[b,h,j,d]  if key j is visible from i,
 *          -inf                                    otherwise;
 *   m_i  = max_j s_ij                               (pass 1);
 *   e_ij = exp(s_ij - m_i),  l_i = sum_j e_ij       (pass 2);
 *   o[b,h,i,:] = (sum_j e_ij * v[b,h,j,:]) / l_i;
 *   lse[b,h,i] = m_i + log(l_i)   (natural log of sum_j exp(s_ij)).
 * A row with no visible key (none exists for the three mask modes, since
 * j = i is always visible) is defined as o = 0, lse = -inf.
 *
 * Inputs are raw 16-bit patterns (IEEE binary16 or bfloat16) in contiguous
 * row-major [B,H,S,D] order. Everything after decoding is fp64; exp and log
 * are the C library's double routines.
 *
 * Readings of points the pages leave open are listed with each function.
 *
 * ORACLE_PLANT (compile-time, tests only): when defined to a nonzero value,
 * one deliberate mistake is built in, so the test suite can show that its
 * pins catch it. The default build defines nothing and is the oracle.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#ifndef ORACLE_PLANT
#define ORACLE_PLANT 0
#endif

/* Element encodings accepted by the oracle (its own codes). */
enum { ORACLE_F16 = 0, ORACLE_BF16 = 1 };
/* Mask modes (its own codes): catlass article, section "usage". */
enum { ORACLE_FULL = 0, ORACLE_CAUSAL = 1, ORACLE_WINDOW = 2 };

/* IEEE 754 binary16 -> double, exact: 1 sign bit, 5 exponent bits (bias 15),
 * 10 fraction bits; exponent 0 encodes zero/subnormals, 31 encodes inf/NaN. */
double oracle_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int ex = (h >> 10) & 0x1f;
    int fr = h & 0x3ff;
    double v;
    if (ex == 0)
        v = ldexp((double)fr, -24);              /* fr * 2^(1-15-10) */
    else if (ex == 31)
        v = fr ? NAN : INFINITY;
    else
        v = ldexp((double)(fr | 0x400), ex - 25); /* (1024+fr) * 2^(ex-15-10) */
    return sign ? -v : v;
}

/* bfloat16 -> double, exact: a bfloat16 is the upper half of an IEEE binary32. */
double oracle_bf16_to_f64(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double decode(uint16_t x, int dtype)
{
    return dtype == ORACLE_BF16 ? oracle_bf16_to_f64(x) : oracle_f16_to_f64(x);
}

/* The element type's value nearest to x, ties to the even significand
 * (round-to-nearest-even), as a double. A binary format with p significand
 * bits (11 for binary16, 8 for bfloat16) and smallest normal 2^emin (2^-14,
 * 2^-126) spaces its values 2^(e - p) apart where x = m 2^e, 0.5 <= |m| < 1,
 * and never closer than its subnormal step 2^(emin - p + 1); a value past the
 * largest finite one (65504, or (2 - 2^-7) 2^127) after rounding is +-inf. */
double oracle_round(double x, int dtype)
{
    const int p = dtype == ORACLE_BF16 ? 8 : 11;
    const int emin = dtype == ORACLE_BF16 ? -126 : -14;
    const double maxf = dtype == ORACLE_BF16 ? ldexp(2.0 - ldexp(1.0, -7), 127) : 65504.0;
    if (x == 0.0 || isnan(x) || isinf(x)) return x;
    int e;
    frexp(x, &e);
    const int q = (e - p > emin - p + 1) ? e - p : emin - p + 1;
#if ORACLE_PLANT == 9
    const double r = ldexp(round(ldexp(x, -q)), q);      /* planted: ties away from zero */
#else
    const double r = ldexp(nearbyint(ldexp(x, -q)), q);  /* exact scaling; RNE */
#endif
    if (fabs(r) > maxf) return x > 0 ? INFINITY : -INFINITY;
    return r;
}

/* Is key j visible from query i?
 *   full:   always (catlass article, "usage": no mask).
 *   causal: j <= i. The Ascend C tile-fusion page, section 4.2, masks a key
 *           exactly when its position is after the query's, so the diagonal
 *           stays visible.
 *   window: i - wl <= j <= i + wr, both ends inclusive; a negative bound means
 *           that side is unbounded. The catlass article ("usage") only names a
 *           (window_left, window_right) pair; this inclusive reading makes
 *           (-1, 0) the causal mask and (-1, -1) the full mask. */
int oracle_visible(int64_t i, int64_t j, int mask_mode, int64_t wl, int64_t wr)
{
    switch (mask_mode) {
    case ORACLE_FULL:
        return 1;
    case ORACLE_CAUSAL:
#if ORACLE_PLANT == 2
        return j < i;                    /* planted: diagonal dropped */
#else
        return j <= i;
#endif
    case ORACLE_WINDOW: {
#if ORACLE_PLANT == 3
        int left_ok = wl < 0 || j > i - wl;   /* planted: left edge exclusive */
#else
        int left_ok = wl < 0 || j >= i - wl;
#endif
        int right_ok = wr < 0 || j <= i + wr;
        return left_ok && right_ok;
    }
    default:
        return 0;
    }
}

/* Number of visible (i, j) pairs of one S x S head, by enumeration. */
int64_t oracle_pair_count(int64_t S, int mask_mode, int64_t wl, int64_t wr)
{
    int64_t total = 0;
#pragma omp parallel for reduction(+ : total) schedule(static)
    for (int64_t i = 0; i < S; ++i)
        for (int64_t j = 0; j < S; ++j)
            total += oracle_visible(i, j, mask_mode, wl, wr);
    return total;
}

static int check_args(int64_t B, int64_t H, int64_t S, int64_t D, int mask_mode, int dtype)
{
    if (B < 0 || H < 0 || S < 0 || D <= 0) return -1;
    if (mask_mode < ORACLE_FULL || mask_mode > ORACLE_WINDOW) return -1;
    if (dtype != ORACLE_F16 && dtype != ORACLE_BF16) return -1;
    return 0;
}

/* The scaled score of a visible pair from its dot product. */
static double scaled(double acc, double scale)
{
#if ORACLE_PLANT == 1
    (void)scale;
    return acc;                          /* planted: scale dropped */
#elif ORACLE_PLANT == 4
    return -scale * acc;                 /* planted: sign flipped */
#else
    return scale * acc;
#endif
}

/* Softmax of a materialised score row (S entries, -inf where hidden) and its
 * product with the head's [S, D] value block vh: two passes over srow.
 * orow (D doubles) is scratch owned by the caller. */
static void finish_row(const double *srow, const uint16_t *vh, int64_t S, int64_t D,
                       int dtype, double *orow, double *o_out, double *lse_out);

/* One query row against S keys: materialise the score row, then two passes.
 * qsrc points at the query row's D values, kh and vh at the head's [S, D] key
 * and value blocks; i is the query's position in the sequence, which the mask
 * compares with the key positions 0 .. S-1. srow (S doubles), qrow and orow (D
 * doubles each) are scratch owned by the caller. */
static void one_row(const uint16_t *qsrc, const uint16_t *kh, const uint16_t *vh,
                    int64_t S, int64_t D, double scale, int mask_mode, int64_t wl,
                    int64_t wr, int dtype, int64_t i, double *srow, double *qrow,
                    double *orow, double *o_out, double *lse_out)
{
    for (int64_t d = 0; d < D; ++d)
        qrow[d] = decode(qsrc[d], dtype);

    /* Scores (Ascend C tile-fusion page, section 1.1; the NPU optimisation
     * page, section "core idea: IO-aware": QK^T times the scale). Masked
     * entries are -inf and need no dot product. */
    for (int64_t j = 0; j < S; ++j) {
        if (!oracle_visible(i, j, mask_mode, wl, wr)) {
            srow[j] = -INFINITY;
            continue;
        }
        double acc = 0.0;
        for (int64_t d = 0; d < D; ++d)
            acc += qrow[d] * decode(kh[j * D + d], dtype);
        srow[j] = scaled(acc, scale);
    }
    finish_row(srow, vh, S, D, dtype, orow, o_out, lse_out);
}

/* As one_row, for a query row and a key block given as fp64 values (the
 * rotated rows of the RoPE attention below). */
static void one_row_f64(const double *qrow, const double *kd, const uint16_t *vh, int64_t S,
                        int64_t D, double scale, int mask_mode, int64_t wl, int64_t wr,
                        int dtype, int64_t i, double *srow, double *orow, double *o_out,
                        double *lse_out)
{
    for (int64_t j = 0; j < S; ++j) {
        if (!oracle_visible(i, j, mask_mode, wl, wr)) {
            srow[j] = -INFINITY;
            continue;
        }
        double acc = 0.0;
        for (int64_t d = 0; d < D; ++d)
            acc += qrow[d] * kd[j * D + d];
        srow[j] = scaled(acc, scale);
    }
    finish_row(srow, vh, S, D, dtype, orow, o_out, lse_out);
}

static void finish_row(const double *srow, const uint16_t *vh, int64_t S, int64_t D,
                       int dtype, double *orow, double *o_out, double *lse_out)
{
    /* Pass 1: row maximum. */
    double m = -INFINITY;
    for (int64_t j = 0; j < S; ++j)
        if (srow[j] > m) m = srow[j];

    if (m == -INFINITY) {                 /* no visible key */
        for (int64_t d = 0; d < D; ++d) o_out[d] = 0.0;
        *lse_out = -INFINITY;
        return;
    }

    /* Pass 2: exponentials, their sum, and the weighted sum of V rows. */
    for (int64_t d = 0; d < D; ++d) orow[d] = 0.0;
    double l = 0.0;
    for (int64_t j = 0; j < S; ++j) {
        if (srow[j] == -INFINITY) continue;        /* exp(-inf) = 0 */
        double e = exp(srow[j] - m);
        l += e;
#if ORACLE_PLANT == 5
        int64_t jv = (j + 1 < S) ? j + 1 : j;      /* planted: wrong V row */
#else
        int64_t jv = j;
#endif
        for (int64_t d = 0; d < D; ++d)
            orow[d] += e * decode(vh[jv * D + d], dtype);
    }
    for (int64_t d = 0; d < D; ++d) o_out[d] = orow[d] / l;
#if ORACLE_PLANT == 6
    *lse_out = m + log2(l);               /* planted: wrong logarithm base */
#else
    *lse_out = m + log(l);
#endif
}

/* Selected rows of a [B,H,S,D] problem.
 * rows[r] is a flat row index (b*H + h)*S + i; o is [n_rows, D] and lse is
 * [n_rows], both fp64. nthreads <= 0 uses the OpenMP default.
 * Returns 0, or -1 on a bad argument. */
int oracle_attention_rows(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                          int64_t B, int64_t H, int64_t S, int64_t D, double scale,
                          int mask_mode, int64_t wl, int64_t wr, int dtype,
                          int64_t n_rows, const int64_t *rows, double *o, double *lse,
                          int nthreads)
{
    if (check_args(B, H, S, D, mask_mode, dtype)) return -1;
    int64_t total_rows = B * H * S;
    for (int64_t r = 0; r < n_rows; ++r)
        if (rows[r] < 0 || rows[r] >= total_rows) return -1;
    if (n_rows == 0) return 0;

#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#else
    nthreads = 1;
#endif
    int failed = 0;
#pragma omp parallel num_threads(nthreads) reduction(| : failed)
    {
        double *srow = (double *)malloc(sizeof(double) * (size_t)(S > 0 ? S : 1));
        double *qrow = (double *)malloc(sizeof(double) * (size_t)D);
        double *orow = (double *)malloc(sizeof(double) * (size_t)D);
        if (!srow || !qrow || !orow) {
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int64_t r = 0; r < n_rows; ++r) {
                int64_t bh = rows[r] / S;
                int64_t i = rows[r] % S;
                const int64_t base = bh * S * D;
                one_row(q + base + i * D, k + base, v + base, S, D, scale, mask_mode, wl, wr,
                        dtype, i, srow, qrow, orow, o + r * D, lse + r);
            }
        }
        free(srow);
        free(qrow);
        free(orow);
    }
    return failed ? -1 : 0;
}

/* One whole head with the probability matrix materialised: p is [S, S] with
 * p[i, j] = exp(s_ij - m_i) / l_i, o is [S, D], lse is [S]. Small S only
 * (the S x S matrix is what the tiled method avoids writing). */
int oracle_attention_probs(const uint16_t *qh, const uint16_t *kh, const uint16_t *vh,
                           int64_t S, int64_t D, double scale, int mask_mode, int64_t wl,
                           int64_t wr, int dtype, double *p, double *o, double *lse)
{
    if (check_args(1, 1, S, D, mask_mode, dtype)) return -1;
    double *qrow = (double *)malloc(sizeof(double) * (size_t)D);
    double *orow = (double *)malloc(sizeof(double) * (size_t)D);
    if (!qrow || !orow) {
        free(qrow);
        free(orow);
        return -1;
    }
    for (int64_t i = 0; i < S; ++i) {
        double *srow = p + i * S;
        one_row(qh + i * D, kh, vh, S, D, scale, mask_mode, wl, wr, dtype, i, srow, qrow, orow,
                o + i * D, lse + i);
        /* one_row leaves the scores in srow; turn them into probabilities. */
        double m = -INFINITY;
        for (int64_t j = 0; j < S; ++j)
            if (srow[j] > m) m = srow[j];
        if (m == -INFINITY) {
            for (int64_t j = 0; j < S; ++j) srow[j] = 0.0;
            continue;
        }
        double l = 0.0;
        for (int64_t j = 0; j < S; ++j)
            l += (srow[j] == -INFINITY) ? 0.0 : exp(srow[j] - m);
        for (int64_t j = 0; j < S; ++j)
            srow[j] = (srow[j] == -INFINITY) ? 0.0 : exp(srow[j] - m) / l;
    }
    free(qrow);
    free(orow);
    return 0;
}

/* New query rows against a key/value cache (incremental decoding).
 * q is [B,H,Sq,D]; k and v are [B,H,Sk,D] and hold the first Sk positions of
 * each sequence, the new rows' own keys included; o is [B,H,Sq,D] and lse is
 * [B,H,Sq], both fp64. Query row i sits at position Sk - Sq + i (the new rows
 * are the last Sq positions), and key j is visible from it under the rules of
 * oracle_visible at that position. Everything else is the definition above.
 * Reading: the NPU optimisation page (hwcomputing.csdn.net, 6a0fe629),
 * section "optimisation 4: KV-cache reuse", computes the attention of the new
 * token against the cached keys and values of its sequence, and its hands-on
 * section (step 3) feeds a [1, 32, 1, 128] query against a [1, 32, 50, 128]
 * cache. The code printed there attends to the last cached key only and then
 * averages outputs, which is not attention; the plain reading is attention of
 * each new row over every visible cached key, which is what this computes.
 * Requires 1 <= Sq <= Sk. nthreads <= 0 uses the OpenMP default.
 * Returns 0, or -1 on a bad argument. */
int oracle_attention_kv(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                        int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D,
                        double scale, int mask_mode, int64_t wl, int64_t wr, int dtype,
                        double *o, double *lse, int nthreads)
{
    if (check_args(B, H, Sk, D, mask_mode, dtype)) return -1;
    if (Sq < 1 || Sq > Sk) return -1;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#else
    nthreads = 1;
#endif
    const int64_t n_rows = B * H * Sq;
    int failed = 0;
#pragma omp parallel num_threads(nthreads) reduction(| : failed)
    {
        double *srow = (double *)malloc(sizeof(double) * (size_t)Sk);
        double *qrow = (double *)malloc(sizeof(double) * (size_t)D);
        double *orow = (double *)malloc(sizeof(double) * (size_t)D);
        if (!srow || !qrow || !orow) {
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int64_t r = 0; r < n_rows; ++r) {
                const int64_t bh = r / Sq, i = r % Sq;
#if ORACLE_PLANT == 7
                const int64_t pos = i;                 /* planted: top-left alignment */
#else
                const int64_t pos = Sk - Sq + i;
#endif
                one_row(q + r * D, k + bh * Sk * D, v + bh * Sk * D, Sk, D, scale,
                        mask_mode, wl, wr, dtype, pos, srow, qrow, orow, o + r * D, lse + r);
            }
        }
        free(srow);
        free(qrow);
        free(orow);
    }
    return failed ? -1 : 0;
}

/* Rotary position embedding (RoPE) of n_rows rows of D values.
 * Ascend C tile-fusion page, section 9 (integration with RoPE): Q and K rows
 * are rotated according to their position, from a cos/sin table, before the
 * scores are formed. The page names the table but not the formula; the
 * reading here is the usual rotary embedding: the D dimensions form D/2 pairs
 * (a_t, b_t), and pair t of a row at position p turns by the angle whose
 * cosine and sine are c = cos_t[p * D/2 + t], s = sin_t[p * D/2 + t]:
 *     x'[a_t] = x[a_t] * c - x[b_t] * s,    x'[b_t] = x[b_t] * c + x[a_t] * s.
 * Pairing mode 0 (halves): a_t = t, b_t = t + D/2. Mode 1 (interleaved):
 * a_t = 2t, b_t = 2t + 1. Row r is at position pos[r]. Table values are taken
 * exactly (fp32 -> fp64); everything is fp64 and out is not rounded. D must
 * be even.
 * Returns 0, or -1 on a bad argument. */
int oracle_rope_rows(const uint16_t *x, int64_t n_rows, int64_t D, const int64_t *pos,
                     const float *cos_t, const float *sin_t, int mode, int dtype, double *out)
{
    if (D <= 0 || D % 2 || (mode != 0 && mode != 1)) return -1;
    if (dtype != ORACLE_F16 && dtype != ORACLE_BF16) return -1;
    const int64_t half = D / 2;
    for (int64_t r = 0; r < n_rows; ++r) {
        const uint16_t *xr = x + r * D;
        double *yr = out + r * D;
        for (int64_t t = 0; t < half; ++t) {
            const int64_t a = mode == 0 ? t : 2 * t;
            const int64_t b = mode == 0 ? t + half : 2 * t + 1;
            const double c = (double)cos_t[pos[r] * half + t];
            const double sn = (double)sin_t[pos[r] * half + t];
            const double xa = decode(xr[a], dtype), xb = decode(xr[b], dtype);
#if ORACLE_PLANT == 8
            yr[a] = xa * c + xb * sn;            /* planted: rotation sign */
            yr[b] = xb * c - xa * sn;
#else
            yr[a] = xa * c - xb * sn;
            yr[b] = xb * c + xa * sn;
#endif
        }
    }
    return 0;
}

/* Selected rows of RoPE attention over [B,H,S,D]: every query and key row is
 * rotated by oracle_rope_rows at its position in the sequence (0 .. S-1, from
 * tables with at least S rows) and each rotated value rounded to the element
 * type (oracle_round), then the attention above is taken of those rows (v is
 * not rotated). Reading: the tile-fusion page, section 9, applies the
 * rotation as the Q and K tiles are loaded for the matrix unit, which takes
 * the element type (section 10: fp16 inputs, fp32 accumulation), so the
 * rotated rows enter QK^T in the element type. rows, o, lse and nthreads as
 * for oracle_attention_rows. Returns 0, or -1 on a bad argument. */
int oracle_attention_rope_rows(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                               int64_t B, int64_t H, int64_t S, int64_t D, double scale,
                               int mask_mode, int64_t wl, int64_t wr, int dtype,
                               const float *cos_t, const float *sin_t, int mode,
                               int64_t n_rows, const int64_t *rows, double *o, double *lse,
                               int nthreads)
{
    if (check_args(B, H, S, D, mask_mode, dtype)) return -1;
    if (D % 2 || (mode != 0 && mode != 1)) return -1;
    const int64_t total_rows = B * H * S;
    for (int64_t r = 0; r < n_rows; ++r)
        if (rows[r] < 0 || rows[r] >= total_rows) return -1;
    if (n_rows == 0) return 0;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#else
    nthreads = 1;
#endif
    double *kd = (double *)malloc(sizeof(double) * (size_t)(S * D));
    if (!kd) return -1;
    int failed = 0;
    /* head by head: rotate the head's keys once, then its selected rows */
    for (int64_t bh = 0; bh < B * H && !failed; ++bh) {
        int64_t any = 0;
        for (int64_t r = 0; r < n_rows && !any; ++r) any = rows[r] / S == bh;
        if (!any) continue;
        const int64_t base = bh * S * D;
#pragma omp parallel for num_threads(nthreads) schedule(static)
        for (int64_t j = 0; j < S; ++j) {
            const int64_t p = j;
            oracle_rope_rows(k + base + j * D, 1, D, &p, cos_t, sin_t, mode, dtype, kd + j * D);
            for (int64_t d = 0; d < D; ++d) kd[j * D + d] = oracle_round(kd[j * D + d], dtype);
        }
#pragma omp parallel num_threads(nthreads) reduction(| : failed)
        {
            double *srow = (double *)malloc(sizeof(double) * (size_t)(S > 0 ? S : 1));
            double *qrow = (double *)malloc(sizeof(double) * (size_t)D);
            double *orow = (double *)malloc(sizeof(double) * (size_t)D);
            if (!srow || !qrow || !orow) {
                failed = 1;
            } else {
#pragma omp for schedule(dynamic, 4)
                for (int64_t r = 0; r < n_rows; ++r) {
                    if (rows[r] / S != bh) continue;
                    const int64_t i = rows[r] % S;
                    oracle_rope_rows(q + base + i * D, 1, D, &i, cos_t, sin_t, mode, dtype,
                                     qrow);
                    for (int64_t d = 0; d < D; ++d) qrow[d] = oracle_round(qrow[d], dtype);
                    one_row_f64(qrow, kd, v + base, S, D, scale, mask_mode, wl, wr, dtype, i,
                                srow, orow, o + r * D, lse + r);
                }
            }
            free(srow);
            free(qrow);
            free(orow);
        }
    }
    free(kd);
    return failed ? -1 : 0;
}

/* New query rows against a key/value cache whose keys are already rotated
 * (a rotary-embedding cache): query row i of a head is rotated by
 * oracle_rope_rows at its position Sk - Sq + i and each value rounded to the
 * element type (as in oracle_attention_rope_rows), then attends to the cached
 * keys as given, under the rules of oracle_attention_kv. Reading: the
 * tile-fusion page, section 9, rotates Q and K as their tiles load; keys
 * enter the cache rotated, so only the new rows are rotated here.
 * Returns 0, or -1 on a bad argument. */
int oracle_attention_kv_rope(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                             int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D,
                             double scale, int mask_mode, int64_t wl, int64_t wr, int dtype,
                             const float *cos_t, const float *sin_t, int mode, double *o,
                             double *lse, int nthreads)
{
    if (check_args(B, H, Sk, D, mask_mode, dtype)) return -1;
    if (Sq < 1 || Sq > Sk || D % 2 || (mode != 0 && mode != 1)) return -1;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#else
    nthreads = 1;
#endif
    double *kd = (double *)malloc(sizeof(double) * (size_t)(Sk * D));
    if (!kd) return -1;
    int failed = 0;
    for (int64_t bh = 0; bh < B * H && !failed; ++bh) {
        for (int64_t t = 0; t < Sk * D; ++t) kd[t] = decode(k[bh * Sk * D + t], dtype);
#pragma omp parallel num_threads(nthreads) reduction(| : failed)
        {
            double *srow = (double *)malloc(sizeof(double) * (size_t)Sk);
            double *qrow = (double *)malloc(sizeof(double) * (size_t)D);
            double *orow = (double *)malloc(sizeof(double) * (size_t)D);
            if (!srow || !qrow || !orow) {
                failed = 1;
            } else {
#pragma omp for schedule(static)
                for (int64_t i = 0; i < Sq; ++i) {
                    const int64_t r = bh * Sq + i, pos = Sk - Sq + i;
                    oracle_rope_rows(q + r * D, 1, D, &pos, cos_t, sin_t, mode, dtype, qrow);
                    for (int64_t d = 0; d < D; ++d) qrow[d] = oracle_round(qrow[d], dtype);
                    one_row_f64(qrow, kd, v + bh * Sk * D, Sk, D, scale, mask_mode, wl, wr,
                                dtype, pos, srow, orow, o + r * D, lse + r);
                }
            }
            free(srow);
            free(qrow);
            free(orow);
        }
    }
    free(kd);
    return failed ? -1 : 0;
}

/* Gradients of the attention (the backward pass) for every head of
 * [B,H,S,D] inputs, given dO = dL/dO for some loss L.
 * The ops-transformer walkthrough (hwcomputing.csdn.net, 6a0ef689), closing
 * remark, notes that the backward pass needs state kept from the forward pass
 * and does not spell it out; what it computes is fixed by the calculus of the
 * forward's plain definition, written out here per head with P materialised:
 *   P_ij  = softmax_j(s_ij) as in the forward (0 where hidden),
 *   dV_j  = sum_i P_ij dO_i,
 *   dP_ij = dO_i . V_j,
 *   dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik)        (the softmax Jacobian),
 *   dQ_i  = scale sum_j dS_ij K_j,    dK_j = scale sum_i dS_ij Q_i.
 * (sum_k P_ik dP_ik equals dO_i . O_i.) A row with no visible key (not
 * reachable with these masks) contributes nothing.
 * Besides the gradients it returns, for the comparison rule of the tests,
 * the sums of the magnitudes of the terms each gradient element adds up,
 * with A_i = sum_d |dO_id O_id| and, for a visible pair, |x|_t = max(|x|, t)
 * where t is the element type's smallest normal (2^-14 for binary16, 2^-126
 * for bfloat16: below it, rounding to the type errs by up to half the
 * subnormal spacing, t times the unit roundoff, rather than by a relative
 * amount):
 *   mag_dv_jd = sum_i |P_ij|_t |dO_id|,
 *   mag_dq_id = |scale| sum_j (|dS_ij|_t + P_ij A_i) |K_jd|,
 *   mag_dk_jd = |scale| sum_i (|dS_ij|_t + P_ij A_i) |Q_id|.
 * All outputs are fp64 [B,H,S,D]. nthreads <= 0 uses the OpenMP default.
 * Returns 0, or -1 on a bad argument or allocation failure. */
int oracle_attention_bwd(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                         const uint16_t *dout, int64_t B, int64_t H, int64_t S, int64_t D,
                         double scale, int mask_mode, int64_t wl, int64_t wr, int dtype,
                         double *dq, double *dk, double *dv, double *mag_dq, double *mag_dk,
                         double *mag_dv, int nthreads)
{
    if (check_args(B, H, S, D, mask_mode, dtype)) return -1;
    if (S == 0) return 0;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#else
    nthreads = 1;
#endif
    const size_t hd = (size_t)(S * D), ss = (size_t)(S * S);
    double *qd = (double *)malloc(sizeof(double) * hd), *kd = (double *)malloc(sizeof(double) * hd);
    double *vd = (double *)malloc(sizeof(double) * hd), *dod = (double *)malloc(sizeof(double) * hd);
    double *P = (double *)malloc(sizeof(double) * ss), *dS = (double *)malloc(sizeof(double) * ss);
    double *A = (double *)malloc(sizeof(double) * (size_t)S);
    int failed = !qd || !kd || !vd || !dod || !P || !dS || !A;
    const double tiny = dtype == ORACLE_BF16 ? ldexp(1.0, -126) : ldexp(1.0, -14);
    for (int64_t bh = 0; bh < B * H && !failed; ++bh) {
        const int64_t base = bh * S * D;
        for (size_t t = 0; t < hd; ++t) {
            qd[t] = decode(q[base + t], dtype);
            kd[t] = decode(k[base + t], dtype);
            vd[t] = decode(v[base + t], dtype);
            dod[t] = decode(dout[base + t], dtype);
        }
        /* rows: probabilities, dS, dQ */
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 4)
        for (int64_t i = 0; i < S; ++i) {
            double *Pi = P + i * S, *dSi = dS + i * S;
            double m = -INFINITY;
            for (int64_t j = 0; j < S; ++j) {
                if (!oracle_visible(i, j, mask_mode, wl, wr)) {
                    Pi[j] = -INFINITY;
                    continue;
                }
                double acc = 0.0;
                for (int64_t d = 0; d < D; ++d) acc += qd[i * D + d] * kd[j * D + d];
                Pi[j] = scaled(acc, scale);
                if (Pi[j] > m) m = Pi[j];
            }
            double l = 0.0;
            for (int64_t j = 0; j < S; ++j) {
                Pi[j] = (m == -INFINITY || Pi[j] == -INFINITY) ? 0.0 : exp(Pi[j] - m);
                l += Pi[j];
            }
            for (int64_t j = 0; j < S; ++j) Pi[j] = l > 0.0 ? Pi[j] / l : 0.0;
            /* dP, its P-weighted row sum, dS; A_i from O_i = sum_j P_ij V_j */
            double dsum = 0.0, a = 0.0;
            for (int64_t j = 0; j < S; ++j) {
                double dp = 0.0;
                if (Pi[j] != 0.0)
                    for (int64_t d = 0; d < D; ++d) dp += dod[i * D + d] * vd[j * D + d];
                dSi[j] = dp;
                dsum += Pi[j] * dp;
            }
            for (int64_t d = 0; d < D; ++d) {
                double o = 0.0;
                for (int64_t j = 0; j < S; ++j) o += Pi[j] * vd[j * D + d];
                a += fabs(dod[i * D + d] * o);
            }
            A[i] = a;
#if ORACLE_PLANT == 10
            (void)dsum;
            for (int64_t j = 0; j < S; ++j) dSi[j] = Pi[j] * dSi[j];  /* planted: no row term */
#else
            for (int64_t j = 0; j < S; ++j) dSi[j] = Pi[j] * (dSi[j] - dsum);
#endif
            for (int64_t d = 0; d < D; ++d) {
                double g = 0.0, mg = 0.0;
                for (int64_t j = 0; j < S; ++j) {
                    if (Pi[j] == 0.0) continue;          /* hidden (or underflowed) pair */
                    g += dSi[j] * kd[j * D + d];
#if ORACLE_PLANT == 12
                    mg += fmax(fabs(dSi[j]), tiny) * fabs(kd[j * D + d]);  /* planted: no P A term */
#else
                    mg += (fmax(fabs(dSi[j]), tiny) + Pi[j] * a) * fabs(kd[j * D + d]);
#endif
                }
                dq[base + i * D + d] = scale * g;
                mag_dq[base + i * D + d] = fabs(scale) * mg;
            }
        }
        /* columns: dK, dV */
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 4)
        for (int64_t j = 0; j < S; ++j) {
            for (int64_t d = 0; d < D; ++d) {
                double gk = 0.0, gv = 0.0, mk = 0.0, mv = 0.0;
                for (int64_t i = 0; i < S; ++i) {
                    const double p = P[i * S + j], ds = dS[i * S + j];
                    if (p == 0.0) continue;              /* hidden (or underflowed) pair */
                    gv += p * dod[i * D + d];
                    mv += fmax(p, tiny) * fabs(dod[i * D + d]);
                    gk += ds * qd[i * D + d];
                    mk += (fmax(fabs(ds), tiny) + p * A[i]) * fabs(qd[i * D + d]);
                }
                dv[base + j * D + d] = gv;
#if ORACLE_PLANT == 11
                mag_dv[base + j * D + d] = 2.0 * mv;     /* planted: doubled sum */
#else
                mag_dv[base + j * D + d] = mv;
#endif
                dk[base + j * D + d] = scale * gk;
                mag_dk[base + j * D + d] = fabs(scale) * mk;
            }
        }
    }
    free(qd);
    free(kd);
    free(vd);
    free(dod);
    free(P);
    free(dS);
    free(A);
    return failed ? -1 : 0;
}

/* Decode n raw 16-bit values to fp64 with the oracle's own decoders. */
void oracle_decode(const uint16_t *x, int64_t n, int dtype, double *out)
{
    for (int64_t t = 0; t < n; ++t) out[t] = decode(x[t], dtype);
}

/* Threads the oracle will use by default (reported by the CPU baseline). */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
