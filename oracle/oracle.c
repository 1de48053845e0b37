/*
 * oracle.c -- plain fp64 CPU reference for causal prefill of one sequence-mixer layer.
 *
 * TEST INFRASTRUCTURE ONLY. The test-suite, the smoke check and the CPU-baseline leg of the
 * benchmark load this library; the product (the HIP library and its Python binding) never
 * does. It shares no source, header or helper with the GPU path.
 *
 * Source: "Placement Is Free, Composition Is Not: The Latin Square as a Provably-Balanced
 * Construction for Heterogeneous Sequence-Mixer Stacks".
 *   Table 1 (sec. 3.1): full attends every earlier position exactly; sliding sees only a
 *   local window of recent positions; differential takes the difference of two attention
 *   maps, each computed over half of the head dimension.
 *   Sec. 8 (causal safety): no mixer may read future positions.
 *   Table 2 (sec. 4.1): heads 16, head_dim 128, bfloat16.
 *
 * Readings taken where the page is silent (each one is a choice):
 *   - causal: key j is visible to query i iff j <= i (the diagonal is visible);
 *   - sliding window W counts the query itself: visible iff 0 <= i - j <= W - 1;
 *   - score scale 1/sqrt(d) for full and sliding, 1/sqrt(d/2) for differential;
 *   - differential splits q and k into the contiguous halves [0, d/2) and [d/2, d); v keeps
 *     all d channels; both maps use the causal mask; out = (P1 - lambda * P2) V with one
 *     scalar lambda.
 *
 * Arithmetic is the definition written out, one query row at a time, in double:
 *   s_j = scale * <q_i, k_j> for visible j;  m = max_j s_j;  w_j = exp(s_j - m);
 *   p_j = w_j / sum_j w_j;  out_i = sum_j p_j v_j   (keys in ascending order).
 * Inputs are widened to double by the caller (the exact values the GPU sees).
 *
 * Built with: gcc -O2 -fopenmp -ffp-contract=off -fPIC -shared (no fast-math).
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_FULL = 0, ORACLE_SLIDING = 1, ORACLE_DIFFERENTIAL = 2 };

/* Visible keys of query i, as the inclusive range [*lo, *hi].
 * `plant` deliberately breaks the mask for the positive control of the causal audit
 * (sec. 8): 1 = one future key leaks (j <= i + 1), 2 = the window admits one key too many.
 * The audit must flag both; plant = 0 is the real definition. */
static void visible_range(int variant, long i, long L, long window, int plant, long *lo, long *hi)
{
    long h = i;
    long l = 0;
    if (variant == ORACLE_SLIDING) {
        long w = window + (plant == 2 ? 1 : 0);
        l = i - (w - 1);
        if (l < 0) l = 0;
    }
    if (plant == 1) {
        h = i + 1;
        if (h > L - 1) h = L - 1;
    }
    *lo = l;
    *hi = h;
}

/* Softmax weights of one query row over keys lo..hi (two passes: max, then exp and sum).
 * q points at dqk channels of the query; k at row 0 of the keys, row pitch ldk; channel
 * offset c0. Writes p[0 .. hi-lo]. */
static void softmax_row(const double *q, const double *k, long ldk, long c0, long dqk,
                        long lo, long hi, double scale, double *p)
{
    double m = -INFINITY;
    for (long j = lo; j <= hi; ++j) {
        const double *kj = k + j * ldk + c0;
        double dot = 0.0;
        for (long c = 0; c < dqk; ++c) dot += q[c0 + c] * kj[c];
        double s = dot * scale;
        p[j - lo] = s;
        if (s > m) m = s;
    }
    double z = 0.0;
    for (long j = lo; j <= hi; ++j) {
        double w = exp(p[j - lo] - m);
        p[j - lo] = w;
        z += w;
    }
    for (long j = lo; j <= hi; ++j) p[j - lo] /= z;
}

/* One head: q, k of width dqk_total (row pitch ldq / ldk), v of width dv (pitch ldv).
 * Computes the listed rows (rows == NULL means every row 0..L-1) into out[r * dv + c]. */
static void head_rows(const double *q, const double *k, const double *v,
                      long ldq, long ldk, long ldv, long L, long dqk_total, long dv,
                      int variant, long window, double lambda, double scale, int plant,
                      const long *rows, long nrows, double *out, int threads)
{
    long n = rows ? nrows : L;
#ifdef _OPENMP
#pragma omp parallel num_threads(threads > 0 ? threads : omp_get_max_threads())
#endif
    {
        double *p1 = (double *)malloc(sizeof(double) * (size_t)L);
        double *p2 = (double *)malloc(sizeof(double) * (size_t)L);
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 16)
#endif
        for (long r = 0; r < n; ++r) {
            long i = rows ? rows[r] : r;
            long lo, hi;
            visible_range(variant, i, L, window, plant, &lo, &hi);
            const double *qi = q + i * ldq;
            double *o = out + r * dv;
            for (long c = 0; c < dv; ++c) o[c] = 0.0;
            if (variant == ORACLE_DIFFERENTIAL) {
                long half = dqk_total / 2;
                softmax_row(qi, k, ldk, 0, half, lo, hi, scale, p1);
                softmax_row(qi, k, ldk, half, half, lo, hi, scale, p2);
                for (long j = lo; j <= hi; ++j) {
                    double wgt = p1[j - lo] - lambda * p2[j - lo];
                    const double *vj = v + j * ldv;
                    for (long c = 0; c < dv; ++c) o[c] += wgt * vj[c];
                }
            } else {
                softmax_row(qi, k, ldk, 0, dqk_total, lo, hi, scale, p1);
                for (long j = lo; j <= hi; ++j) {
                    double wgt = p1[j - lo];
                    const double *vj = v + j * ldv;
                    for (long c = 0; c < dv; ++c) o[c] += wgt * vj[c];
                }
            }
        }
        free(p1);
        free(p2);
    }
}

static int check_args(int variant, long window, long B, long H, long L, long d)
{
    if (B < 1 || H < 1 || L < 1 || d < 1) return -1;
    if (variant < ORACLE_FULL || variant > ORACLE_DIFFERENTIAL) return -1;
    if (variant == ORACLE_SLIDING && window < 1) return -1;
    if (variant == ORACLE_DIFFERENTIAL && (d % 2) != 0) return -1;
    return 0;
}

/* One mixer layer over [B, H, L, d] contiguous row-major q, k, v.
 * rows: NULL for every row, else nrows query indices (each in [0, L)) computed for every
 * (b, h). out: [B, H, nrows_or_L, d]. threads <= 0 uses every core. plant: see
 * visible_range (0 in every use except the positive control). Returns 0, or -1 on bad
 * arguments. */
int oracle_prefill_rows(const double *q, const double *k, const double *v,
                        int variant, long window, double lambda,
                        long B, long H, long L, long d,
                        const long *rows, long nrows, double *out, int threads, int plant)
{
    if (check_args(variant, window, B, H, L, d) != 0) return -1;
    if (rows) {
        if (nrows < 0) return -1;
        for (long r = 0; r < nrows; ++r)
            if (rows[r] < 0 || rows[r] >= L) return -1;
    }
    long n = rows ? nrows : L;
    double scale = (variant == ORACLE_DIFFERENTIAL) ? 1.0 / sqrt((double)(d / 2))
                                                    : 1.0 / sqrt((double)d);
    for (long bh = 0; bh < B * H; ++bh) {
        const double *qh = q + bh * L * d;
        const double *kh = k + bh * L * d;
        const double *vh = v + bh * L * d;
        head_rows(qh, kh, vh, d, d, d, L, d, d, variant, window, lambda, scale, plant,
                  rows, nrows, out + bh * n * d, threads);
    }
    return 0;
}

/* Every row of one layer. */
int oracle_prefill(const double *q, const double *k, const double *v,
                   int variant, long window, double lambda,
                   long B, long H, long L, long d, double *out, int threads)
{
    return oracle_prefill_rows(q, k, v, variant, window, lambda, B, H, L, d,
                               NULL, 0, out, threads, 0);
}

/* Single-head causal softmax attention with independent widths: q, k are [L, dqk], v is
 * [L, dv], out is [L, dv], with an explicit score scale. Full causal mask, or a sliding
 * window when window >= 1 (window <= 0 means no window). Used to state the differential
 * identity: with equal halves, differential(lambda) = (1 - lambda) * attention over the
 * half-width scores with full-width values. */
int oracle_attention_general(const double *q, const double *k, const double *v,
                             long L, long dqk, long dv, double scale, long window,
                             double *out, int threads)
{
    if (L < 1 || dqk < 1 || dv < 1) return -1;
    int variant = window >= 1 ? ORACLE_SLIDING : ORACLE_FULL;
    head_rows(q, k, v, dqk, dqk, dv, L, dqk, dv, variant, window, 0.0, scale, 0,
              NULL, 0, out, threads);
    return 0;
}

/* Cores OpenMP would use by default (reported next to the CPU-baseline timing). */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
