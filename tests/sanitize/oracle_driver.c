/* Runs the C oracle (oracle/oracle.c) under AddressSanitizer and UndefinedBehaviorSanitizer:
 * every variant on ragged shapes with OpenMP threads, row subsets against the full output
 * (bitwise: the same code per row), the row-sum invariant (v = 1 gives 1, or 1 - lambda for
 * the differential's two maps, Table 1 of "Placement Is Free, Composition Is Not"), the
 * general single-head routine, and argument rejection. Prints "OK <checks>", exits 0. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_prefill_rows(const double *q, const double *k, const double *v, int variant,
                        long window, double lambda, long B, long H, long L, long d,
                        const long *rows, long nrows, double *out, int threads, int plant);
int oracle_prefill(const double *q, const double *k, const double *v, int variant, long window,
                   double lambda, long B, long H, long L, long d, double *out, int threads);
int oracle_attention_general(const double *q, const double *k, const double *v, long L,
                             long dqk, long dv, double scale, long window, double *out,
                             int threads);

static int checks = 0, fails = 0;
#define CHECK(c)                                                   \
    do {                                                           \
        ++checks;                                                  \
        if (!(c)) {                                                \
            ++fails;                                               \
            printf("FAILED line %d: %s\n", __LINE__, #c);          \
        }                                                          \
    } while (0)

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double uniform_pm1(void) /* splitmix64 to [-1, 1) */
{
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return (double)(z >> 11) / (double)(1ull << 52) - 1.0;
}

static double *alloc_fill(long n, double scale)
{
    double *p = malloc((size_t)n * sizeof(double));
    for (long i = 0; i < n; ++i) p[i] = scale * uniform_pm1();
    return p;
}

static void run_shape(int variant, long window, double lambda, long B, long H, long L, long d)
{
    long n = B * H * L * d;
    double *q = alloc_fill(n, 2.0), *k = alloc_fill(n, 2.0), *v = alloc_fill(n, 1.0);
    double *out = malloc((size_t)n * sizeof(double));
    CHECK(oracle_prefill(q, k, v, variant, window, lambda, B, H, L, d, out, 3) == 0);
    int finite = 1;
    for (long i = 0; i < n; ++i) finite &= isfinite(out[i]) != 0;
    CHECK(finite);

    /* a row subset, last row first: each listed row equals the full output's row */
    long rows[3] = {L - 1, 0, L / 2};
    long nr = L >= 3 ? 3 : 1;
    double *sub = malloc((size_t)(B * H * nr * d) * sizeof(double));
    CHECK(oracle_prefill_rows(q, k, v, variant, window, lambda, B, H, L, d, rows, nr, sub, 2,
                              0) == 0);
    int same = 1;
    for (long bh = 0; bh < B * H; ++bh)
        for (long r = 0; r < nr; ++r)
            same &= memcmp(sub + (bh * nr + r) * d, out + (bh * L + rows[r]) * d,
                           (size_t)d * sizeof(double)) == 0;
    CHECK(same);

    /* v = 1: every output is the sum of its row's weights (1, or 1 - lambda) */
    for (long i = 0; i < n; ++i) v[i] = 1.0;
    CHECK(oracle_prefill(q, k, v, variant, window, lambda, B, H, L, d, out, 1) == 0);
    double want = variant == 2 ? 1.0 - lambda : 1.0, err = 0.0;
    for (long i = 0; i < n; ++i) err = fmax(err, fabs(out[i] - want));
    CHECK(err < 1e-12);
    free(q);
    free(k);
    free(v);
    free(out);
    free(sub);
}

int main(void)
{
    const long Ls[] = {1, 2, 7, 33, 100};
    for (int li = 0; li < 5; ++li) {
        run_shape(0, 0, 0.0, 1, 2, Ls[li], 8);
        run_shape(1, 1, 0.0, 2, 1, Ls[li], 4);
        run_shape(1, 5, 0.0, 1, 2, Ls[li], 8);
        run_shape(2, 0, 0.8, 1, 2, Ls[li], 8);
        run_shape(2, 0, -0.3, 2, 1, Ls[li], 4);
    }
    /* the general routine: causal and windowed */
    {
        long L = 17, dqk = 3, dv = 5;
        double *q = alloc_fill(L * dqk, 1.0), *k = alloc_fill(L * dqk, 1.0);
        double *v = alloc_fill(L * dv, 1.0), *o = malloc((size_t)(L * dv) * sizeof(double));
        CHECK(oracle_attention_general(q, k, v, L, dqk, dv, 0.7, 0, o, 2) == 0);
        CHECK(oracle_attention_general(q, k, v, L, dqk, dv, 0.7, 4, o, 2) == 0);
        CHECK(oracle_attention_general(q, k, v, 0, dqk, dv, 0.7, 0, o, 2) != 0);
        free(q);
        free(k);
        free(v);
        free(o);
    }
    /* rejected arguments (no output is touched) */
    double x[64] = {0};
    long badrow[1] = {8};
    CHECK(oracle_prefill(x, x, x, 3, 0, 0.0, 1, 1, 8, 8, x, 1) != 0);
    CHECK(oracle_prefill(x, x, x, 1, 0, 0.0, 1, 1, 8, 8, x, 1) != 0);
    CHECK(oracle_prefill(x, x, x, 2, 0, 0.5, 1, 1, 8, 7, x, 1) != 0);
    CHECK(oracle_prefill(x, x, x, 0, 0, 0.0, 0, 1, 8, 8, x, 1) != 0);
    CHECK(oracle_prefill_rows(x, x, x, 0, 0, 0.0, 1, 1, 8, 8, badrow, 1, x, 1, 0) != 0);
    CHECK(oracle_prefill_rows(x, x, x, 0, 0, 0.0, 1, 1, 8, 8, badrow, -1, x, 1, 0) != 0);
    if (fails) {
        printf("%d of %d checks failed\n", fails, checks);
        return 1;
    }
    printf("OK %d\n", checks);
    return 0;
}
