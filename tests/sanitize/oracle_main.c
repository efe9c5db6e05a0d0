/*
 * Driver for the AddressSanitizer / UndefinedBehaviorSanitizer build of the
 * C oracle (tests/test_sanitizers_cpu.py).  Calls every entry point of
 * oracle/grkan_oracle.c over all degree pairs up to the limit, edge shapes
 * (no rows, one row, groups of one channel), rejected arguments and special
 * values (+-0, subnormals, huge, +-inf, NaN, exact roots of Q), and checks a
 * few closed forms so that the run also exercises the arithmetic, not only
 * the memory accesses.  Exit status 0 = every check passed; a sanitizer
 * report aborts the run with a non-zero status.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int grkan_oracle_nout(int m, int n);
void grkan_oracle_point(double x, double dy, int m, int n, const double *a, const double *b, double *out);
int grkan_oracle_rows(const double *x, const double *dy, long rows, long d, int n_g, int m, int n,
                      const double *A, const double *B, double *y, double *ymag, double *dx,
                      double *dxmag, double *sums, double *sumsq, double *magsq);
int grkan_oracle_points(const double *xv, const double *dyv, const long *idx, long n_el, long d, int n_g,
                        int m, int n, const double *A, const double *B, double *out);

static int failures = 0;
#define CHECK(c)                                                          \
    do {                                                                  \
        if (!(c)) {                                                       \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            ++failures;                                                   \
        }                                                                 \
    } while (0)

static double rnd(unsigned *s)
{
    *s = *s * 1664525u + 1013904223u;
    return ((double)(*s >> 8) / 16777216.0 - 0.5) * 4.0;
}

int main(void)
{
    unsigned seed = 12345u;
    const double specials[] = {0.0, -0.0, 1e-310, -1e-310, 1e300, -1e300, INFINITY, -INFINITY, NAN,
                               0.75, 1.0, 2.5, -3.0, 1e-30};
    const int ns = (int)(sizeof specials / sizeof specials[0]);
    double a[16], b[16], *out = malloc(sizeof(double) * (size_t)grkan_oracle_nout(15, 15));
    for (int m = 0; m <= 15; ++m) {
        for (int n = 0; n <= 15; ++n) {
            for (int i = 0; i <= m; ++i) a[i] = rnd(&seed);
            for (int j = 0; j < n; ++j) b[j] = rnd(&seed);
            for (int k = 0; k < ns; ++k) grkan_oracle_point(specials[k], 1.0, m, n, a, b, out);
            for (int k = 0; k < 8; ++k) grkan_oracle_point(rnd(&seed), rnd(&seed), m, n, a, b, out);
        }
    }
    /* closed form: a = x, b = 0 gives F = x and dF/dx = 1 */
    {
        double ai[6] = {0, 1, 0, 0, 0, 0}, bz[4] = {0, 0, 0, 0};
        for (int k = 0; k < 8; ++k) {
            double x = rnd(&seed);
            grkan_oracle_point(x, 2.0, 5, 4, ai, bz, out);
            CHECK(out[0] == x && out[1] == 2.0);
        }
        /* an exact root of Q: b = (-0.75, 1) makes Q(0.75) = 0, so s = 0 */
        double br[4] = {-0.75, 1.0, 0.0, 0.0};
        grkan_oracle_point(0.75, 1.0, 5, 4, ai, br, out);
        CHECK(out[4] == 0.0 && out[1] == 1.0);
    }
    /* whole tensors: shapes with no rows, one row, one channel per group */
    const long shapes[][3] = {{0, 8, 8}, {1, 8, 8}, {3, 24, 8}, {5, 7, 7}, {4, 6, 1}, {2, 64, 64}};
    for (int t = 0; t < 6; ++t) {
        long rows = shapes[t][0], d = shapes[t][1];
        int ng = (int)shapes[t][2];
        long nel = rows * d;
        size_t sz = sizeof(double) * (size_t)(nel > 0 ? nel : 1);
        double *x = malloc(sz), *dy = malloc(sz), *y = malloc(sz), *ym = malloc(sz), *dx = malloc(sz),
               *dxm = malloc(sz);
        double *A = malloc(sizeof(double) * (size_t)ng * 6), *B = malloc(sizeof(double) * (size_t)ng * 4);
        double *sums = calloc((size_t)ng * 10, sizeof(double)), *sq = calloc((size_t)ng * 10, sizeof(double)),
               *mq = calloc((size_t)ng * 10, sizeof(double));
        for (long i = 0; i < nel; ++i) {
            x[i] = (i % 5 == 0) ? specials[i % ns] : rnd(&seed);
            dy[i] = rnd(&seed);
        }
        for (int i = 0; i < ng * 6; ++i) A[i] = rnd(&seed);
        for (int i = 0; i < ng * 4; ++i) B[i] = rnd(&seed);
        CHECK(grkan_oracle_rows(x, dy, rows, d, ng, 5, 4, A, B, y, ym, dx, dxm, sums, sq, mq) == 0);
        CHECK(grkan_oracle_rows(x, NULL, rows, d, ng, 5, 4, A, B, y, ym, NULL, NULL, NULL, NULL, NULL) == 0);
        if (nel > 0) {
            long idx[3] = {0, nel / 2, nel - 1};
            double *rec = malloc(sizeof(double) * 3 * (size_t)grkan_oracle_nout(5, 4));
            double xv[3] = {x[0], x[nel / 2], x[nel - 1]}, dv[3] = {dy[0], dy[nel / 2], dy[nel - 1]};
            CHECK(grkan_oracle_points(xv, dv, idx, 3, d, ng, 5, 4, A, B, rec) == 0);
            free(rec);
        }
        free(x); free(dy); free(y); free(ym); free(dx); free(dxm); free(A); free(B);
        free(sums); free(sq); free(mq);
    }
    /* rejected arguments: the routines return -1 and touch nothing */
    {
        double x1 = 1.0, o1 = 0.0;
        CHECK(grkan_oracle_rows(&x1, &x1, 1, 7, 2, 5, 4, a, b, &o1, NULL, NULL, NULL, NULL, NULL, NULL) == -1);
        CHECK(grkan_oracle_rows(&x1, &x1, 1, 1, 1, 16, 4, a, b, &o1, NULL, NULL, NULL, NULL, NULL, NULL) == -1);
        CHECK(grkan_oracle_rows(&x1, NULL, 1, 1, 1, 5, 4, a, b, NULL, NULL, &o1, NULL, NULL, NULL, NULL) == -1);
        CHECK(grkan_oracle_rows(&x1, &x1, -1, 1, 1, 5, 4, a, b, &o1, NULL, NULL, NULL, NULL, NULL, NULL) == -1);
    }
    free(out);
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    puts("oracle sanitizer run: ok");
    return 0;
}
