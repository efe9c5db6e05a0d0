/*
 * grkan_oracle.c -- fp64 CPU oracle for the Group-Rational KAN (GR-KAN)
 * safe Pade activation, forward and backward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, constant or helper
 * with the HIP library; the only thing both sides share is the seeded input
 * generator, which holds none of the method's arithmetic.
 *
 * Pages cited
 *   [FlashKAT notes]  "FlashKAT: Understanding and Addressing Performance
 *                     Bottlenecks in the Kolmogorov-Arnold Transformer",
 *                     Paper-Notes page (AAAI 2026), arXiv 2505.13813.
 *
 * What is computed (the plain definition, in fp64, from the exact fp64 value
 * of every fp32/bf16 input):
 *
 *   GR-KAN splits the d channels into n_g groups whose channels share one
 *   coefficient set, and uses a "safe" Pade activation unit instead of a
 *   B-spline ([FlashKAT notes], section "KAT 的突破与残留问题").  Each group
 *   has 6 numerator and 4 denominator coefficients ([FlashKAT notes],
 *   section "损失函数 / 训练策略"), i.e. m = 5, n = 4, which also gives the
 *   m+n+1 = 10 coefficient accesses per element counted in section
 *   "2. 原始 KAT 的 atomic add 问题分析".  The pages print no formula; the
 *   reading taken here is
 *
 *       P(x) = sum_{i=0..5} a_i x^i,   Q(x) = sum_{j=1..4} b_j x^j,
 *       F(x) = P(x) / (1 + |Q(x)|).
 *
 *   Channel c belongs to group floor(c / d_g) (contiguous groups: each
 *   Algorithm-2 block handles all d_g channels of one group, section
 *   "3. FlashKAT 核函数重构（Algorithm 2）").
 *
 *   Backward (the gradients the pages call Eq. 10-11 in section
 *   "2. 原始 KAT 的 atomic add 问题分析" but do not print), by the chain rule
 *   with d|Q|/dQ = s = sign(Q), sign(0) = 0:
 *
 *       dX          = dY * ( P'/D - s P Q'/D^2 ),     D = 1 + |Q|
 *       dA[g][i]    = sum over every element of group g of  dY x^i / D
 *       dB[g][j-1]  = sum over every element of group g of -dY s P x^j / D^2
 *
 *   The sums run over all rows (batch x sequence) and all d_g channels of the
 *   group (same section).
 *
 * How: powers by repeated multiplication, polynomial values as plain sums in
 * ascending order (deliberately not Horner), one division per quotient.
 * sign(Q) is taken from the fp64 value unless |Q| is within the fp64
 * rounding bound of zero, in which case Q is re-evaluated in binary128
 * (x and b are fp32 values, so x^4 is exact there and the sign is right for
 * every input that is not an exact root).  Group sums are accumulated in
 * long double, row by row in index order.
 */
#include <math.h>
#include <float.h>
#include <stddef.h>

#define ORC_NA 6 /* numerator coefficients a_0..a_5   */
#define ORC_NB 4 /* denominator coefficients b_1..b_4 */

/* Per-element record written by grkan_oracle_point (doubles, in order). */
enum {
    ORC_F = 0,       /* F(x)                                            */
    ORC_DX = 1,      /* dY * dF/dx                                      */
    ORC_TA = 2,      /* 6 terms dY * dF/da_i = dY x^i / D               */
    ORC_TB = 8,      /* 4 terms dY * dF/db_j = -dY s P x^j / D^2        */
    ORC_FMAG = 12,   /* first-order rounding scale of F  (see below)    */
    ORC_DXMAG = 13,  /* first-order rounding scale of dX                */
    ORC_SIGN = 14,   /* s = sign(Q) as -1, 0, +1                        */
    ORC_D = 15,      /* D = 1 + |Q|                                     */
    ORC_NOUT = 16
};

int grkan_oracle_nout(void) { return ORC_NOUT; }

static int sign_of(double v) { return (v > 0.0) - (v < 0.0); }

/* sign(Q(x)) with Q(x) = sum_j b_j x^j; exact for fp32 x and b. */
static int sign_q(double x, const double b[ORC_NB], double q, double qabs)
{
    if (fabs(q) > 64.0 * DBL_EPSILON * qabs)
        return sign_of(q);
    __float128 xq = (__float128)x, pw = 1, acc = 0;
    for (int j = 1; j <= ORC_NB; ++j) {
        pw = pw * xq;
        acc = acc + (__float128)b[j - 1] * pw;
    }
    return (acc > 0) - (acc < 0);
}

/*
 * One element.  a[6] = a_0..a_5, b[4] = b_1..b_4.
 *
 * The two magnitude fields are the first-order error scale of an fp32
 * evaluation of the same quantity (sums of absolute values of every term,
 * propagated through the quotient): a correctly implemented fp32 kernel
 * differs from F and dX by a small multiple of 2^-24 times these, which is
 * what the comparator scales its relative tolerance by where F or dX is
 * itself close to zero.
 */
void grkan_oracle_point(double x, double dy, const double *a, const double *b,
                        double *out)
{
    double xp[ORC_NA];
    xp[0] = 1.0;
    for (int i = 1; i < ORC_NA; ++i)
        xp[i] = xp[i - 1] * x;
    double ax = fabs(x), axp[ORC_NA];
    axp[0] = 1.0;
    for (int i = 1; i < ORC_NA; ++i)
        axp[i] = axp[i - 1] * ax;

    double P = 0, Pd = 0, Pabs = 0, Pdabs = 0;
    for (int i = 0; i < ORC_NA; ++i) {
        P += a[i] * xp[i];
        Pabs += fabs(a[i]) * axp[i];
    }
    for (int i = 1; i < ORC_NA; ++i) {
        Pd += (double)i * a[i] * xp[i - 1];
        Pdabs += (double)i * fabs(a[i]) * axp[i - 1];
    }
    double Q = 0, Qd = 0, Qabs = 0, Qdabs = 0;
    for (int j = 1; j <= ORC_NB; ++j) {
        Q += b[j - 1] * xp[j];
        Qabs += fabs(b[j - 1]) * axp[j];
        Qd += (double)j * b[j - 1] * xp[j - 1];
        Qdabs += (double)j * fabs(b[j - 1]) * axp[j - 1];
    }
    int s = sign_q(x, b, Q, Qabs);
    double D = 1.0 + fabs(Q);
    double D2 = D * D;

    double F = P / D;
    double dFdx = Pd / D - (double)s * P * Qd / D2;
    out[ORC_F] = F;
    out[ORC_DX] = dy * dFdx;
    for (int i = 0; i < ORC_NA; ++i)
        out[ORC_TA + i] = dy * xp[i] / D;
    for (int j = 1; j <= ORC_NB; ++j)
        out[ORC_TB + j - 1] = -dy * (double)s * P * xp[j] / D2;

    double aP = fabs(P), aPd = fabs(Pd), aQd = fabs(Qd);
    out[ORC_FMAG] = (Pabs + aP * Qabs / D) / D;
    out[ORC_DXMAG] = fabs(dy) * ((Pdabs + aPd * Qabs / D) / D
                                 + (Pabs * aQd + aP * Qdabs + 2.0 * aP * aQd * Qabs / D) / D2);
    out[ORC_SIGN] = (double)s;
    out[ORC_D] = D;
}

/*
 * Rows [0, rows) of a row-major [rows][d] block.  x, dy: fp64 copies of the
 * inputs.  A: [n_g][6], B: [n_g][4] (fp64 copies of the fp32 coefficients).
 * Any output pointer may be NULL to skip it.
 *   y, ymag, dx, dxmag : [rows][d]
 *   sums, sumsq        : [n_g][10], accumulated into (+=), long double
 *                        internally; sums[g][k] += the group's terms,
 *                        sumsq[g][k] += their squares (for the L2 norm the
 *                        comparator scales its tolerance by).
 * dy may be NULL for a forward-only call (then dx, dxmag, sums, sumsq must
 * be NULL too).  Returns 0, or -1 on a bad shape.
 */
int grkan_oracle_rows(const double *x, const double *dy, long rows, long d,
                      int n_g, const double *A, const double *B,
                      double *y, double *ymag, double *dx, double *dxmag,
                      double *sums, double *sumsq)
{
    if (rows < 0 || d <= 0 || n_g <= 0 || d % n_g != 0)
        return -1;
    if (dy == NULL && (dx || dxmag || sums || sumsq))
        return -1;
    long dg = d / n_g;
    const int nk = ORC_NA + ORC_NB;
    long double acc[nk], acc2[nk];
    for (int g = 0; g < n_g; ++g) {
        for (int k = 0; k < nk; ++k)
            acc[k] = acc2[k] = 0.0L;
        for (long r = 0; r < rows; ++r) {
            for (long c = g * dg; c < (g + 1) * dg; ++c) {
                long idx = r * d + c;
                double out[ORC_NOUT];
                grkan_oracle_point(x[idx], dy ? dy[idx] : 0.0, A + ORC_NA * g,
                                   B + ORC_NB * g, out);
                if (y)
                    y[idx] = out[ORC_F];
                if (ymag)
                    ymag[idx] = out[ORC_FMAG];
                if (dx)
                    dx[idx] = out[ORC_DX];
                if (dxmag)
                    dxmag[idx] = out[ORC_DXMAG];
                for (int k = 0; k < nk; ++k) {
                    long double t = (long double)out[ORC_TA + k];
                    acc[k] += t;
                    acc2[k] += t * t;
                }
            }
        }
        if (sums)
            for (int k = 0; k < nk; ++k)
                sums[g * nk + k] += (double)acc[k];
        if (sumsq)
            for (int k = 0; k < nk; ++k)
                sumsq[g * nk + k] += (double)acc2[k];
    }
    return 0;
}

/*
 * Selected elements of a [rows][d] tensor: idx[n] are flat indices, xv/dyv
 * the fp64 values at them (gathered by the caller).  Writes n records of
 * ORC_NOUT doubles.
 */
int grkan_oracle_points(const double *xv, const double *dyv, const long *idx,
                        long n, long d, int n_g, const double *A,
                        const double *B, double *out)
{
    if (n < 0 || d <= 0 || n_g <= 0 || d % n_g != 0)
        return -1;
    long dg = d / n_g;
    for (long k = 0; k < n; ++k) {
        long c = idx[k] % d;
        int g = (int)(c / dg);
        grkan_oracle_point(xv[k], dyv ? dyv[k] : 0.0, A + ORC_NA * g,
                           B + ORC_NB * g, out + (long)ORC_NOUT * k);
    }
    return 0;
}
