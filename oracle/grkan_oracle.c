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
 * Other degrees (the PAU family).  The pages state that the same kernel
 * restructuring carries over to PAU and its variants ([FlashKAT notes],
 * section "局限性与未来工作"; PAU is the rational unit P/(1 + |Q|) with free
 * degrees).  Every routine here therefore takes the numerator degree m and
 * the denominator degree n: a_0..a_m and b_1..b_n per group, m + n + 1
 * gradient sums.  GR-KAN is m = 5, n = 4; n = 0 is a plain polynomial
 * (Q = 0, D = 1, s = 0).
 *
 * How: powers by repeated multiplication, polynomial values as plain sums in
 * ascending order (deliberately not Horner), one division per quotient.
 * sign(Q) is taken from the fp64 value unless |Q| is within the fp64
 * rounding bound of zero; then it is decided exactly: every term b_j x^j is
 * formed as a floating-point expansion (a sum of doubles with no rounding
 * error, built with the error-free transformations TwoSum and TwoProduct)
 * and the terms are added as expansions, after Shewchuk, "Adaptive Precision
 * Floating-Point Arithmetic and Fast Robust Geometric Predicates" (1997).
 * The sign of the exact sum is that of its largest component, so the sign is
 * exact for every input whose products stay clear of fp64 underflow.  Group
 * sums are accumulated in long double, row by row in index order.
 */
#include <math.h>
#include <float.h>
#include <stddef.h>
#include <stdio.h>
#include <stdlib.h>

#define ORC_MAXDEG 15 /* largest numerator or denominator degree accepted */

/* Per-element record written by grkan_oracle_point (doubles, in order). */
enum {
    ORC_F = 0,      /* F(x)                                              */
    ORC_DX = 1,     /* dY * dF/dx                                        */
    ORC_FMAG = 2,   /* first-order rounding scale of F  (see below)      */
    ORC_DXMAG = 3,  /* first-order rounding scale of dX                  */
    ORC_SIGN = 4,   /* s = sign(Q) as -1, 0, +1                          */
    ORC_D = 5,      /* D = 1 + |Q|                                       */
    ORC_T = 6       /* m+1 terms dY dF/da_i = dY x^i / D, then           */
                    /* n terms dY dF/db_j = -dY s P x^j / D^2, then       */
                    /* the first-order rounding scale of each of them     */
};

/* Record length for degrees (m, n). */
int grkan_oracle_nout(int m, int n) { return ORC_T + 2 * (m + 1 + n); }

static int sign_of(double v) { return (v > 0.0) - (v < 0.0); }

/* ---- exact sign of Q by expansion arithmetic (Shewchuk 1997) ---------- */

/* a + b = s + e exactly (Knuth's TwoSum). */
static void two_sum(double a, double b, double *s, double *e)
{
    double x = a + b;
    double bv = x - a;
    double av = x - bv;
    *s = x;
    *e = (a - av) + (b - bv);
}

/* a * b = p + e exactly (TwoProduct with a fused multiply-add). */
static void two_prod(double a, double b, double *p, double *e)
{
    double x = a * b;
    *p = x;
    *e = fma(a, b, -x);
}

/* h = e * b for an expansion e (components in increasing magnitude, no
 * zeros); returns the length of h, zeros removed (Shewchuk's
 * SCALE-EXPANSION-ZEROELIM). */
static int scale_expansion(int elen, const double *e, double b, double *h)
{
    double q, hh, p1, p0, sum;
    int hi = 0;
    two_prod(e[0], b, &q, &hh);
    if (hh != 0.0)
        h[hi++] = hh;
    for (int i = 1; i < elen; ++i) {
        two_prod(e[i], b, &p1, &p0);
        two_sum(q, p0, &sum, &hh);
        if (hh != 0.0)
            h[hi++] = hh;
        two_sum(p1, sum, &q, &hh);
        if (hh != 0.0)
            h[hi++] = hh;
    }
    if (q != 0.0 || hi == 0)
        h[hi++] = q;
    return hi;
}

/* h = e + f (Shewchuk's EXPANSION-SUM-ZEROELIM1: add f's components one
 * at a time with GROW-EXPANSION, then drop zeros). */
static int expansion_sum(int elen, const double *e, int flen, const double *f, double *h)
{
    int hlen = elen;
    for (int i = 0; i < elen; ++i)
        h[i] = e[i];
    for (int i = 0; i < flen; ++i) {
        double q = f[i], hh;
        for (int j = 0; j < hlen; ++j) {
            two_sum(q, h[j], &q, &hh);
            h[j] = hh;
        }
        h[hlen++] = q;
    }
    int k = 0;
    for (int i = 0; i < hlen; ++i)
        if (h[i] != 0.0)
            h[k++] = h[i];
    if (k == 0)
        h[k++] = 0.0;
    return k;
}

#define ORC_EXP 4096 /* room for every expansion below at degree <= ORC_MAXDEG */

/* sign(Q(x)), Q(x) = sum_{j=1..n} b_j x^j, exactly: x^j and b_j x^j as
 * expansions, summed as expansions; the sign of a nonoverlapping expansion
 * is the sign of its largest (last) component. */
static int sign_q_exact(double x, int n, const double *b)
{
    static _Thread_local double pw[ORC_EXP], term[ORC_EXP], acc[ORC_EXP], tmp[ORC_EXP];
    int plen = 1, alen = 1;
    pw[0] = 1.0;
    acc[0] = 0.0;
    for (int j = 1; j <= n; ++j) {
        if (4 * plen + alen > ORC_EXP) { /* cannot happen for degrees <= ORC_MAXDEG */
            fprintf(stderr, "grkan_oracle: expansion overflow in sign_q_exact\n");
            abort();
        }
        int l = scale_expansion(plen, pw, x, tmp);
        for (int i = 0; i < l; ++i)
            pw[i] = tmp[i];
        plen = l;
        int tl = scale_expansion(plen, pw, b[j - 1], term);
        alen = expansion_sum(alen, acc, tl, term, tmp);
        for (int i = 0; i < alen; ++i)
            acc[i] = tmp[i];
    }
    return sign_of(acc[alen - 1]);
}

/* sign(Q(x)) from the fp64 value q when its rounding bound allows, else
 * exactly.  qabs = sum_j |b_j| |x|^j bounds the rounding error of q:
 * |q - Q| <= (2n + 2) eps qabs for the ascending sum of products used here,
 * so the factor below leaves a wide margin. */
static int sign_q(double x, int n, const double *b, double q, double qabs)
{
    /* Non-finite x, or terms that overflow fp64 (|x| beyond ~1e300 / |b|):
     * no exact evaluation exists; the sign is IEEE's, that of q (0 for NaN),
     * and the outputs propagate as IEEE arithmetic does (the pages are
     * silent on such inputs). */
    if (!isfinite(q) || !isfinite(qabs))
        return sign_of(q);
    if (fabs(q) > (8.0 * n + 16.0) * DBL_EPSILON * qabs)
        return sign_of(q);
    return sign_q_exact(x, n, b);
}

/*
 * One element.  a[m+1] = a_0..a_m, b[n] = b_1..b_n (0 <= m, n <= 15);
 * out: grkan_oracle_nout(m, n) doubles.
 *
 * The magnitude fields are the first-order error scale of an fp32
 * evaluation of the same quantity (sums of absolute values of every term,
 * propagated through the quotient): a correctly implemented fp32 kernel
 * differs from F and dX by a small multiple of 2^-24 times these, which is
 * what the comparator scales its relative tolerance by where F or dX is
 * itself close to zero.  The same holds for each gradient term: dY x^i / D
 * inherits D's rounding (scale |dY| |x|^i (1 + Qabs/D) / D) and
 * -dY s P x^j / D^2 that of P and D^2 (scale |dY| |x|^j (Pabs +
 * 2 |P| Qabs / D) / D^2), where Pabs, Qabs are P and Q evaluated with
 * absolute values.  Near a root of Q whose terms are large (high degree,
 * large |x|), these scales exceed |term| by orders of magnitude.
 */
void grkan_oracle_point(double x, double dy, int m, int n, const double *a,
                        const double *b, double *out)
{
    const int top = m > n ? m : n;
    double xp[ORC_MAXDEG + 1], axp[ORC_MAXDEG + 1];
    double ax = fabs(x);
    xp[0] = 1.0;
    axp[0] = 1.0;
    for (int i = 1; i <= top; ++i) {
        xp[i] = xp[i - 1] * x;
        axp[i] = axp[i - 1] * ax;
    }

    double P = 0, Pd = 0, Pabs = 0, Pdabs = 0;
    for (int i = 0; i <= m; ++i) {
        P += a[i] * xp[i];
        Pabs += fabs(a[i]) * axp[i];
    }
    for (int i = 1; i <= m; ++i) {
        Pd += (double)i * a[i] * xp[i - 1];
        Pdabs += (double)i * fabs(a[i]) * axp[i - 1];
    }
    double Q = 0, Qd = 0, Qabs = 0, Qdabs = 0;
    for (int j = 1; j <= n; ++j) {
        Q += b[j - 1] * xp[j];
        Qabs += fabs(b[j - 1]) * axp[j];
        Qd += (double)j * b[j - 1] * xp[j - 1];
        Qdabs += (double)j * fabs(b[j - 1]) * axp[j - 1];
    }
    int s = n > 0 ? sign_q(x, n, b, Q, Qabs) : 0;
    double D = 1.0 + fabs(Q);
    double D2 = D * D;

    double F = P / D;
    double dFdx = Pd / D - (double)s * P * Qd / D2;
    out[ORC_F] = F;
    out[ORC_DX] = dy * dFdx;
    const int nk = m + 1 + n;
    double ady = fabs(dy), aP = fabs(P), aPd = fabs(Pd), aQd = fabs(Qd);
    for (int i = 0; i <= m; ++i) {
        out[ORC_T + i] = dy * xp[i] / D;
        out[ORC_T + nk + i] = ady * axp[i] * (1.0 + Qabs / D) / D;
    }
    for (int j = 1; j <= n; ++j) {
        out[ORC_T + m + j] = -dy * (double)s * P * xp[j] / D2;
        out[ORC_T + nk + m + j] = ady * axp[j] * (Pabs + 2.0 * aP * Qabs / D) / D2;
    }

    out[ORC_FMAG] = (Pabs + aP * Qabs / D) / D;
    out[ORC_DXMAG] = ady * ((Pdabs + aPd * Qabs / D) / D
                                 + (Pabs * aQd + aP * Qdabs + 2.0 * aP * aQd * Qabs / D) / D2);
    out[ORC_SIGN] = (double)s;
    out[ORC_D] = D;
}

static int bad_degrees(int m, int n)
{
    return m < 0 || n < 0 || m > ORC_MAXDEG || n > ORC_MAXDEG;
}

/*
 * Rows [0, rows) of a row-major [rows][d] block.  x, dy: fp64 copies of the
 * inputs.  A: [n_g][m+1], B: [n_g][n] (fp64 copies of the fp32
 * coefficients).  Any output pointer may be NULL to skip it.
 *   y, ymag, dx, dxmag  : [rows][d]
 *   sums, sumsq, magsq  : [n_g][m+1+n], accumulated into (+=), long double
 *                         internally; sums[g][k] += the group's terms,
 *                         sumsq[g][k] += their squares and magsq[g][k] +=
 *                         the squares of their rounding scales (the L2
 *                         norms the comparator scales its tolerance by).
 * dy may be NULL for a forward-only call (then dx, dxmag, sums, sumsq, magsq
 * must be NULL too).  Returns 0, or -1 on a bad shape or degree.
 */
int grkan_oracle_rows(const double *x, const double *dy, long rows, long d,
                      int n_g, int m, int n, const double *A, const double *B,
                      double *y, double *ymag, double *dx, double *dxmag,
                      double *sums, double *sumsq, double *magsq)
{
    if (rows < 0 || d <= 0 || n_g <= 0 || d % n_g != 0 || bad_degrees(m, n))
        return -1;
    if (dy == NULL && (dx || dxmag || sums || sumsq || magsq))
        return -1;
    long dg = d / n_g;
    const int nk = m + 1 + n;
    long double acc[2 * ORC_MAXDEG + 1], acc2[2 * ORC_MAXDEG + 1], acc3[2 * ORC_MAXDEG + 1];
    double out[ORC_T + 2 * (2 * ORC_MAXDEG + 1)];
    for (int g = 0; g < n_g; ++g) {
        for (int k = 0; k < nk; ++k)
            acc[k] = acc2[k] = acc3[k] = 0.0L;
        for (long r = 0; r < rows; ++r) {
            for (long c = g * dg; c < (g + 1) * dg; ++c) {
                long idx = r * d + c;
                grkan_oracle_point(x[idx], dy ? dy[idx] : 0.0, m, n,
                                   A + (long)(m + 1) * g, B + (long)n * g, out);
                if (y)
                    y[idx] = out[ORC_F];
                if (ymag)
                    ymag[idx] = out[ORC_FMAG];
                if (dx)
                    dx[idx] = out[ORC_DX];
                if (dxmag)
                    dxmag[idx] = out[ORC_DXMAG];
                for (int k = 0; k < nk; ++k) {
                    long double t = (long double)out[ORC_T + k];
                    long double u = (long double)out[ORC_T + nk + k];
                    acc[k] += t;
                    acc2[k] += t * t;
                    acc3[k] += u * u;
                }
            }
        }
        if (sums)
            for (int k = 0; k < nk; ++k)
                sums[g * nk + k] += (double)acc[k];
        if (sumsq)
            for (int k = 0; k < nk; ++k)
                sumsq[g * nk + k] += (double)acc2[k];
        if (magsq)
            for (int k = 0; k < nk; ++k)
                magsq[g * nk + k] += (double)acc3[k];
    }
    return 0;
}

/*
 * Selected elements of a [rows][d] tensor: idx[n_el] are flat indices,
 * xv/dyv the fp64 values at them (gathered by the caller).  Writes n_el
 * records of grkan_oracle_nout(m, n) doubles.
 */
int grkan_oracle_points(const double *xv, const double *dyv, const long *idx,
                        long n_el, long d, int n_g, int m, int n,
                        const double *A, const double *B, double *out)
{
    if (n_el < 0 || d <= 0 || n_g <= 0 || d % n_g != 0 || bad_degrees(m, n))
        return -1;
    long dg = d / n_g;
    const int nout = grkan_oracle_nout(m, n);
    for (long k = 0; k < n_el; ++k) {
        long c = idx[k] % d;
        int g = (int)(c / dg);
        grkan_oracle_point(xv[k], dyv ? dyv[k] : 0.0, m, n, A + (long)(m + 1) * g,
                           B + (long)n * g, out + (long)nout * k);
    }
    return 0;
}
