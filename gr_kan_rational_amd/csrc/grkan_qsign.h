// grkan_qsign.h -- the sign of q(x) = b_1 + b_2 x + ... + b_N x^(N-1) for
// fp32 x and b.
//
// The backward of F = P / (1 + |Q|) needs s = sign(Q), Q = x q(x), for the
// derivative of |Q| (FlashKAT Paper-Notes page, arXiv 2505.13813, section
// "KAT 的突破与残留问题": the safe-PAU form and its gradients with respect to x,
// a and b).  Almost every element proves its sign from the fp64 value of Q;
// these routines decide the rest (x within rounding of a root of q), so they
// are cold code, written for registers, not speed.
//
// qsign_integer, exact.  Every finite fp32 value is an integer times a power
// of two: x = +-X 2^e and b_j = B_j 2^(f_j) with |X|, |B_j| < 2^24.  Hence
//     q(x) = 2^G sum_j C_j X^(j-1),   C_j = +-B_j 2^(d_j),
// with g_j = f_j + (j-1) e, G = min_j g_j over the nonzero b_j, d_j = g_j - G
// >= 0 and the sign of C_j that of b_j times sign(x)^(j-1).  The sum is an
// integer; Horner's rule over it in kQSignWords 32-bit words of two's
// complement (S <- S X + C_j) gives it exactly whenever every |C_j X^(j-1)|
// stays below 2^(32 kQSignWords - 4), which is checked before from the bit
// lengths.  That holds whenever the aligned terms span fewer bits than the
// window: at fp32's 24-bit mantissas, |x| = 3 and degree N - 1 = 5 they span
// about 150 bits; the window fails only for |x| far from 1 at high degree
// (below ~2^-20 at degree 5) or for coefficients far apart in magnitude, and
// the caller then keeps the sign of its fp64 evaluation of Q.
//
// qsign_compensated: compensated Horner in fp64 (Graillat, Langlois & Louvet,
// "Compensated Horner scheme", 2005), about twice fp64's precision: right
// unless |q(x)| < ~2^-100 sum_j |b_j x^(j-1)|.  Next to a 5-fold root of a
// degree-5 q that happens (at the fp32 neighbours of 2.75 the sign sits
// ~2^-117 below the terms), so the kernels use it only for N <= 4, where no
// such input was found among clustered and exact roots, and qsign_integer
// above that.
#pragma once

#include <stdint.h>

#ifdef __HIPCC__
#define GRKAN_QS_HD __host__ __device__
#else
#define GRKAN_QS_HD
#endif

namespace grkan {

constexpr int kQSignWords = 8;  // 256-bit window

GRKAN_QS_HD inline uint32_t qs_bits(float f) {
    uint32_t u;
    __builtin_memcpy(&u, &f, sizeof u);
    return u;
}

// |f| = m 2^e with m odd (f finite and nonzero); returns the sign of f.
GRKAN_QS_HD inline int qs_split(float f, uint32_t &m, int &e) {
    const uint32_t u = qs_bits(f);
    const uint32_t ef = (u >> 23) & 0xffu;
    const uint32_t mf = u & 0x7fffffu;
    m = ef ? (mf | 0x800000u) : mf;
    e = ef ? (int)ef - 150 : -149;
    const int tz = __builtin_ctz(m);
    m >>= tz;
    e += tz;
    return (u >> 31) ? -1 : 1;
}

GRKAN_QS_HD inline int qs_bitlen(uint32_t m) { return 32 - __builtin_clz(m); }

// Exact sign of q(x) by integer Horner (see the header comment).  Returns
// false, leaving s alone, when x or a coefficient is not finite or the terms
// do not fit the window.
template <int N>
GRKAN_QS_HD inline bool qsign_integer(float x, const float (&b)[N], int &s) {
    static_assert(N >= 1 && N <= 8, "denominator degree");
    constexpr int kBits = 32 * kQSignWords;
    if ((qs_bits(x) & 0x7f800000u) == 0x7f800000u) return false;  // Inf, NaN
#pragma unroll
    for (int j = 0; j < N; ++j)
        if ((qs_bits(b[j]) & 0x7f800000u) == 0x7f800000u) return false;
    if (x == 0.0f) {  // q(0) = b_1
        s = (b[0] > 0.0f) - (b[0] < 0.0f);
        return true;
    }
    uint32_t X;
    int e;
    const int sx = qs_split(x, X, e);
    const int lx = qs_bitlen(X);
    // G = min_j g_j over the nonzero b_j; the per-coefficient values are
    // formed again in each pass below rather than kept, to hold few registers.
    int G = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < N; ++j) {
        if (b[j] == 0.0f) continue;
        uint32_t B;
        int f;
        qs_split(b[j], B, f);
        const int g = f + j * e;
        G = g < G ? g : G;
    }
    if (G == 0x7fffffff) {  // b = 0
        s = 0;
        return true;
    }
    // Window check: |C_j X^(j-1)| < 2^(bitlen(B_j) + d_j + (j-1) bitlen(X)).
    // The N <= 8 terms then sum to below 2^(max + 3); every Horner partial sum
    // is bounded by the same (X >= 1), so kBits - 1 bits of magnitude suffice.
#pragma unroll
    for (int j = 0; j < N; ++j) {
        if (b[j] == 0.0f) continue;
        uint32_t B;
        int f;
        qs_split(b[j], B, f);
        if (qs_bitlen(B) + (f + j * e - G) + j * lx + 3 > kBits - 1) return false;
    }
    uint32_t S[kQSignWords];
#pragma unroll
    for (int i = 0; i < kQSignWords; ++i) S[i] = 0u;
#pragma unroll
    for (int j = N - 1; j >= 0; --j) {
        // S <- S X (mod 2^kBits; exact, as the true product fits)
        uint32_t carry = 0u;
#pragma unroll
        for (int i = 0; i < kQSignWords; ++i) {
            const uint64_t t = (uint64_t)S[i] * X + carry;
            S[i] = (uint32_t)t;
            carry = (uint32_t)(t >> 32);
        }
        if (b[j] == 0.0f) continue;
        // S <- S + C_j, C_j = +-B_j 2^(d_j) with d_j = 32 w + r < kBits
        uint32_t B;
        int f;
        const int sb = qs_split(b[j], B, f);
        const bool neg = (sb * ((j & 1) ? sx : 1)) < 0;
        const int d = f + j * e - G;
        const int w = d >> 5;
        const uint64_t mag = (uint64_t)B << (d & 31);  // < 2^55
        const uint64_t v = neg ? (uint64_t)0 - mag : mag;
        const uint32_t v0 = (uint32_t)v, v1 = (uint32_t)(v >> 32);
        const uint32_t ext = neg ? 0xffffffffu : 0u;
        uint32_t c = 0u;
#pragma unroll
        for (int i = 0; i < kQSignWords; ++i) {
            const uint32_t a = (i < w) ? 0u : (i == w) ? v0 : (i == w + 1) ? v1 : ext;
            const uint64_t t = (uint64_t)S[i] + a + c;
            S[i] = (uint32_t)t;
            c = (uint32_t)(t >> 32);
        }
    }
    uint32_t nz = 0u;
#pragma unroll
    for (int i = 0; i < kQSignWords; ++i) nz |= S[i];
    s = ((int32_t)S[kQSignWords - 1] < 0) ? -1 : (nz ? 1 : 0);
    return true;
}

// Sign of compensated Horner's value of q(x) in fp64.
template <int N>
GRKAN_QS_HD inline int qsign_compensated(float xf, const float (&b)[N]) {
    // The error-free transformations need every product and sum rounded on its
    // own: no contraction of s*x + b into one FMA.
#pragma clang fp contract(off)
    static_assert(N >= 1, "denominator degree");
    const double x = (double)xf;
    double s = (double)b[N - 1];
    double c = 0.0;
#pragma unroll
    for (int j = N - 2; j >= 0; --j) {
        const double p = s * x;
        const double pe = __builtin_fma(s, x, -p);  // s*x = p + pe exactly
        const double t = p + (double)b[j];
        const double bb = t - p;
        const double te = (p - (t - bb)) + ((double)b[j] - bb);  // p + b = t + te exactly
        s = t;
        c = __builtin_fma(c, x, pe + te);
    }
    const double q = s + c;
    return (q > 0.0) - (q < 0.0);
}

}  // namespace grkan
