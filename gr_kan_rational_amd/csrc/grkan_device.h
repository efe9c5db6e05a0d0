// grkan_device.h -- device-side building blocks of the GR-KAN kernels (gfx950).
//
// Pages cited
//   [FlashKAT notes]  "FlashKAT: Understanding and Addressing Performance
//                     Bottlenecks in the Kolmogorov-Arnold Transformer",
//                     Paper-Notes page (AAAI 2026), arXiv 2505.13813.
//
// The activation is F(x) = P(x) / (1 + |Q(x)|) with P of degree 5 (a_0..a_5)
// and Q of degree 4 without constant term (b_1..b_4), one coefficient set per
// channel group ([FlashKAT notes], sections "KAT 的突破与残留问题" and
// "损失函数 / 训练策略").  Everything here is fp32 register arithmetic; the
// only fp64 use is (a) the carry of the long gradient sums and (b) deciding
// the sign of Q for the rare element whose fp32 Q is within rounding of 0.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace grkan {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kNumA = 6;             // a_0..a_5
constexpr int kNumB = 4;             // b_1..b_4
constexpr int kNumCoef = kNumA + kNumB;

// Tag type for bf16 storage (values are handled as fp32 in registers).
struct bf16io {};

// One 16-byte global access worth of I/O elements.
template <class T> struct Io;

template <> struct Io<float> {
    static constexpr int kElems = 4;
    __device__ static inline void unpack(const u32x4 v, float (&f)[kElems]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v[i]);
    }
    __device__ static inline u32x4 pack(const float (&f)[kElems]) {
        u32x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = __float_as_uint(f[i]);
        return v;
    }
};

template <> struct Io<bf16io> {
    static constexpr int kElems = 8;
    // bf16 -> fp32 is exact: the bf16 bits are the top half of the fp32 bits.
    __device__ static inline void unpack(const u32x4 v, float (&f)[kElems]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(v[i] << 16);
            f[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
        }
    }
    // fp32 -> bf16 rounds to nearest even (gfx950 v_cvt_pk_bf16_f32).
    __device__ static inline u32x4 pack(const float (&f)[kElems]) {
        u32x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f32x2 p = {f[2 * i], f[2 * i + 1]};
            bf16x2 h = __builtin_convertvector(p, bf16x2);
            v[i] = __builtin_bit_cast(unsigned int, h);
        }
        return v;
    }
};

template <bool NT>
__device__ static inline u32x4 load16(const u32x4 *p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}
template <bool NT>
__device__ static inline void store16(u32x4 *p, u32x4 v) {
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

// Coefficients of one group.  Loaded with uniform addresses, so they live in
// scalar registers; the derived constants below are computed once per
// workgroup.
struct Coefs {
    float a[kNumA];
    float b[kNumB];
};

__device__ static inline Coefs load_coefs(const float *__restrict__ A, const float *__restrict__ B,
                                          int g) {
    Coefs c;
#pragma unroll
    for (int i = 0; i < kNumA; ++i) c.a[i] = A[g * kNumA + i];
#pragma unroll
    for (int j = 0; j < kNumB; ++j) c.b[j] = B[g * kNumB + j];
    return c;
}

// Forward value, Horner form: 5 + 3 FMA, 1 mul, 1 add, 1 reciprocal, 1 mul.
// D >= 1, so the hardware reciprocal (1 ulp) cannot under- or overflow.
__device__ static inline float rational(float x, const Coefs &c) {
    float P = fmaf(fmaf(fmaf(fmaf(fmaf(c.a[5], x, c.a[4]), x, c.a[3]), x, c.a[2]), x, c.a[1]), x,
                   c.a[0]);
    float q = fmaf(fmaf(fmaf(c.b[3], x, c.b[2]), x, c.b[1]), x, c.b[0]);
    float D = 1.0f + fabsf(x * q);
    return P * __builtin_amdgcn_rcpf(D);
}

// Constants of the backward pass derived from one group's coefficients.
struct BwdCoefs {
    float a[kNumA];     // a_0..a_5
    float da[kNumA - 1];  // i * a_i, i = 1..5   (P')
    float b[kNumB];     // b_1..b_4
    float db[kNumB];    // j * b_j, j = 1..4   (Q')
    float kb[kNumB];    // 2^-18 |b_j|: rounding guard of the sign of Q
    bool q_zero;        // b_1 = .. = b_4 = 0: Q vanishes identically, s = 0
};

// Margin of the sign guard: |fl(q) - q| stays below ~5 * 2^-24 * sum|b_j||x|^(j-1)
// for the evaluation order used here; 2^-18 leaves a factor > 10 of slack.
constexpr float kSignGuard = 1.0f / 262144.0f;

__device__ static inline BwdCoefs derive(const Coefs &c) {
    BwdCoefs k;
#pragma unroll
    for (int i = 0; i < kNumA; ++i) k.a[i] = c.a[i];
#pragma unroll
    for (int i = 1; i < kNumA; ++i) k.da[i - 1] = (float)i * c.a[i];
#pragma unroll
    for (int j = 0; j < kNumB; ++j) {
        k.b[j] = c.b[j];
        k.db[j] = (float)(j + 1) * c.b[j];
        k.kb[j] = kSignGuard * fabsf(c.b[j]);
    }
    k.q_zero = (c.b[0] == 0.0f) && (c.b[1] == 0.0f) && (c.b[2] == 0.0f) && (c.b[3] == 0.0f);
    return k;
}

// sign of q(x) = b_1 + b_2 x + b_3 x^2 + b_4 x^3 by compensated Horner in fp64
// (error-free products by FMA and error-free sums; Graillat, Langlois & Louvet,
// "Compensated Horner scheme", 2005).  The result carries about twice fp64's
// precision, enough to fix the sign of every fp32 x that is not an exact root.
__device__ static inline int sign_q_exact(float xf, const BwdCoefs &k) {
    // The error-free transformations need every product and sum rounded on its
    // own: no contraction of s*x + b into one FMA.
#pragma clang fp contract(off)
    const double x = (double)xf;
    double s = (double)k.b[3];
    double c = 0.0;
#pragma unroll
    for (int j = 2; j >= 0; --j) {
        double p = s * x;
        double pe = fma(s, x, -p);         // s*x = p + pe exactly
        double t = p + (double)k.b[j];
        double bb = t - p;
        double te = (p - (t - bb)) + ((double)k.b[j] - bb);  // p + b = t + te exactly
        s = t;
        c = fma(c, x, pe + te);
    }
    double q = s + c;
    return (q > 0.0) - (q < 0.0);
}

// Q(x) = x q(x) in fp32 and its rounding scale 2^-18 * sum_j |b_j| |x|^j.
// When |Q| is above the scale, Q != 0 and the fp32 sign of Q is the true one.
// The backward pass and its correction pass both decide through this one
// function, so they always agree on which elements are guarded.
struct QGuard {
    float Q;
    bool sure;
};
__device__ static inline QGuard q_guard(float x, float x2, float x3, const BwdCoefs &k) {
    const float q = fmaf(k.b[3], x3, fmaf(k.b[2], x2, fmaf(k.b[1], x, k.b[0])));
    const float Q = x * q;
    const float ax = fabsf(x);
    const float guard = ax * fmaf(k.kb[3], fabsf(x3), fmaf(k.kb[2], x2, fmaf(k.kb[1], ax, k.kb[0])));
    return QGuard{Q, fabsf(Q) > guard};
}

// Per-element backward, fast part.  Returns dX and adds the element's ten
// gradient terms into acc (dA terms dY x^i / D, then dB terms -dY s P x^j / D^2).
//
// s = sign(Q) is taken from the fp32 Q when q_guard() is sure of it.
// Otherwise -- x == 0, a group with b = 0, x within rounding of a root of Q,
// NaN -- the element is computed with s = 0 and *guarded* is set; the caller
// later applies exact_sign_terms() to add the s-terms with the exact sign.
// The hot loop thus has no data-dependent branch and a small register
// footprint.
__device__ static inline float backward_element(float x, float dy, const BwdCoefs &k,
                                                float (&acc)[kNumCoef], bool &guarded) {
    const float x2 = x * x;
    const float x3 = x2 * x;
    const float x4 = x2 * x2;
    const float x5 = x4 * x;
    const float P = fmaf(k.a[5], x5, fmaf(k.a[4], x4, fmaf(k.a[3], x3, fmaf(k.a[2], x2,
                    fmaf(k.a[1], x, k.a[0])))));
    const float Pd = fmaf(k.da[4], x4, fmaf(k.da[3], x3, fmaf(k.da[2], x2, fmaf(k.da[1], x, k.da[0]))));
    const float Qd = fmaf(k.db[3], x3, fmaf(k.db[2], x2, fmaf(k.db[1], x, k.db[0])));
    const QGuard qg = q_guard(x, x2, x3, k);
    const float r = __builtin_amdgcn_rcpf(1.0f + fabsf(qg.Q));
    const float w = dy * r;      // dY / D
    const float v = w * (P * r); // dY P / D^2
    guarded = !qg.sure;
    const float sv_fast = __uint_as_float(__float_as_uint(v) ^ (__float_as_uint(qg.Q) & 0x80000000u));
    const float sv = qg.sure ? sv_fast : 0.0f;   // s * v
    acc[0] += w;
    acc[1] = fmaf(w, x, acc[1]);
    acc[2] = fmaf(w, x2, acc[2]);
    acc[3] = fmaf(w, x3, acc[3]);
    acc[4] = fmaf(w, x4, acc[4]);
    acc[5] = fmaf(w, x5, acc[5]);
    acc[6] = fmaf(-sv, x, acc[6]);
    acc[7] = fmaf(-sv, x2, acc[7]);
    acc[8] = fmaf(-sv, x3, acc[8]);
    acc[9] = fmaf(-sv, x4, acc[9]);
    return fmaf(-sv, Qd, w * Pd);
}

// The s-terms a guarded element is missing, with s = sign(x) sign(q(x))
// decided exactly (Q is exactly 0 at x = 0 and for a group with b = 0).
// Returns false when s = 0 (nothing to add); otherwise sets ddx (to add to
// dX) and tb[0..3] (to add to the dB sums).
__device__ static inline bool exact_sign_terms(float x, float dy, const BwdCoefs &k, float &ddx,
                                               float (&tb)[kNumB]) {
    if (x == 0.0f || k.q_zero) return false;
    const int s = sign_q_exact(x, k) * ((x > 0.0f) ? 1 : -1);
    if (s == 0) return false;
    const float x2 = x * x;
    const float x3 = x2 * x;
    const float x4 = x2 * x2;
    const float x5 = x4 * x;
    const float P = fmaf(k.a[5], x5, fmaf(k.a[4], x4, fmaf(k.a[3], x3, fmaf(k.a[2], x2,
                    fmaf(k.a[1], x, k.a[0])))));
    const float Qd = fmaf(k.db[3], x3, fmaf(k.db[2], x2, fmaf(k.db[1], x, k.db[0])));
    const QGuard qg = q_guard(x, x2, x3, k);
    const float r = __builtin_amdgcn_rcpf(1.0f + fabsf(qg.Q));
    const float v = (dy * r) * (P * r);
    const float sv = (s > 0) ? v : -v;
    tb[0] = -sv * x;
    tb[1] = -sv * x2;
    tb[2] = -sv * x3;
    tb[3] = -sv * x4;
    ddx = -sv * Qd;
    return true;
}

}  // namespace grkan
