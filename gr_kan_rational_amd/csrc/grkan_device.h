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
    float a[kNumA];       // a_0..a_5
    float da[kNumA - 1];  // i * a_i, i = 1..5   (P')
    float b[kNumB];       // b_1..b_4
    float db[kNumB];      // j * b_j, j = 1..4   (Q')
    float kguard;         // 2^-18 * (|b_1| + .. + |b_4|): rounding guard of sign(Q)
    bool q_zero;          // b_1 = .. = b_4 = 0: Q vanishes identically, s = 0
};

// The sign guard.  The fp32 Q below differs from the exact Q(x) by at most
// about 6 * 2^-24 * sum_j |b_j| |x|^j, and sum_j |b_j| |x|^j is at most
// (sum_j |b_j|) * (|x| + x^4).  So |Q| > 2^-18 (sum_j |b_j|) (|x| + x^4)
// -- ten times that bound -- proves Q != 0 and sign(fl(Q)) = sign(Q).
constexpr float kSignGuard = 1.0f / 262144.0f;

__device__ static inline BwdCoefs derive(const Coefs &c) {
    BwdCoefs k;
#pragma unroll
    for (int i = 0; i < kNumA; ++i) k.a[i] = c.a[i];
#pragma unroll
    for (int i = 1; i < kNumA; ++i) k.da[i - 1] = (float)i * c.a[i];
    float bsum = 0.0f;
#pragma unroll
    for (int j = 0; j < kNumB; ++j) {
        k.b[j] = c.b[j];
        k.db[j] = (float)(j + 1) * c.b[j];
        bsum += fabsf(c.b[j]);
    }
    k.kguard = kSignGuard * bsum;
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

// Everything the backward needs about one element, fast fp32 evaluation.
// s = sign(Q) is taken from the fp32 Q; `sure` says whether the guard proves
// that sign right.  When it does not (x == 0, x within rounding of a root of
// Q, NaN), the element still gets the fp32 sign here and exact_fix() later
// swaps in the exact one.  One function so that the hot loop and the fix
// agree bit for bit.
struct ElemBwd {
    float dx;   // dY (P'/D - s P Q'/D^2)
    float w;    // dY / D          (dA terms: w x^i)
    float v;    // dY P / D^2
    float sv;   // s v             (dB terms: -sv x^j)
    float Qd;   // Q'
    float wPd;  // w P'
    bool sure;
};

__device__ static inline ElemBwd backward_element(float x, float x2, float x3, float x4, float x5,
                                                  float dy, const BwdCoefs &k) {
    const float P = fmaf(k.a[5], x5, fmaf(k.a[4], x4, fmaf(k.a[3], x3, fmaf(k.a[2], x2,
                    fmaf(k.a[1], x, k.a[0])))));
    const float Pd = fmaf(k.da[4], x4, fmaf(k.da[3], x3, fmaf(k.da[2], x2, fmaf(k.da[1], x, k.da[0]))));
    const float q = fmaf(k.b[3], x3, fmaf(k.b[2], x2, fmaf(k.b[1], x, k.b[0])));
    const float Qd = fmaf(k.db[3], x3, fmaf(k.db[2], x2, fmaf(k.db[1], x, k.db[0])));
    const float Q = x * q;
    const float r = __builtin_amdgcn_rcpf(1.0f + fabsf(Q));
    ElemBwd e;
    e.w = dy * r;
    e.v = e.w * (P * r);
    e.sv = __uint_as_float(__float_as_uint(e.v) ^ (__float_as_uint(Q) & 0x80000000u));
    e.sure = fabsf(Q) > k.kguard * (fabsf(x) + x4);
    e.Qd = Qd;
    e.wPd = e.w * Pd;
    e.dx = fmaf(-e.sv, Qd, e.wPd);
    return e;
}

// Adds one element's ten gradient terms (dA: w x^i; dB: -sv x^j) to acc.
__device__ static inline void accumulate(float w, float sv, float x, float x2, float x3, float x4,
                                         float x5, float (&acc)[kNumCoef]) {
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
}

// For an element whose sign was not proven: recomputes it, decides
// s = sign(x) sign(q(x)) exactly (0 at x == 0), replaces the dB terms that
// were accumulated with the fp32 sign and returns the exact dX.
__device__ static inline float exact_fix(float x, float dy, const BwdCoefs &k, float (&acc)[kNumCoef]) {
    const float x2 = x * x, x3 = x2 * x, x4 = x2 * x2, x5 = x4 * x;
    const ElemBwd e = backward_element(x, x2, x3, x4, x5, dy, k);
    if (e.sure) return e.dx;
    const int s = (x == 0.0f || k.q_zero) ? 0 : sign_q_exact(x, k) * ((x > 0.0f) ? 1 : -1);
    const float sv = (s == 0) ? 0.0f : ((s > 0) ? e.v : -e.v);
    const float diff = e.sv - sv;  // undo -e.sv x^j, add -sv x^j
    acc[6] = fmaf(diff, x, acc[6]);
    acc[7] = fmaf(diff, x2, acc[7]);
    acc[8] = fmaf(diff, x3, acc[8]);
    acc[9] = fmaf(diff, x4, acc[9]);
    return fmaf(-sv, e.Qd, e.wPd);
}

}  // namespace grkan
