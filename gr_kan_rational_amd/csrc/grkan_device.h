// grkan_device.h -- device-side building blocks of the GR-KAN / PAU kernels
// (gfx950).
//
// Pages cited
//   [FlashKAT notes]  "FlashKAT: Understanding and Addressing Performance
//                     Bottlenecks in the Kolmogorov-Arnold Transformer",
//                     Paper-Notes page (AAAI 2026), arXiv 2505.13813.
//
// The activation is F(x) = P(x) / (1 + |Q(x)|) with P of degree M (a_0..a_M)
// and Q of degree N without constant term (b_1..b_N), one coefficient set per
// channel group.  GR-KAN is M = 5, N = 4 ([FlashKAT notes], sections "KAT 的
// 突破与残留问题" and "损失函数 / 训练策略"); the pages note that the same
// kernel restructuring applies to PAU and its variants (section "局限性与未来
// 工作"), i.e. to other (M, N), which the templates below cover.  N = 0 is a
// plain polynomial.  Everything here is fp32 register arithmetic except two
// fp64 uses in the backward: Q is evaluated in fp64 (see backward_element),
// and the sign of Q is decided again for the rare element whose Q is within
// rounding of 0 (exactly for N >= kExactSignMinN, by compensated Horner in
// fp64 below that).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "grkan_qsign.h"

namespace grkan {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

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

// ------------------------------------------------------------ windows
//
// The streaming kernels address each tensor through a window: a base pointer
// (uniform, in scalar registers) and a byte length, plus a 32-bit per-lane
// byte offset.  An access at an offset past the length is skipped -- a load
// gives zeros, a store does nothing -- which is how the kernels handle the
// ragged last row tile and ragged column parts with one code path.  Offsets
// stay below 2^31 and lengths at most 2^31, so kOffsetOutOfRange is past
// every window.  (Buffer-resource instructions do the same check in
// hardware, but streamed ~3% slower than plain global loads and stores at
// the KAT-B shapes on MI355X.)

struct Span {
    const char *p;
    uint32_t n;
};

constexpr uint32_t kOffsetOutOfRange = 0x80000000u;
constexpr int64_t kMaxWindow = int64_t(1) << 31;

// The window [base, base + min(bytes, 2^31)).
__device__ static inline Span make_span(const void *base, int64_t bytes) {
    const int64_t n = bytes < kMaxWindow ? bytes : kMaxWindow;
    return Span{static_cast<const char *>(base), (uint32_t)n};
}

// 16-byte accesses, non-temporal: the data is streamed once.  CHECK = false
// is for workgroups whose every access is known to be inside the window
// (full tiles, the vast majority): no compare, no branch.
template <bool CHECK>
__device__ static inline u32x4 win_load16(Span w, uint32_t off) {
    if (CHECK && off >= w.n) return u32x4{0u, 0u, 0u, 0u};
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(w.p + off));
}
template <bool CHECK>
__device__ static inline void win_store16(Span w, uint32_t off, u32x4 v) {
    if (CHECK && off >= w.n) return;
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(const_cast<char *>(w.p) + off));
}
// A second read of data already loaded once, through a volatile access so
// that the compiler issues it again instead of keeping the first load's
// registers live until this point (the rare exact-sign path of the backward).
template <bool CHECK>
__device__ static inline u32x4 win_reload16(Span w, uint32_t off) {
    if (CHECK && off >= w.n) return u32x4{0u, 0u, 0u, 0u};
    return *reinterpret_cast<const volatile u32x4 *>(w.p + off);
}

// One I/O element per access, for the narrow-group kernels (one channel
// column per lane): 4-byte fp32 or 2-byte bf16, non-temporal.
template <class T> struct Elem;
template <> struct Elem<float> {
    static constexpr int kBytes = 4;
    template <bool CHECK>
    __device__ static inline float load(Span w, uint32_t off) {
        if (CHECK && off >= w.n) return 0.0f;
        return __builtin_nontemporal_load(reinterpret_cast<const float *>(w.p + off));
    }
    template <bool CHECK>
    __device__ static inline void store(Span w, uint32_t off, float v) {
        if (CHECK && off >= w.n) return;
        __builtin_nontemporal_store(v, reinterpret_cast<float *>(const_cast<char *>(w.p) + off));
    }
};
template <> struct Elem<bf16io> {
    static constexpr int kBytes = 2;
    // bf16 -> fp32 is exact; fp32 -> bf16 rounds to nearest even.
    template <bool CHECK>
    __device__ static inline float load(Span w, uint32_t off) {
        if (CHECK && off >= w.n) return 0.0f;
        const unsigned short h = __builtin_nontemporal_load(reinterpret_cast<const unsigned short *>(w.p + off));
        return __uint_as_float((uint32_t)h << 16);
    }
    template <bool CHECK>
    __device__ static inline void store(Span w, uint32_t off, float v) {
        if (CHECK && off >= w.n) return;
        const __bf16 h = (__bf16)v;
        __builtin_nontemporal_store(__builtin_bit_cast(unsigned short, h),
                                    reinterpret_cast<unsigned short *>(const_cast<char *>(w.p) + off));
    }
};

// ------------------------------------------------------------ coefficients

template <int M, int N> struct Deg {
    static_assert(M >= 0 && N >= 0, "degrees");
    static constexpr int kNumA = M + 1;          // a_0..a_M
    static constexpr int kNumB = N;              // b_1..b_N
    static constexpr int kNumCoef = M + 1 + N;   // gradient sums per group
    static constexpr int kTop = M > N ? M : N;   // highest power of x needed
};

// Coefficients of one group.  Loaded with uniform addresses, so they live in
// scalar registers; the derived constants below are computed once per
// workgroup.
template <int M, int N> struct Coefs {
    float a[M + 1];
    float b[N > 0 ? N : 1];
};

template <int M, int N>
__device__ static inline Coefs<M, N> load_coefs(const float *__restrict__ A,
                                                const float *__restrict__ B, int g) {
    Coefs<M, N> c;
#pragma unroll
    for (int i = 0; i <= M; ++i) c.a[i] = A[g * (M + 1) + i];
#pragma unroll
    for (int j = 0; j < N; ++j) c.b[j] = B[g * N + j];
    if constexpr (N == 0) c.b[0] = 0.0f;
    return c;
}

// Forward value, Horner form: M + (N - 1) FMA, 1 mul, 1 add, 1 reciprocal,
// 1 mul.  D >= 1, so the hardware reciprocal (1 ulp) cannot under- or
// overflow.
template <int M, int N>
__device__ static inline float rational(float x, const Coefs<M, N> &c) {
    float P = c.a[M];
#pragma unroll
    for (int i = M - 1; i >= 0; --i) P = fmaf(P, x, c.a[i]);
    if constexpr (N == 0) {
        return P;
    } else {
        float q = c.b[N - 1];
#pragma unroll
        for (int j = N - 2; j >= 0; --j) q = fmaf(q, x, c.b[j]);
        const float D = 1.0f + fabsf(x * q);
        return P * __builtin_amdgcn_rcpf(D);
    }
}

// Powers x^0..x^K: even powers as squares, odd ones as x times the previous
// (for K = 5: x^2 = x x, x^3 = x^2 x, x^4 = x^2 x^2, x^5 = x^4 x).
template <int K> struct Pow {
    float p[K + 1];
    __device__ inline explicit Pow(float x) {
        p[0] = 1.0f;
        if constexpr (K >= 1) p[1] = x;
#pragma unroll
        for (int k = 2; k <= K; ++k) p[k] = (k % 2 == 0) ? p[k / 2] * p[k / 2] : p[k - 1] * x;
    }
};

// Exact fp64 value of an fp32 number, formed with integer operations only:
// for a coefficient loaded with a uniform address (held in scalar registers)
// the whole conversion runs on the scalar unit, where gfx950 has no float
// conversion instruction, instead of taking vector registers and instructions
// in every lane.  Normal numbers move their exponent and mantissa fields;
// subnormals are normalised; zeros, infinities and NaNs keep their class.
__device__ static inline double widen_exact(float f) {
    // Every case is formed and the right one selected (fewer scalar branches
    // in the backward's prologue than an if-chain; KAT-T backward ~1% faster).
    const uint32_t u = __float_as_uint(f);
    const uint32_t sign = u & 0x80000000u;
    const uint32_t e = (u >> 23) & 0xffu;
    const uint32_t m = u & 0x7fffffu;
    // normal: 2^(e - 127) * 1.m; infinity or NaN keep m under an all-ones exponent
    const uint32_t hi_n = sign | ((e == 0xffu ? 0x7ffu : e + 896u) << 20) | (m >> 3);
    const uint32_t lo_n = m << 29;
    // subnormal: m * 2^-149 with its top bit at p (m | 1 keeps clz defined for m = 0,
    // whose result is not selected)
    const uint32_t p = 31u - (uint32_t)__builtin_clz(m | 1u);
    const uint32_t mm = (m << (23u - p)) & 0x7fffffu;
    const uint32_t hi_s = sign | ((p + 874u) << 20) | (mm >> 3);
    const uint32_t lo_s = mm << 29;
    const bool sub = e == 0u;
    const uint32_t hi = sub ? (m == 0u ? sign : hi_s) : hi_n;  // e = 0, m = 0: signed zero
    const uint32_t lo = sub ? (m == 0u ? 0u : lo_s) : lo_n;
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Constants of the backward pass derived from one group's coefficients:
// the fp32 ones (BwdCoefs) and b_1..b_N in fp64 (QWide, exact copies, for Q).
// Two objects rather than one: with the fp64 array inside, BwdCoefs outgrows
// 128 bytes at degrees (6, 5) and (7, 6), and hipcc then keeps the gradient
// sums as separate scalars instead of one register vector, which costs those
// kernels 40-60 VGPRs (62 -> 110 and 66 -> 122 at fp32) and the bf16 (7, 6)
// kernel scratch spills.
template <int M, int N> struct BwdCoefs {
    float a[M + 1];              // a_0..a_M
    float da[M > 0 ? M : 1];     // i * a_i, i = 1..M   (P')
    float b[N > 0 ? N : 1];      // b_1..b_N
    float db[N > 0 ? N : 1];     // j * b_j, j = 1..N   (Q')
    float kguard;                // sign guard scale, see below
    bool q_zero;                 // b = 0 (or N = 0): Q vanishes identically, s = 0
};
template <int N> struct QWide {
    double b[N > 0 ? N : 1];     // b_1..b_N
};

// The sign guard.  The backward's Q is x q(x), q(x) = b_1 + b_2 x + ... +
// b_N x^(N-1) by Horner's rule with FMAs in fp64 from exact fp64 copies of x
// and b, then x q and its rounding to fp32 (backward_element).  Rounding
// keeps signs, so sign(Q) = sign(x) sign(q_computed) whenever Q != 0, and
// q_computed has q(x)'s sign when |q_computed| exceeds Horner's error bound,
// gamma_{N-1} S with S = sum_j |b_j| |x|^(j-1) and gamma_n ~ n 2^-53
// (Higham, "Accuracy and Stability of Numerical Algorithms", Horner's rule).
// Since |x| S <= (sum_j |b_j|) (1 + |x|^N), the test
//   |Q| > kguard (1 + |x|^N),  kguard = 2^-46 sum_j |b_j|
// -- one FMA and one compare -- proves the sign with a margin of 8x over
// gamma_{2N} for N <= 8, which also covers the fp32 roundings of Q, of |x|^N
// and of the bound itself.  kguard is kept at least 2^-126, so that a passing
// |Q| is a normal number (relative rounding) even for tiny coefficients.  The
// test fails at x = 0 (Q = 0), for NaN, infinite or huge x (|x|^N
// overflows), for |x| below ~2^-46 (relative to the coefficients), and within
// ~2^-46 (relative) of a root of q -- in practice only x = 0 at the
// workloads' inputs; those elements take the exact path.
template <int N> constexpr float sign_guard_scale() { return 1.0f / 70368744177664.0f; }  // 2^-46
constexpr float kGuardFloor = 1.17549435e-38f;  // 2^-126

template <int M, int N>
__device__ static inline BwdCoefs<M, N> derive(const Coefs<M, N> &c) {
    BwdCoefs<M, N> k;
#pragma unroll
    for (int i = 0; i <= M; ++i) k.a[i] = c.a[i];
#pragma unroll
    for (int i = 1; i <= M; ++i) k.da[i - 1] = (float)i * c.a[i];
    if constexpr (M == 0) k.da[0] = 0.0f;
    float bsum = 0.0f;
    // b == 0 (either sign of zero) tested on the bits, so that the uniform
    // test runs on the scalar unit (gfx950 has no scalar float compare)
    uint32_t nonzero = 0u;
#pragma unroll
    for (int j = 0; j < N; ++j) {
        k.b[j] = c.b[j];
        k.db[j] = (float)(j + 1) * c.b[j];
        bsum += fabsf(c.b[j]);
        nonzero |= __float_as_uint(c.b[j]) << 1;
    }
    const bool zero = nonzero == 0u;
    if constexpr (N == 0) {
        k.b[0] = 0.0f;
        k.db[0] = 0.0f;
    }
    k.kguard = fmaxf(sign_guard_scale<N>() * bsum, kGuardFloor);
    k.q_zero = zero;
    return k;
}

// UNIFORM: the coefficients are the same in every lane (scalar registers), so
// their fp64 copies are formed on the scalar unit; otherwise (per-lane
// coefficients) by the vector conversion.
template <int M, int N, bool UNIFORM = true>
__device__ static inline QWide<N> widen(const Coefs<M, N> &c) {
    QWide<N> q;
#pragma unroll
    for (int j = 0; j < N; ++j) q.b[j] = UNIFORM ? widen_exact(c.b[j]) : (double)c.b[j];
    if constexpr (N == 0) q.b[0] = 0.0;
    return q;
}

// Denominator degrees from which the backward decides an unproven sign of Q
// exactly (qsign_lanes, exact_signs, exact_apply below) instead of by
// compensated Horner (sign_q_compensated, compensated_fix): compensated
// Horner was measured wrong next to 5-fold roots of a degree-5 q, and
// matched the exact sign on every clustered and exact root tried below that.
// The split also keeps the GR-KAN (5, 4) kernels' code as it was: the scalar
// sign loop, present in a kernel, changes how its main loop is scheduled
// (2-3% slower at KAT-B), while it did not slow the (7, 6) ones.
constexpr int kExactSignMinN = 5;

// sign of q(x) = b_1 + b_2 x + ... + b_N x^(N-1) by compensated Horner in
// fp64 (grkan_qsign.h), for denominators of degree N < kExactSignMinN.
template <int M, int N>
__device__ static inline int sign_q_compensated(float xf, const BwdCoefs<M, N> &k) {
    static_assert(N >= 1, "no denominator");
    return qsign_compensated<N>(xf, k.b);
}

// sign(q(x)), q(x) = b_1 + b_2 x + ... + b_N x^(N-1), exactly by the integer
// evaluation of grkan_qsign.h, for the elements x[i] of each lane whose bit i
// of `need` is set: bit i of `pos` / `neg` for a positive / negative q(x[i]),
// of `keep` for an element beyond the integer window (it keeps the sign of
// its fp64-evaluated Q).  One (lane, element) at a time, its x and b are read
// into scalar registers and the evaluation runs on the scalar unit, so this
// rare decision takes almost no vector registers from the loop around it, and
// its code appears once per call.  A wave-wide loop: every active lane must
// call it.
template <int N, int E>
__device__ static inline void qsign_lanes(uint32_t need, const float (&x)[E], const float (&b)[N],
                                          uint32_t &pos, uint32_t &neg, uint32_t &keep) {
    static_assert(N >= 1 && E >= 1 && E <= 32, "sizes");
    const uint32_t me = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    pos = 0u;
    neg = 0u;
    keep = 0u;
    for (;;) {
        const uint64_t m = __builtin_amdgcn_ballot_w64(need != 0u);
        if (m == 0) break;
        const int l = __builtin_ctzll(m);
        const int i = need ? __builtin_ctz(need) : 0;  // this lane's next element
        // Chosen by selects; the asm keeps the compiler from turning them
        // into an indexed load from a stack copy of x.
        float xi = 0.0f;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            float xe = x[e];
            asm volatile("" : "+v"(xe));
            xi = (i == e) ? xe : xi;
        }
        // The asm keeps the coefficients' decomposition inside the loop
        // rather than hoisted out of it and held in registers throughout.
        float bl[N];
#pragma unroll
        for (int j = 0; j < N; ++j) {
            int bj = __builtin_amdgcn_readlane(__float_as_int(b[j]), l);
            asm volatile("" : "+s"(bj));
            bl[j] = __int_as_float(bj);
        }
        int sl = 0;
        const bool ok = qsign_integer<N>(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(xi), l)), bl, sl);
        if (me == (uint32_t)l) {
            pos |= (uint32_t)(ok && sl > 0) << i;
            neg |= (uint32_t)(ok && sl < 0) << i;
            keep |= (uint32_t)!ok << i;
            need &= need - 1u;
        }
    }
}

// Everything the backward needs about one element.  fp32 arithmetic except Q:
// Q = x q(x) is evaluated by Horner's rule in fp64 from the exact fp64 value
// of x and rounded once to fp32.  In fp32, Q's rounding error is relative to
// sum_j |b_j x^j| rather than to |Q|; next to a root of Q with large terms
// (|x| ~ 3 at GR-KAN's coefficients) that error reaches ~1e-6 of D = 1 + |Q|
// and passes into every gradient term of the element, which is enough to move
// a group sum that cancels to a few thousandths of its terms' norm by more
// than 1e-4 of itself.  In fp64 D is correctly rounded up to 2 units.  (gfx950
// issues fp64 FMAs at the fp32 rate; this costs two conversions per element.)
// s = sign(Q) is taken from that Q; `sure` says whether the guard proves
// that sign right.  When it does not (x == 0, x within rounding of a root of
// Q, NaN), the element still gets that sign here and compensated_fix() or
// exact_apply() later swap in the one decided again.  One function so that
// the hot loop and the fix agree bit for bit.
struct ElemBwd {
    float dx;   // dY (P'/D - s P Q'/D^2)
    float w;    // dY / D          (dA terms: w x^i)
    float v;    // dY P / D^2
    float sv;   // s v             (dB terms: -sv x^j)
    float Qd;   // Q'
    float wPd;  // w P'
    float F;    // P / D, the forward value
    bool sure;
};

template <int M, int N, int K>
__device__ static inline ElemBwd backward_element(const Pow<K> &X, float dy, const BwdCoefs<M, N> &k,
                                                  const QWide<N> &kw) {
    static_assert(K >= M && K >= N, "powers");
    const float x = X.p[K >= 1 ? 1 : 0];
    float P = k.a[0];
#pragma unroll
    for (int i = 1; i <= M; ++i) P = fmaf(k.a[i], X.p[i], P);
    float Pd = (M >= 1) ? k.da[0] : 0.0f;
#pragma unroll
    for (int i = 2; i <= M; ++i) Pd = fmaf(k.da[i - 1], X.p[i - 1], Pd);
    ElemBwd e;
    if constexpr (N == 0) {
        e.w = dy;
        e.v = 0.0f;
        e.sv = 0.0f;
        e.Qd = 0.0f;
        e.wPd = dy * Pd;
        e.dx = e.wPd;
        e.F = P;
        e.sure = true;
    } else {
        const double xd = (double)x;
        double qd = kw.b[N - 1];
#pragma unroll
        for (int j = N - 2; j >= 0; --j) qd = fma(qd, xd, kw.b[j]);
        const float Q = (float)(xd * qd);
        float Qd = k.db[0];
#pragma unroll
        for (int j = 1; j < N; ++j) Qd = fmaf(k.db[j], X.p[j], Qd);
        const float r = __builtin_amdgcn_rcpf(1.0f + fabsf(Q));
        e.w = dy * r;
        e.F = P * r;
        e.v = e.w * e.F;
        e.sv = __uint_as_float(__float_as_uint(e.v) ^ (__float_as_uint(Q) & 0x80000000u));
        e.sure = fabsf(Q) > fmaf(fabsf(X.p[N]), k.kguard, k.kguard);
        e.Qd = Qd;
        e.wPd = e.w * Pd;
        e.dx = fmaf(-e.sv, Qd, e.wPd);
    }
    return e;
}

// Adds one element's M + 1 + N gradient terms (dA: w x^i; dB: -sv x^j).
template <int M, int N, int K>
__device__ static inline void accumulate(float w, float sv, const Pow<K> &X,
                                         float (&acc)[Deg<M, N>::kNumCoef]) {
    acc[0] += w;
#pragma unroll
    for (int i = 1; i <= M; ++i) acc[i] = fmaf(w, X.p[i], acc[i]);
#pragma unroll
    for (int j = 1; j <= N; ++j) acc[M + j] = fmaf(-sv, X.p[j], acc[M + j]);
}

// For an element whose sign was not proven (N < kExactSignMinN): recomputes
// it, decides s = sign(x) sign(q(x)) by compensated Horner (0 at x == 0),
// replaces the dB terms that were accumulated with the fp64-Q sign and
// returns dX with the new sign.
template <int M, int N>
__device__ static inline float compensated_fix(float x, float dy, const BwdCoefs<M, N> &k,
                                               const QWide<N> &kw, float (&acc)[Deg<M, N>::kNumCoef]) {
    constexpr int K = Deg<M, N>::kTop;
    const Pow<K> X(x);
    const ElemBwd e = backward_element<M, N, K>(X, dy, k, kw);
    if constexpr (N == 0) {
        return e.dx;
    } else {
        if (e.sure) return e.dx;
        const int s = (x == 0.0f || k.q_zero) ? 0 : sign_q_compensated<M, N>(x, k) * ((x > 0.0f) ? 1 : -1);
        const float sv = (s == 0) ? 0.0f : ((s > 0) ? e.v : -e.v);
        const float diff = e.sv - sv;  // undo -e.sv x^j, add -sv x^j
#pragma unroll
        for (int j = 1; j <= N; ++j) acc[M + j] = fmaf(diff, X.p[j], acc[M + j]);
        return fmaf(-sv, e.Qd, e.wPd);
    }
}

// Where the exact-sign steps below take the coefficients from: the caller's
// registers.
template <int M, int N> struct CoefHeld {
    const BwdCoefs<M, N> &k;
    const QWide<N> &kw;
    __device__ void get(BwdCoefs<M, N> &k2, QWide<N> &kw2) const {
        k2 = k;
        kw2 = kw;
    }
};

// The exact sign for a lane's E elements of a tile in which some sign was
// not proven, in two steps.  exact_signs: which elements the guard did not
// prove and that are to be redone (unsure: all of them but those beyond the
// integer window, which keep their sign) and, for those with x != 0, the sign
// of q(x) (pos / neg bits).  A wave-wide call.  Only the guard's verdicts of
// its evaluation are used; the rest is dead code.
template <int M, int N, int E, class Src>
__device__ static inline void exact_signs(const float (&x)[E], const Src &src, uint32_t &unsure,
                                          uint32_t &pos, uint32_t &neg) {
    constexpr int K = Deg<M, N>::kTop;
    BwdCoefs<M, N> k;
    QWide<N> kw;
    src.get(k, kw);
    uint32_t need = 0u;
    unsure = 0u;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        // one element after another (the asm ties x[e] to the bits so far):
        // interleaved, the E evaluations would need E times the registers
        float xe = x[e];
        asm volatile("" : "+v"(xe) : "v"(unsure));
        const bool sure = backward_element<M, N, K>(Pow<K>(xe), 0.0f, k, kw).sure;
        unsure |= (uint32_t)!sure << e;
        need |= (uint32_t)(!sure && xe != 0.0f && !k.q_zero) << e;
    }
    pos = 0u;
    neg = 0u;
    uint32_t keep = 0u;
    if constexpr (N > 0) qsign_lanes<N, E>(need, x, k.b, pos, neg, keep);
    unsure &= ~keep;
}

// exact_apply: evaluates the E elements, replaces the dB terms of the unsure
// ones (accumulated with the fp64-Q sign) by those of the exact sign and
// returns every element's dX in dx.  x and dy must be the same values that
// went through the main loop and exact_signs.
template <int M, int N, int E, class Src>
__device__ static inline void exact_apply(const float (&x)[E], const float (&dy)[E], const Src &src,
                                          uint32_t unsure, uint32_t pos, uint32_t neg,
                                          float (&acc)[Deg<M, N>::kNumCoef], float (&dx)[E]) {
    constexpr int K = Deg<M, N>::kTop;
    BwdCoefs<M, N> k;
    QWide<N> kw;
    src.get(k, kw);
#pragma unroll
    for (int e = 0; e < E; ++e) {
        float xe = x[e];
        if (e > 0) asm volatile("" : "+v"(xe) : "v"(dx[e - 1]));  // one after another, as above
        const Pow<K> X(xe);
        const ElemBwd el = backward_element<M, N, K>(X, dy[e], k, kw);
        dx[e] = el.dx;
        if constexpr (N > 0) {
            if ((unsure >> e) & 1u) {
                const int sq = ((pos >> e) & 1u) ? 1 : (((neg >> e) & 1u) ? -1 : 0);
                const int s = sq * ((xe > 0.0f) ? 1 : -1);
                const float sv = (s == 0) ? 0.0f : ((s > 0) ? el.v : -el.v);
                const float diff = el.sv - sv;  // undo -el.sv x^j, add -sv x^j
#pragma unroll
                for (int j = 1; j <= N; ++j) acc[M + j] = fmaf(diff, X.p[j], acc[M + j]);
                dx[e] = fmaf(-sv, el.Qd, el.wPd);
            }
        }
    }
}

// backward_element with the sign fixed: when the guard does not prove
// sign(Q), s = sign(x) sign(q(x)) is decided again (0 at x == 0; exactly from
// kExactSignMinN on, a wave-wide call there; by compensated Horner below) and
// sv and dX are recomputed with it.  Bit for bit equal to backward_element
// wherever the guard holds.
template <int M, int N, int K>
__device__ static inline ElemBwd sign_fixed_element(const Pow<K> &X, float dy, const BwdCoefs<M, N> &k,
                                                    const QWide<N> &kw) {
    ElemBwd e = backward_element<M, N, K>(X, dy, k, kw);
    if constexpr (N >= kExactSignMinN) {
        const float x[1] = {X.p[1]};
        uint32_t pos, neg, keep;
        qsign_lanes<N, 1>((uint32_t)(!e.sure && x[0] != 0.0f && !k.q_zero), x, k.b, pos, neg, keep);
        if (!e.sure && !keep) {
            const int s = (pos ? 1 : (neg ? -1 : 0)) * ((x[0] > 0.0f) ? 1 : -1);
            e.sv = (s == 0) ? 0.0f : ((s > 0) ? e.v : -e.v);
            e.dx = fmaf(-e.sv, e.Qd, e.wPd);
        }
        e.sure = true;
    } else if constexpr (N > 0) {
        if (!e.sure) {
            const float x = X.p[1];
            const int s = (x == 0.0f || k.q_zero) ? 0 : sign_q_compensated<M, N>(x, k) * ((x > 0.0f) ? 1 : -1);
            e.sv = (s == 0) ? 0.0f : ((s > 0) ? e.v : -e.v);
            e.dx = fmaf(-e.sv, e.Qd, e.wPd);
            e.sure = true;
        }
    }
    return e;
}

}  // namespace grkan
