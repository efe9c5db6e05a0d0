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
// plain polynomial.  Everything here is fp32 register arithmetic; the only
// fp64 use is deciding the sign of Q for the rare element whose fp32 Q is
// within rounding of 0.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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

// Constants of the backward pass derived from one group's coefficients.
template <int M, int N> struct BwdCoefs {
    float a[M + 1];              // a_0..a_M
    float da[M > 0 ? M : 1];     // i * a_i, i = 1..M   (P')
    float b[N > 0 ? N : 1];      // b_1..b_N
    float db[N > 0 ? N : 1];     // j * b_j, j = 1..N   (Q')
    float kguard;                // sign guard scale, see below
    bool q_zero;                 // b = 0 (or N = 0): Q vanishes identically, s = 0
};

// The sign guard.  With powers formed as above and Q = x (b_1 + b_2 x + ...)
// summed by FMAs over them, the fp32 Q differs from the exact Q(x) by at most
// about (2N + 1) 2^-24 sum_j |b_j| |x|^j, and sum_j |b_j| |x|^j is at most
// (sum_j |b_j|) (|x| + |x|^N).  So |Q| > (N + 4) 2^-21 (sum_j |b_j|)
// (|x| + |x|^N) -- at least four times that bound -- proves Q != 0 and
// sign(fl(Q)) = sign(Q).  (For GR-KAN's N = 4 the scale is 2^-18.)
template <int N> constexpr float sign_guard_scale() { return (float)(N + 4) / 2097152.0f; }

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
    k.kguard = sign_guard_scale<N>() * bsum;
    k.q_zero = zero;
    return k;
}

// sign of q(x) = b_1 + b_2 x + ... + b_N x^(N-1) by compensated Horner in
// fp64 (error-free products by FMA and error-free sums; Graillat, Langlois &
// Louvet, "Compensated Horner scheme", 2005).  The result carries about twice
// fp64's precision, enough to fix the sign of every fp32 x that is not within
// ~2^-100 (relative) of a root.
template <int M, int N>
__device__ static inline int sign_q_exact(float xf, const BwdCoefs<M, N> &k) {
    // The error-free transformations need every product and sum rounded on its
    // own: no contraction of s*x + b into one FMA.
#pragma clang fp contract(off)
    static_assert(N >= 1, "no denominator");
    const double x = (double)xf;
    double s = (double)k.b[N - 1];
    double c = 0.0;
#pragma unroll
    for (int j = N - 2; j >= 0; --j) {
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
    float F;    // P / D, the forward value
    bool sure;
};

template <int M, int N, int K>
__device__ static inline ElemBwd backward_element(const Pow<K> &X, float dy, const BwdCoefs<M, N> &k) {
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
        float q = k.b[0];
#pragma unroll
        for (int j = 1; j < N; ++j) q = fmaf(k.b[j], X.p[j], q);
        float Qd = k.db[0];
#pragma unroll
        for (int j = 1; j < N; ++j) Qd = fmaf(k.db[j], X.p[j], Qd);
        const float Q = x * q;
        const float r = __builtin_amdgcn_rcpf(1.0f + fabsf(Q));
        e.w = dy * r;
        e.F = P * r;
        e.v = e.w * e.F;
        e.sv = __uint_as_float(__float_as_uint(e.v) ^ (__float_as_uint(Q) & 0x80000000u));
        e.sure = fabsf(Q) > k.kguard * (fabsf(x) + fabsf(X.p[N]));
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

// For an element whose sign was not proven: recomputes it, decides
// s = sign(x) sign(q(x)) exactly (0 at x == 0), replaces the dB terms that
// were accumulated with the fp32 sign and returns the exact dX.
template <int M, int N>
__device__ static inline float exact_fix(float x, float dy, const BwdCoefs<M, N> &k,
                                         float (&acc)[Deg<M, N>::kNumCoef]) {
    constexpr int K = Deg<M, N>::kTop;
    const Pow<K> X(x);
    const ElemBwd e = backward_element<M, N, K>(X, dy, k);
    if constexpr (N == 0) {
        return e.dx;
    } else {
        if (e.sure) return e.dx;
        const int s = (x == 0.0f || k.q_zero) ? 0 : sign_q_exact<M, N>(x, k) * ((x > 0.0f) ? 1 : -1);
        const float sv = (s == 0) ? 0.0f : ((s > 0) ? e.v : -e.v);
        const float diff = e.sv - sv;  // undo -e.sv x^j, add -sv x^j
#pragma unroll
        for (int j = 1; j <= N; ++j) acc[M + j] = fmaf(diff, X.p[j], acc[M + j]);
        return fmaf(-sv, e.Qd, e.wPd);
    }
}

// backward_element with the exact sign: when the fp32 guard does not prove
// sign(Q), s = sign(x) sign(q(x)) is decided exactly (0 at x == 0) and sv and
// dX are recomputed with it.  Bit for bit equal to backward_element wherever
// the guard holds.
template <int M, int N, int K>
__device__ static inline ElemBwd exact_element(const Pow<K> &X, float dy, const BwdCoefs<M, N> &k) {
    ElemBwd e = backward_element<M, N, K>(X, dy, k);
    if constexpr (N > 0) {
        if (!e.sure) {
            const float x = X.p[1];
            const int s = (x == 0.0f || k.q_zero) ? 0 : sign_q_exact<M, N>(x, k) * ((x > 0.0f) ? 1 : -1);
            e.sv = (s == 0) ? 0.0f : ((s > 0) ? e.v : -e.v);
            e.dx = fmaf(-e.sv, e.Qd, e.wPd);
            e.sure = true;
        }
    }
    return e;
}

}  // namespace grkan
