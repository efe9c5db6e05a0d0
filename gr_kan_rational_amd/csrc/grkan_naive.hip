// grkan_naive.hip -- per-element-atomic backward: the measurement baseline.
//
// Pages cited
//   [FlashKAT notes]  "FlashKAT: Understanding and Addressing Performance
//                     Bottlenecks in the Kolmogorov-Arnold Transformer",
//                     Paper-Notes page (AAAI 2026), arXiv 2505.13813.
//
// [FlashKAT notes] (section "2. 原始 KAT 的 atomic add 问题分析") describe the
// original KAT backward: a 1D grid, one element per thread, each thread
// reading its group's coefficients and adding its ten gradient terms straight
// into the global dA / dB with atomic adds, which serialises on 80 addresses.
// This kernel does the same on gfx950 so that its time and its fp32 rounding
// error can be set beside the block-reduced kernels.  Same element math as the
// fast path; only the accumulation differs.  This translation unit is built
// with the compiler's atomic optimizer off, so every lane's atomic stays one
// hardware atomic (no wave-level pre-reduction).
#include "grkan_device.h"
#include "grkan_launch.h"

namespace grkan {

template <class IO> struct Scalar;
template <> struct Scalar<float> {
    __device__ static inline float load(const void *p, int64_t i) { return static_cast<const float *>(p)[i]; }
    __device__ static inline void store(void *p, int64_t i, float v) { static_cast<float *>(p)[i] = v; }
};
template <> struct Scalar<bf16io> {
    __device__ static inline float load(const void *p, int64_t i) {
        return __uint_as_float((unsigned)static_cast<const unsigned short *>(p)[i] << 16);
    }
    __device__ static inline void store(void *p, int64_t i, float v) {
        static_cast<__bf16 *>(p)[i] = (__bf16)v;
    }
};

constexpr int kM = 5, kN = 4;  // GR-KAN's degrees
constexpr int kNumA = kM + 1, kNumB = kN, kNumCoef = kM + 1 + kN;

template <class IO>
__global__ __launch_bounds__(256) void grkan_bwd_naive_kernel(const void *x, const void *dy, void *dx,
                                                              const float *A, const float *B,
                                                              float *dA, float *dB, int64_t n,
                                                              int64_t d, int64_t d_g) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const int g = (int)((i % d) / d_g);
        const Coefs<kM, kN> c = load_coefs<kM, kN>(A, B, g);
        const BwdCoefs<kM, kN> k = derive<kM, kN>(c);
        const QWide<kN> kw = widen<kM, kN, false>(c);
        float acc[kNumCoef];
#pragma unroll
        for (int c = 0; c < kNumCoef; ++c) acc[c] = 0.0f;
        const float xv = Scalar<IO>::load(x, i), dyv = Scalar<IO>::load(dy, i);
        const Pow<kM> X(xv);
        const ElemBwd e = sign_fixed_element<kM, kN, kM>(X, dyv, k, kw);
        accumulate<kM, kN>(e.w, e.sv, X, acc);
        Scalar<IO>::store(dx, i, e.dx);
#pragma unroll
        for (int c = 0; c < kNumA; ++c) unsafeAtomicAdd(dA + g * kNumA + c, acc[c]);
#pragma unroll
        for (int c = 0; c < kNumB; ++c) unsafeAtomicAdd(dB + g * kNumB + c, acc[kNumA + c]);
    }
}

hipError_t launch_naive(grkan_dtype_t io, const void *x, const void *dy, void *dx, const float *A,
                        const float *B, float *dA, float *dB, int64_t rows, int64_t d,
                        int32_t n_groups, hipStream_t s) {
    const int64_t n = rows * d;
    int64_t blocks = (n + 255) / 256;
    if (blocks > (1 << 20)) blocks = 1 << 20;
    if (blocks < 1) blocks = 1;
    const int64_t d_g = d / n_groups;
    if (io == GRKAN_BF16)
        hipLaunchKernelGGL(grkan_bwd_naive_kernel<bf16io>, dim3((unsigned)blocks), dim3(256), 0, s,
                           x, dy, dx, A, B, dA, dB, n, d, d_g);
    else
        hipLaunchKernelGGL(grkan_bwd_naive_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, s, x,
                           dy, dx, A, B, dA, dB, n, d, d_g);
    return hipGetLastError();
}

}  // namespace grkan
