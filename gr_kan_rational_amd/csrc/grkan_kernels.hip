// grkan_kernels.hip -- GR-KAN forward / backward kernels for gfx950 (MI355X).
//
// Pages cited
//   [FlashKAT notes]  "FlashKAT: Understanding and Addressing Performance
//                     Bottlenecks in the Kolmogorov-Arnold Transformer",
//                     Paper-Notes page (AAAI 2026), arXiv 2505.13813.
//   [PolyKAN]         "PolyKAN: Efficient Fused GPU Operators for Polynomial
//                     Kolmogorov-Arnold Network Variants", abstract page
//                     (arXiv 2511.14852).
//
// Work decomposition.  [FlashKAT notes] (section "3. FlashKAT 核函数重构
// （Algorithm 2）") restructures the backward as a 2D grid of row tiles x
// groups in which a block loads its group's coefficients once, accumulates
// all of its gradient terms locally and then makes one global update per
// coefficient, instead of one atomic per element and coefficient.  Here the
// same (row slice, group) decomposition is shaped for CDNA4:
//   * the launch is 1D with the group index fastest (blockIdx % n_groups), so
//     consecutive workgroups -- which the dispatcher deals round-robin to the
//     8 XCDs -- read neighbouring parts of the same rows, and with 8 groups
//     every XCD keeps one group (its coefficients and its 128-byte lines);
//   * the grid is sized to the resident capacity of the device (CUs x
//     workgroups per CU), one wave of workgroups, each walking an equal
//     contiguous range of row steps -- no tail of half-filled rounds;
//   * a workgroup's lanes tile rows_per_iter rows x the group's 16-byte
//     vectors, so every global access is a 16-byte load/store, a wave reads
//     whole 128-byte lines, and a lane's column (hence its group) is fixed;
//   * the gradient terms of one loop iteration are summed in fp32 registers,
//     then carried in fp64 per lane, reduced across the wave by butterfly
//     shuffles and across waves through LDS, and leave the workgroup either as
//     ten fp32 atomics (one per coefficient, as in the pages' Algorithm 2) or
//     as ten fp64 partials merged afterwards in a fixed order (the two-stage
//     reduction of [PolyKAN]), which makes the result bitwise reproducible.
#include "grkan_device.h"
#include "grkan_launch.h"

namespace grkan {

constexpr bool kNonTemporal = true;  // stream-once data: do not keep it in the caches
constexpr int kMaxBlock = 1024;
constexpr int kMaxWaves = kMaxBlock / 64;

template <class IO, int pass> struct Tune;
template <> struct Tune<float, 0> { static constexpr int U = 4; };
template <> struct Tune<bf16io, 0> { static constexpr int U = 2; };
template <> struct Tune<float, 1> { static constexpr int U = 4; };
template <> struct Tune<bf16io, 1> { static constexpr int U = 2; };

int unroll(grkan_dtype_t io, int pass) {
    if (io == GRKAN_BF16) return pass ? Tune<bf16io, 1>::U : Tune<bf16io, 0>::U;
    return pass ? Tune<float, 1>::U : Tune<float, 0>::U;
}

// Step range [s0, s1) of this workgroup, and the lane's vector offset.
struct LaneMap {
    int g;
    int slice;
    int64_t s0, s1, s1_full;
    int64_t step_vecs;
    int64_t lane_vec;
    int roff;
};

__device__ static inline LaneMap lane_map(const Geometry &G) {
    LaneMap m;
    m.g = blockIdx.x % G.n_groups;
    m.slice = blockIdx.x / G.n_groups;
    const int tid = threadIdx.x;
    const int col = tid % G.seg_vecs;
    m.roff = tid / G.seg_vecs;
    m.s0 = (int64_t)m.slice * G.steps / G.slices;
    m.s1 = (int64_t)(m.slice + 1) * G.steps / G.slices;
    const int64_t full = G.rows / G.rows_per_iter;  // steps whose rows all exist
    m.s1_full = m.s1 < full ? m.s1 : full;
    m.step_vecs = (int64_t)G.rows_per_iter * G.row_vecs;
    m.lane_vec = (int64_t)m.roff * G.row_vecs + (int64_t)m.g * G.seg_vecs + col;
    return m;
}

// ----------------------------------------------------------------- forward

template <class IO, int U>
__global__ __launch_bounds__(kMaxBlock) void grkan_fwd_kernel(FwdArgs a) {
    using V = Io<IO>;
    constexpr int E = V::kElems;
    const Geometry &G = a.geo;
    const LaneMap m = lane_map(G);
    const Coefs c = load_coefs(a.A, a.B, m.g);
    const u32x4 *xp = static_cast<const u32x4 *>(a.x) + m.lane_vec;
    u32x4 *yp = static_cast<u32x4 *>(a.y) + m.lane_vec;

    int64_t s = m.s0;
    for (; s + U <= m.s1_full; s += U) {
        u32x4 in[U];
#pragma unroll
        for (int u = 0; u < U; ++u) in[u] = load16<kNonTemporal>(xp + (s + u) * m.step_vecs);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float f[E];
            V::unpack(in[u], f);
#pragma unroll
            for (int e = 0; e < E; ++e) f[e] = rational(f[e], c);
            store16<kNonTemporal>(yp + (s + u) * m.step_vecs, V::pack(f));
        }
    }
    for (; s < m.s1; ++s) {
        if (s * G.rows_per_iter + m.roff < G.rows) {
            float f[E];
            V::unpack(load16<kNonTemporal>(xp + s * m.step_vecs), f);
#pragma unroll
            for (int e = 0; e < E; ++e) f[e] = rational(f[e], c);
            store16<kNonTemporal>(yp + s * m.step_vecs, V::pack(f));
        }
    }
}

// ---------------------------------------------------------------- backward

// Sum v[0..N) over the workgroup; the totals are valid in threads 0..N-1 as
// out (thread k holds total k).  Fixed order: butterfly within each wave,
// then waves in index order.
template <int N>
__device__ static inline double block_sum(double (&v)[N], double (*lds)[N]) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nwaves = (blockDim.x + 63) >> 6;
    // Lanes [0, nlane) exist in this wave (the last wave of a block that is not
    // a multiple of 64 is partial).  Reads of a lane that does not exist count
    // as 0; every lane lane 0 depends on then holds a sum over existing lanes
    // only, so lane 0 ends with the wave total.
    const int nlane = min(64, (int)blockDim.x - wave * 64);
#pragma unroll
    for (int k = 0; k < N; ++k) {
#pragma unroll
        for (int mask = 32; mask >= 1; mask >>= 1) {
            const double o = __shfl_xor(v[k], mask, 64);
            v[k] += ((lane ^ mask) < nlane) ? o : 0.0;
        }
    }
    if (lane == 0) {
#pragma unroll
        for (int k = 0; k < N; ++k) lds[wave][k] = v[k];
    }
    __syncthreads();
    double t = 0.0;
    if (threadIdx.x < N) {
        for (int w = 0; w < nwaves; ++w) t += lds[w][threadIdx.x];
    }
    return t;
}

// Exact-sign correction of the steps [lo, hi) of one lane: re-reads x, dy and
// the dx it stored, and for every guarded element adds the s-terms with the
// exact sign (to dx in place and to the dB sums).  Runs only for lanes that
// met a guarded element, over the steps that held one.
template <class IO>
__device__ __forceinline__ static void correct_steps(const u32x4 *xp, const u32x4 *dyp, u32x4 *dxp,
                                                  const BwdCoefs &k, const Geometry &G,
                                                  const LaneMap &m, int64_t lo, int64_t hi,
                                                  double (&acc64)[kNumCoef]) {
    using V = Io<IO>;
    constexpr int E = V::kElems;
    for (int64_t t = lo; t < hi; ++t) {
        if (t * G.rows_per_iter + m.roff >= G.rows) break;
        float xf[E], dyf[E], dxf[E];
        V::unpack(xp[t * m.step_vecs], xf);
        V::unpack(dyp[t * m.step_vecs], dyf);
        V::unpack(dxp[t * m.step_vecs], dxf);
        bool changed = false;
        for (int e = 0; e < E; ++e) {
            const float x = xf[e];
            const QGuard qg = q_guard(x, x * x, (x * x) * x, k);
            float ddx, tb[kNumB];
            if (!qg.sure && exact_sign_terms(x, dyf[e], k, ddx, tb)) {
                dxf[e] += ddx;
                for (int j = 0; j < kNumB; ++j) acc64[kNumA + j] += (double)tb[j];
                changed = true;
            }
        }
        if (changed) dxp[t * m.step_vecs] = V::pack(dxf);
    }
}

template <class IO, int U>
__global__ __launch_bounds__(kMaxBlock) void grkan_bwd_kernel(BwdArgs a) {
    using V = Io<IO>;
    constexpr int E = V::kElems;
    const Geometry &G = a.geo;
    const LaneMap m = lane_map(G);
    const BwdCoefs k = derive(load_coefs(a.A, a.B, m.g));
    const u32x4 *xp = static_cast<const u32x4 *>(a.x) + m.lane_vec;
    const u32x4 *dyp = static_cast<const u32x4 *>(a.dy) + m.lane_vec;
    u32x4 *dxp = static_cast<u32x4 *>(a.dx) + m.lane_vec;

    double acc64[kNumCoef];
#pragma unroll
    for (int i = 0; i < kNumCoef; ++i) acc64[i] = 0.0;
    // Steps [fix_lo, fix_hi) hold every guarded element of this lane.
    int64_t fix_lo = m.s1, fix_hi = m.s0;

    int64_t s = m.s0;
    for (; s + U <= m.s1_full; s += U) {
        u32x4 xin[U], din[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            xin[u] = load16<kNonTemporal>(xp + (s + u) * m.step_vecs);
            din[u] = load16<kNonTemporal>(dyp + (s + u) * m.step_vecs);
        }
        float acc[kNumCoef];
#pragma unroll
        for (int i = 0; i < kNumCoef; ++i) acc[i] = 0.0f;
        bool any = false;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float xf[E], dyf[E], dxf[E];
            V::unpack(xin[u], xf);
            V::unpack(din[u], dyf);
#pragma unroll
            for (int e = 0; e < E; ++e) {
                bool gd;
                dxf[e] = backward_element(xf[e], dyf[e], k, acc, gd);
                any |= gd;
            }
            store16<kNonTemporal>(dxp + (s + u) * m.step_vecs, V::pack(dxf));
        }
#pragma unroll
        for (int i = 0; i < kNumCoef; ++i) acc64[i] += (double)acc[i];
        fix_lo = (any && s < fix_lo) ? s : fix_lo;
        fix_hi = any ? s + U : fix_hi;
    }
    for (; s < m.s1; ++s) {
        if (s * G.rows_per_iter + m.roff < G.rows) {
            float xf[E], dyf[E], dxf[E];
            V::unpack(load16<kNonTemporal>(xp + s * m.step_vecs), xf);
            V::unpack(load16<kNonTemporal>(dyp + s * m.step_vecs), dyf);
            float acc[kNumCoef];
#pragma unroll
            for (int i = 0; i < kNumCoef; ++i) acc[i] = 0.0f;
            bool any = false;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                bool gd;
                dxf[e] = backward_element(xf[e], dyf[e], k, acc, gd);
                any |= gd;
            }
            store16<kNonTemporal>(dxp + s * m.step_vecs, V::pack(dxf));
#pragma unroll
            for (int i = 0; i < kNumCoef; ++i) acc64[i] += (double)acc[i];
            fix_lo = (any && s < fix_lo) ? s : fix_lo;
            fix_hi = any ? s + 1 : fix_hi;
        }
    }
    if (__builtin_expect(fix_lo < fix_hi, 0) && !k.q_zero)
        correct_steps<IO>(xp, dyp, dxp, k, G, m, fix_lo, fix_hi, acc64);

    __shared__ double lds[kMaxWaves][kNumCoef];
    const double total = block_sum<kNumCoef>(acc64, lds);
    const int t = threadIdx.x;
    if (t < kNumCoef) {
        if (a.mode == kModePartials) {
            a.partials[((int64_t)m.g * G.slices + m.slice) * kNumCoef + t] = total;
        } else {
            float *dst = (t < kNumA) ? (a.dA + m.g * kNumA + t) : (a.dB + m.g * kNumB + (t - kNumA));
            unsafeAtomicAdd(dst, (float)total);
        }
    }
}

// Second stage of the deterministic mode: one wave per group adds that
// group's slice partials in a fixed order and writes fp32 dA, dB.
__global__ __launch_bounds__(64) void grkan_merge_kernel(const double *__restrict__ partials,
                                                          int32_t slices, float *__restrict__ dA,
                                                          float *__restrict__ dB) {
    const int g = blockIdx.x;
    const int lane = threadIdx.x;
    double acc[kNumCoef];
#pragma unroll
    for (int i = 0; i < kNumCoef; ++i) acc[i] = 0.0;
    const double *base = partials + (int64_t)g * slices * kNumCoef;
    for (int p = lane; p < slices; p += 64) {
#pragma unroll
        for (int i = 0; i < kNumCoef; ++i) acc[i] += base[(int64_t)p * kNumCoef + i];
    }
#pragma unroll
    for (int i = 0; i < kNumCoef; ++i) {
#pragma unroll
        for (int mask = 32; mask >= 1; mask >>= 1) acc[i] += __shfl_xor(acc[i], mask, 64);
    }
    if (lane < kNumA) dA[g * kNumA + lane] = (float)acc[lane];
    else if (lane < kNumCoef) dB[g * kNumB + lane - kNumA] = (float)acc[lane];
}

__global__ __launch_bounds__(256) void grkan_zero_kernel(float *__restrict__ dA,
                                                         float *__restrict__ dB, int32_t n_groups) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n_groups * kNumA) dA[i] = 0.0f;
    if (i < n_groups * kNumB) dB[i] = 0.0f;
}

// ------------------------------------------------------------ host launchers

template <class IO>
static hipError_t fwd_impl(const FwdArgs &a, hipStream_t s) {
    const int64_t grid = (int64_t)a.geo.slices * a.geo.n_groups;
    hipLaunchKernelGGL((grkan_fwd_kernel<IO, Tune<IO, 0>::U>), dim3((unsigned)grid),
                       dim3(a.geo.block), 0, s, a);
    return hipGetLastError();
}

template <class IO>
static hipError_t bwd_impl(const BwdArgs &a, hipStream_t s) {
    const int64_t grid = (int64_t)a.geo.slices * a.geo.n_groups;
    hipLaunchKernelGGL((grkan_bwd_kernel<IO, Tune<IO, 1>::U>), dim3((unsigned)grid),
                       dim3(a.geo.block), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_forward(grkan_dtype_t io, const FwdArgs &a, hipStream_t s) {
    return io == GRKAN_BF16 ? fwd_impl<bf16io>(a, s) : fwd_impl<float>(a, s);
}

hipError_t launch_backward(grkan_dtype_t io, const BwdArgs &a, hipStream_t s) {
    return io == GRKAN_BF16 ? bwd_impl<bf16io>(a, s) : bwd_impl<float>(a, s);
}

hipError_t launch_merge(const double *partials, int32_t n_groups, int32_t slices, float *dA,
                        float *dB, hipStream_t s) {
    hipLaunchKernelGGL(grkan_merge_kernel, dim3((unsigned)n_groups), dim3(64), 0, s, partials,
                       slices, dA, dB);
    return hipGetLastError();
}

hipError_t launch_zero(float *dA, float *dB, int32_t n_groups, hipStream_t s) {
    const int n = n_groups * kNumA;
    hipLaunchKernelGGL(grkan_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, dA,
                       dB, n_groups);
    return hipGetLastError();
}

hipError_t occupancy(grkan_dtype_t io, int pass, int block, int *blocks_per_cu) {
    const void *fn;
    if (io == GRKAN_BF16)
        fn = pass ? (const void *)grkan_bwd_kernel<bf16io, Tune<bf16io, 1>::U>
                  : (const void *)grkan_fwd_kernel<bf16io, Tune<bf16io, 0>::U>;
    else
        fn = pass ? (const void *)grkan_bwd_kernel<float, Tune<float, 1>::U>
                  : (const void *)grkan_fwd_kernel<float, Tune<float, 0>::U>;
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, fn, block, 0);
}

}  // namespace grkan
