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
// coefficient, instead of one atomic per element and coefficient.  The same
// (row tile, group) decomposition is kept here, shaped for CDNA4 and HBM3E:
//   * One workgroup per (tile, group), short-lived: it issues all its 16-byte
//     loads at once, computes, stores and exits.  A large grid of such
//     workgroups, dispatched in order, keeps the set of addresses in flight
//     small and moving forward through memory, which HBM serves best; a
//     persistent loop would also wait, each iteration, for the previous
//     iteration's stores (gfx9 counts stores and loads in one counter).
//   * The dispatcher deals consecutive workgroups round-robin to the 8 XCDs;
//     workgroup b is mapped so that XCD (b mod 8) takes whole row tiles (all
//     groups of tiles b mod 8, +8, +16, ...).  The 8 XCDs then work on
//     different rows at any moment rather than all on the same ones.
//   * Lanes cover rows_per_iter rows x the group's 16-byte vectors: each wave
//     reads whole 128-byte lines, and a lane's group -- hence coefficients,
//     which sit in scalar registers -- is the workgroup's.
//   * Backward: the tile's gradient terms are summed in fp32 registers (at
//     most 16 terms per lane), then across the workgroup through LDS, and
//     leave the workgroup as ten fp32 atomics (one per coefficient,
//     as in the pages' Algorithm 2) or as ten partials merged afterwards in
//     fp64 in a fixed order (the two-stage reduction of [PolyKAN]), which is
//     bitwise reproducible: the tiling depends only on the shape.
#include "grkan_device.h"
#include "grkan_launch.h"

namespace grkan {

constexpr bool kNonTemporal = true;  // stream-once data: do not keep it in the caches
constexpr int kMaxBlock = 1024;

// Tuning per (I/O type, pass): U = passes per workgroup (all of a lane's
// loads are issued together), block = target workgroup size.  Chosen by
// measurement on MI355X at the KAT-B shapes: the backward prefers small
// blocks (with ~90 VGPRs a SIMD holds 5 of its waves; 3-wave blocks fill
// those slots in finer steps than 6-wave ones) and 4 passes to amortise the
// block reduction.
template <class IO, int pass> struct Tune;
template <> struct Tune<float, 0> { static constexpr int U = 2, block = 384; };
template <> struct Tune<bf16io, 0> { static constexpr int U = 2, block = 384; };
template <> struct Tune<float, 1> { static constexpr int U = 4, block = 192; };
template <> struct Tune<bf16io, 1> { static constexpr int U = 2, block = 192; };
// One fp32 atomic per coefficient per workgroup serialises on the few cache
// lines of dA and dB in L2, so the atomic mode uses 4x larger workgroups.
constexpr int kAtomicModeBlock = 768;

int unroll(grkan_dtype_t io, int pass) {
    if (io == GRKAN_BF16) return pass ? Tune<bf16io, 1>::U : Tune<bf16io, 0>::U;
    return pass ? Tune<float, 1>::U : Tune<float, 0>::U;
}

int target_block(grkan_dtype_t io, int pass, bool atomic_mode) {
    if (pass == 1 && atomic_mode) return kAtomicModeBlock;
    if (io == GRKAN_BF16) return pass ? Tune<bf16io, 1>::block : Tune<bf16io, 0>::block;
    return pass ? Tune<float, 1>::block : Tune<float, 0>::block;
}

// (tile, group) of this workgroup; false for the padding workgroups of the
// last round of 8 tiles.
__device__ static inline bool tile_of(const Geometry &G, int &g, int64_t &tile) {
    const int64_t b = blockIdx.x;
    const int64_t k = b >> 3;
    tile = (k / G.n_groups) * 8 + (b & 7);
    g = (int)(k % G.n_groups);
    return tile < G.tiles;
}

// Where a tile's partial sums go.  Tiles run on XCD (tile mod 8); slot
// (tile mod 8) * ceil(tiles / 8) + tile / 8 puts the tiles of one XCD next to
// each other, so that XCD's L2 assembles whole lines of partials before
// writing them back instead of sending scattered 4-byte writes.
__host__ __device__ static inline int64_t partial_tiles8(const Geometry &G) { return (G.tiles + 7) / 8; }
__host__ __device__ static inline int64_t partial_slots(const Geometry &G) { return 8 * partial_tiles8(G); }
__device__ static inline int64_t partial_slot(const Geometry &G, int64_t tile) {
    return (tile & 7) * partial_tiles8(G) + (tile >> 3);
}

// Lane placement inside a tile.
struct Lane {
    int64_t off;     // vector offset of pass 0
    int64_t stride;  // vectors between passes (rows_per_iter rows)
    int64_t row;     // row of pass 0
    bool active;     // one of the tile's `lanes` (not wave padding)
};

__device__ static inline Lane lane_of(const Geometry &G, int g, int64_t tile, int U) {
    const int tid = threadIdx.x;
    const int col = tid % G.seg_vecs;
    const int roff = tid / G.seg_vecs;
    Lane l;
    l.row = tile * (int64_t)U * G.rows_per_iter + roff;
    l.off = l.row * G.row_vecs + (int64_t)g * G.seg_vecs + col;
    l.stride = (int64_t)G.rows_per_iter * G.row_vecs;
    l.active = tid < G.lanes;
    return l;
}

// ----------------------------------------------------------------- forward

template <class IO, int U>
__global__ __launch_bounds__(kMaxBlock) void grkan_fwd_kernel(FwdArgs a) {
    using V = Io<IO>;
    constexpr int E = V::kElems;
    const Geometry &G = a.geo;
    int g;
    int64_t tile;
    if (!tile_of(G, g, tile)) return;
    const Coefs c = load_coefs(a.A, a.B, g);
    const Lane l = lane_of(G, g, tile, U);
    const u32x4 *xp = static_cast<const u32x4 *>(a.x) + l.off;
    u32x4 *yp = static_cast<u32x4 *>(a.y) + l.off;

    bool ok[U];
    u32x4 in[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        ok[u] = l.active && (l.row + (int64_t)u * G.rows_per_iter < G.rows);
        in[u] = ok[u] ? load16<kNonTemporal>(xp + u * l.stride) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        float f[E];
        V::unpack(in[u], f);
#pragma unroll
        for (int e = 0; e < E; ++e) f[e] = rational(f[e], c);
        if (ok[u]) store16<kNonTemporal>(yp + u * l.stride, V::pack(f));
    }
}

// ---------------------------------------------------------------- backward

// One tile's elements: dX stored, the ten gradient sums of this lane in acc.
// The rare exact-sign fix runs once per tile, before any dX is stored; it
// re-reads x and dy, which is safe even when dx aliases x or dy.
template <class IO, int U, bool QZERO>
__device__ static inline void bwd_tile(const BwdArgs &a, const BwdCoefs &k, const Lane &l,
                                       float (&acc)[kNumCoef]) {
    using V = Io<IO>;
    constexpr int E = V::kElems;
    const Geometry &G = a.geo;
    const u32x4 *xp = static_cast<const u32x4 *>(a.x) + l.off;
    const u32x4 *dyp = static_cast<const u32x4 *>(a.dy) + l.off;
    u32x4 *dxp = static_cast<u32x4 *>(a.dx) + l.off;

    bool ok[U];
    u32x4 xin[U], din[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        ok[u] = l.active && (l.row + (int64_t)u * G.rows_per_iter < G.rows);
        xin[u] = ok[u] ? load16<kNonTemporal>(xp + u * l.stride) : u32x4{0u, 0u, 0u, 0u};
        din[u] = ok[u] ? load16<kNonTemporal>(dyp + u * l.stride) : u32x4{0u, 0u, 0u, 0u};
    }
    float dxf[U][E];
    bool sure = true;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        float xf[E], dyf[E];
        V::unpack(xin[u], xf);
        V::unpack(din[u], dyf);
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const float x = xf[e], dy = dyf[e];
            const float x2 = x * x, x3 = x2 * x, x4 = x2 * x2, x5 = x4 * x;
            if constexpr (QZERO) {
                // Q == 0: D = 1, s = 0: dX = dY P', dA terms dY x^i, no dB terms.
                const float Pd = fmaf(k.da[4], x4, fmaf(k.da[3], x3, fmaf(k.da[2], x2,
                                 fmaf(k.da[1], x, k.da[0]))));
                dxf[u][e] = dy * Pd;
                accumulate(dy, 0.0f, x, x2, x3, x4, x5, acc);
            } else {
                const ElemBwd eb = backward_element(x, x2, x3, x4, x5, dy, k);
                accumulate(eb.w, eb.sv, x, x2, x3, x4, x5, acc);
                dxf[u][e] = eb.dx;
                sure = sure && eb.sure;
            }
        }
    }
    if constexpr (!QZERO) {
        // Rare: some element's sign of Q was not proven by the fp32 guard.
        if (__builtin_expect(!sure, 0)) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (ok[u]) {
                    float xf[E], dyf[E];
                    V::unpack(xp[u * l.stride], xf);
                    V::unpack(dyp[u * l.stride], dyf);
#pragma unroll
                    for (int e = 0; e < E; ++e) dxf[u][e] = exact_fix(xf[e], dyf[e], k, acc);
                }
            }
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
        if (ok[u]) store16<kNonTemporal>(dxp + u * l.stride, V::pack(dxf[u]));
}

template <class IO, int U>
__global__ __launch_bounds__(kMaxBlock) void grkan_bwd_kernel(BwdArgs a) {
    const Geometry &G = a.geo;
    int g;
    int64_t tile;
    if (!tile_of(G, g, tile)) return;
    const BwdCoefs k = derive(load_coefs(a.A, a.B, g));
    const Lane l = lane_of(G, g, tile, U);
    float acc[kNumCoef];
#pragma unroll
    for (int i = 0; i < kNumCoef; ++i) acc[i] = 0.0f;
    if (k.q_zero)
        bwd_tile<IO, U, true>(a, k, l, acc);
    else
        bwd_tile<IO, U, false>(a, k, l, acc);

    // Workgroup sum of the ten terms, in a fixed order: transposed through LDS
    // (lane sums -> red[k][lane]); 16 threads per coefficient add block/16
    // consecutive lanes each in fp32; thread k adds its coefficient's 16 slices
    // in fp64.  About 13 VALU operations per lane, against 60 for DPP sums of
    // the ten values across each wave (measured faster on MI355X, where the
    // backward's VALU load and power draw matter).
    extern __shared__ float red[];  // [kNumCoef][block]; later [kNumCoef][16]
    const int t = threadIdx.x;
    const int nb = G.block;
#pragma unroll
    for (int i = 0; i < kNumCoef; ++i) red[i * nb + t] = acc[i];
    __syncthreads();
    const int per = nb / 16;  // a multiple of 4: blocks are whole waves
    float slice = 0.0f;
    if (t < kNumCoef * 16) {
        const int k = t >> 4, seg = t & 15;
        const float4 *src = reinterpret_cast<const float4 *>(red + k * nb + seg * per);
        for (int j = 0; j < per / 4; ++j) {
            const float4 q = src[j];
            slice += ((q.x + q.y) + q.z) + q.w;
        }
    }
    __syncthreads();
    if (t < kNumCoef * 16) red[t] = slice;
    __syncthreads();
    double total = 0.0;
    if (t < kNumCoef) {
#pragma unroll
        for (int j = 0; j < 16; ++j) total += (double)red[t * 16 + j];
    }
    if (t < kNumCoef) {
        if (a.mode == kModePartials) {
            a.partials[((int64_t)g * kNumCoef + t) * partial_slots(G) + partial_slot(G, tile)] = (float)total;
        } else {
            float *dst = (t < kNumA) ? (a.dA + g * kNumA + t) : (a.dB + g * kNumB + (t - kNumA));
            unsafeAtomicAdd(dst, (float)total);
        }
    }
}

// Second stage of the deterministic mode: workgroup (g, k) adds the tile
// partials of group g, coefficient k in a fixed order in fp64.  Each thread
// issues all of its loads before adding, so the kernel costs about one memory
// round trip rather than one per loop iteration.
constexpr int kMergeThreads = 1024;
constexpr int kMergeLoads = 8;
__global__ __launch_bounds__(kMergeThreads) void grkan_merge_kernel(const float *__restrict__ partials,
                                                                    int64_t tiles, float *__restrict__ dA,
                                                                    float *__restrict__ dB) {
    const int gk = blockIdx.x;
    const int64_t t8 = (tiles + 7) / 8, slots = 8 * t8;
    const float *p = partials + (int64_t)gk * slots;
    double s = 0.0;
    for (int64_t base = 0; base < slots; base += (int64_t)kMergeThreads * kMergeLoads) {
        float v[kMergeLoads];
#pragma unroll
        for (int i = 0; i < kMergeLoads; ++i) {
            const int64_t q = base + (int64_t)i * kMergeThreads + threadIdx.x;
            const int64_t tile = (q % t8) * 8 + q / t8;  // slot -> tile; padding slots hold nothing
            v[i] = (q < slots && tile < tiles) ? p[q] : 0.0f;
        }
#pragma unroll
        for (int i = 0; i < kMergeLoads; ++i) s += (double)v[i];
    }
#pragma unroll
    for (int mask = 32; mask >= 1; mask >>= 1) s += __shfl_xor(s, mask, 64);
    __shared__ double lds[kMergeThreads / 64];
    if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
        double total = 0.0;
        for (int w = 0; w < kMergeThreads / 64; ++w) total += lds[w];
        const int g = gk / kNumCoef, k = gk % kNumCoef;
        if (k < kNumA) dA[g * kNumA + k] = (float)total;
        else dB[g * kNumB + k - kNumA] = (float)total;
    }
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
    hipLaunchKernelGGL((grkan_fwd_kernel<IO, Tune<IO, 0>::U>), dim3((unsigned)a.geo.grid),
                       dim3(a.geo.block), 0, s, a);
    return hipGetLastError();
}

template <class IO>
static hipError_t bwd_impl(const BwdArgs &a, hipStream_t s) {
    const size_t lds = (size_t)kNumCoef * a.geo.block * sizeof(float);
    hipLaunchKernelGGL((grkan_bwd_kernel<IO, Tune<IO, 1>::U>), dim3((unsigned)a.geo.grid),
                       dim3(a.geo.block), lds, s, a);
    return hipGetLastError();
}

hipError_t launch_forward(grkan_dtype_t io, const FwdArgs &a, hipStream_t s) {
    return io == GRKAN_BF16 ? fwd_impl<bf16io>(a, s) : fwd_impl<float>(a, s);
}

hipError_t launch_backward(grkan_dtype_t io, const BwdArgs &a, hipStream_t s) {
    return io == GRKAN_BF16 ? bwd_impl<bf16io>(a, s) : bwd_impl<float>(a, s);
}

hipError_t launch_merge(const float *partials, int32_t n_groups, int64_t tiles, float *dA,
                        float *dB, hipStream_t s) {
    hipLaunchKernelGGL(grkan_merge_kernel, dim3((unsigned)(n_groups * kNumCoef)), dim3(kMergeThreads), 0, s,
                       partials, tiles, dA, dB);
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
    const size_t lds = pass ? (size_t)kNumCoef * block * sizeof(float) : 0;
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, fn, block, lds);
}

}  // namespace grkan
