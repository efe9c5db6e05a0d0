// grkan_merge.hip -- degree-independent kernels of the backward pass: the
// fixed-order merge of the per-tile partial sums, and zeroing of dA / dB for
// the atomic schemes.
//
// Pages cited
//   [PolyKAN]  "PolyKAN: Efficient Fused GPU Operators for Polynomial
//              Kolmogorov-Arnold Network Variants", abstract page
//              (arXiv 2511.14852): a two-stage reduction of the coefficient
//              gradients in place of atomics.
#include "grkan_launch.h"

namespace grkan {

namespace {

// Second stage of the deterministic backward: the partials of group g,
// coefficient k -- one per (column part, row tile) -- are added in a fixed
// order in fp64.  Up to 16384 slots per (g, k) one workgroup takes them all,
// 8 or 16 per thread, and writes dA / dB directly (GR-KAN's 8 groups at KAT-B
// and at the hidden-layer shapes); beyond that (few groups, many tiles)
// workgroup (g, k, c) takes the c-th chunk of 8 slots per thread and writes
// an fp64 chunk sum, and grkan_merge_chunks_kernel adds the chunk sums in
// order.  Each thread issues all of its loads before adding, so a chunk
// costs about one memory round trip.  Slots are [parts][8 * bundles];
// within a part, slot r = (t mod 8) * bundles + t / 8 holds tile t, and the
// slots of tiles past the end hold nothing.
constexpr int kMergeThreads = 1024;
constexpr int kMergeLoads = 8;
constexpr int kMergeLoadsOne = 16;  // per thread when one workgroup takes all the slots
constexpr uint32_t kMergeChunk = (uint32_t)kMergeThreads * kMergeLoads;
constexpr uint32_t kMergeOneChunk = (uint32_t)kMergeThreads * kMergeLoadsOne;
// Coefficients with at most this many slots (many groups, few tiles: one
// function per channel) are merged one wave each: lane l adds slots l,
// l + 64, ... in order, then the wave adds its lanes in a fixed tree.
constexpr int kWaveLoads = 32;
constexpr uint32_t kSmallChunk = 64u * kWaveLoads;
constexpr int kWaveMergeThreads = 256;

__device__ static inline void write_sum(int gk, int32_t na, int32_t nb, double total, float *dA,
                                        float *dB) {
    const int nc = na + nb;
    const int g = gk / nc, k = gk % nc;
    if (k < na) dA[g * na + k] = (float)total;
    else dB[g * nb + k - na] = (float)total;
}

// fp64 sum over the workgroup of one value per thread, in a fixed order.
template <int T>
__device__ static inline double block_sum(double s) {
#pragma unroll
    for (int mask = 32; mask >= 1; mask >>= 1) s += __shfl_xor(s, mask, 64);
    __shared__ double lds[T / 64];
    if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = s;
    __syncthreads();
    double total = 0.0;
    if (threadIdx.x == 0)
        for (int w = 0; w < T / 64; ++w) total += lds[w];
    return total;
}

// Parts of group g's slots that hold partials: all of them for segment
// plans; for narrow plans the column blocks its channels span.
__device__ static inline uint32_t parts_of(int g, uint32_t parts, int32_t dg, int32_t cpb) {
    if (dg == 0) return parts;
    const int64_t first = (int64_t)g * dg / cpb, last = ((int64_t)g * dg + dg - 1) / cpb;
    return (uint32_t)(last - first + 1);
}

// Slot geometry of a launch: tile t of a part sits at slot (t mod 8) * bundles
// + t / 8; the divisions by the part length and by bundles are multiply-highs
// by host-computed constants (a vector integer division costs tens of
// instructions, and the merge does two per slot).
struct SlotMap {
    uint32_t tiles, bundles, per_part;
    FastDiv div_part, div_bundles;
};

// Whether slot q (below 2^31) holds a tile's partial.
__device__ static inline bool slot_holds_tile(uint32_t q, const SlotMap &sm) {
    const uint32_t r = q - fastdiv(q, sm.div_part) * sm.per_part;
    const uint32_t a = fastdiv(r, sm.div_bundles);
    return (r - a * sm.bundles) * 8u + a < sm.tiles;
}

template <int T, int L>
__global__ __launch_bounds__(T) void grkan_merge_kernel(
    const float *__restrict__ partials, SlotMap sm, uint32_t slots,
    int32_t na, int32_t nb, int32_t dg, int32_t cpb, uint32_t chunks, double *__restrict__ chunk_sums,
    float *__restrict__ dA, float *__restrict__ dB) {
    constexpr uint32_t chunk = (uint32_t)T * L;
    const int gk = (int)blockIdx.x;
    const uint32_t c = blockIdx.y;
    const uint32_t valid = parts_of(gk / (na + nb), slots / sm.per_part, dg, cpb) * sm.per_part;
    const float *p = partials + (int64_t)gk * slots;
    float v[L];
#pragma unroll
    for (int i = 0; i < L; ++i) {
        const uint32_t q = c * chunk + (uint32_t)i * T + threadIdx.x;
        v[i] = (q < valid && slot_holds_tile(q, sm)) ? p[q] : 0.0f;
    }
    double s = 0.0;
#pragma unroll
    for (int i = 0; i < L; ++i) s += (double)v[i];
    const double total = block_sum<T>(s);
    if (threadIdx.x == 0) {
        if (chunks == 1) write_sum(gk, na, nb, total, dA, dB);
        else chunk_sums[(int64_t)gk * chunks + c] = total;
    }
}

template <int L>
__global__ __launch_bounds__(kWaveMergeThreads) void grkan_merge_wave_kernel(
    const float *__restrict__ partials, SlotMap sm, uint32_t slots, int32_t na,
    int32_t nb, int32_t dg, int32_t cpb, uint32_t n_gk, float *__restrict__ dA, float *__restrict__ dB) {
    const uint32_t gk = blockIdx.x * (kWaveMergeThreads / 64) + (threadIdx.x >> 6);
    if (gk >= n_gk) return;  // whole waves: the shuffles below see only active waves
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t valid = parts_of((int)gk / (na + nb), slots / sm.per_part, dg, cpb) * sm.per_part;
    const float *p = partials + (int64_t)gk * slots;
    float v[L];
#pragma unroll
    for (int i = 0; i < L; ++i) {
        const uint32_t q = (uint32_t)i * 64u + lane;
        v[i] = (q < valid && slot_holds_tile(q, sm)) ? p[q] : 0.0f;
    }
    double s = 0.0;
#pragma unroll
    for (int i = 0; i < L; ++i) s += (double)v[i];
#pragma unroll
    for (int mask = 32; mask >= 1; mask >>= 1) s += __shfl_xor(s, mask, 64);
    if (lane == 0) write_sum((int)gk, na, nb, s, dA, dB);
}

constexpr int kChunkThreads = 256;

__global__ __launch_bounds__(kChunkThreads) void grkan_merge_chunks_kernel(
    const double *__restrict__ chunk_sums, uint32_t chunks, int32_t na, int32_t nb,
    float *__restrict__ dA, float *__restrict__ dB) {
    const int gk = (int)blockIdx.x;
    const double *p = chunk_sums + (int64_t)gk * chunks;
    double s = 0.0;
    for (uint32_t c = threadIdx.x; c < chunks; c += kChunkThreads) s += p[c];
    const double total = block_sum<kChunkThreads>(s);
    if (threadIdx.x == 0) write_sum(gk, na, nb, total, dA, dB);
}

__global__ __launch_bounds__(256) void grkan_zero_kernel(float *__restrict__ dA, float *__restrict__ dB,
                                                         int64_t na, int64_t nb) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < na) dA[i] = 0.0f;
    if (i < nb) dB[i] = 0.0f;
}

}  // namespace

uint32_t merge_chunks(int64_t slots) {
    if (slots <= (int64_t)kMergeOneChunk) return 1;
    return (uint32_t)((slots + kMergeChunk - 1) / kMergeChunk);
}

hipError_t launch_merge(const float *partials, double *chunk_sums, int32_t n_groups, int32_t m,
                        int32_t n, int64_t tiles, int64_t bundles, int32_t parts, int32_t narrow_dg,
                        int32_t narrow_cpb, float *dA, float *dB, hipStream_t s) {
    const int32_t na = m + 1, nc = m + 1 + n;
    const int64_t slots = (int64_t)parts * 8 * bundles;
    SlotMap sm;
    sm.tiles = (uint32_t)tiles;
    sm.bundles = (uint32_t)bundles;
    sm.per_part = 8u * (uint32_t)bundles;
    sm.div_part = make_fastdiv(sm.per_part);
    sm.div_bundles = make_fastdiv(sm.bundles);
    const dim3 grid_gk((unsigned)(n_groups * nc));
    if (slots <= (int64_t)kSmallChunk) {
        const uint32_t n_gk = (uint32_t)(n_groups * nc);
        const dim3 grid((n_gk + kWaveMergeThreads / 64 - 1) / (kWaveMergeThreads / 64));
        const uint32_t sl = (uint32_t)slots;
        if (slots <= 64 * 8)
            hipLaunchKernelGGL(grkan_merge_wave_kernel<8>, grid, dim3(kWaveMergeThreads), 0, s, partials,
                               sm, sl, na, n, narrow_dg, narrow_cpb, n_gk, dA, dB);
        else if (slots <= 64 * 16)
            hipLaunchKernelGGL(grkan_merge_wave_kernel<16>, grid, dim3(kWaveMergeThreads), 0, s, partials,
                               sm, sl, na, n, narrow_dg, narrow_cpb, n_gk, dA, dB);
        else
            hipLaunchKernelGGL(grkan_merge_wave_kernel<kWaveLoads>, grid, dim3(kWaveMergeThreads), 0, s, partials,
                               sm, sl, na, n, narrow_dg, narrow_cpb, n_gk, dA, dB);
        return hipGetLastError();
    }
    const uint32_t chunks = merge_chunks(slots);
    if (chunks == 1) {
        if (slots <= (int64_t)kMergeChunk)
            hipLaunchKernelGGL((grkan_merge_kernel<kMergeThreads, kMergeLoads>), grid_gk, dim3(kMergeThreads), 0, s,
                               partials, sm, (uint32_t)slots, na, n, narrow_dg, narrow_cpb, 1u, chunk_sums, dA, dB);
        else
            hipLaunchKernelGGL((grkan_merge_kernel<kMergeThreads, kMergeLoadsOne>), grid_gk, dim3(kMergeThreads), 0,
                               s, partials, sm, (uint32_t)slots, na, n, narrow_dg, narrow_cpb, 1u, chunk_sums, dA, dB);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((grkan_merge_kernel<kMergeThreads, kMergeLoads>), dim3(grid_gk.x, chunks), dim3(kMergeThreads),
                       0, s, partials, sm, (uint32_t)slots, na, n, narrow_dg, narrow_cpb, chunks, chunk_sums, dA, dB);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(grkan_merge_chunks_kernel, grid_gk, dim3(kChunkThreads), 0, s, chunk_sums, chunks, na,
                       n, dA, dB);
    return hipGetLastError();
}

hipError_t launch_zero(float *dA, float *dB, int64_t na, int64_t nb, hipStream_t s) {
    const int64_t n = na > nb ? na : nb;
    const int64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(grkan_zero_kernel, dim3((unsigned)(blocks > 0 ? blocks : 1)), dim3(256), 0, s,
                       dA, dB, na, nb);
    return hipGetLastError();
}

}  // namespace grkan
