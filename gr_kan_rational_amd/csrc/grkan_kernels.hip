// grkan_kernels.hip -- GR-KAN / PAU forward and backward kernels for gfx950
// (MI355X), for one degree pair (GRKAN_M, GRKAN_N).  The build compiles this
// file once per pair listed in GRKAN_FOR_EACH_DEGREE (grkan_launch.h).
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
//   * One workgroup per (tile, group, column part), short-lived: it issues
//     all its 16-byte loads at once, computes, stores and exits.  A large
//     grid of such workgroups, dispatched in order, keeps the set of
//     addresses in flight small and moving forward through memory, which HBM
//     serves best; a persistent loop would also wait, each iteration, for the
//     previous iteration's stores (gfx9 counts stores and loads in one
//     counter).
//   * The dispatcher deals consecutive workgroups round-robin to the 8 XCDs;
//     the grid is laid out so that XCD (x mod 8) takes whole row tiles (all
//     groups and parts of tiles x mod 8, +8, +16, ...).  The 8 XCDs then work
//     on different rows at any moment rather than all on the same ones.
//   * A 2D block of (vector column, row) lanes: each wave reads whole
//     128-byte lines, and a lane's group -- hence coefficients, which sit in
//     scalar registers -- is the workgroup's.  Block coordinates give the
//     lane's column and row, and the workgroup index is split into tile,
//     group and part by multiply-high divisions on the scalar unit: no
//     vector integer division anywhere.
//   * Every access goes through a window (base, length): the ragged last
//     tile and ragged column parts are cut off by one compare per access
//     (loads give zeros, stores are skipped), so full and partial tiles run
//     the same code.
//   * Backward: the tile's gradient terms are summed in fp32 registers (at
//     most 16 terms per lane), then across the workgroup through LDS, and
//     leave the workgroup as one fp32 atomic per coefficient (as in the
//     pages' Algorithm 2) or as one partial per coefficient merged afterwards
//     in fp64 in a fixed order (the two-stage reduction of [PolyKAN]), which
//     is bitwise reproducible: the tiling depends only on the shape.
#include "grkan_device.h"
#include "grkan_launch.h"

#ifndef GRKAN_M
#error "compile with -DGRKAN_M=<numerator degree> -DGRKAN_N=<denominator degree>"
#endif

namespace grkan {

namespace {

constexpr int kMaxBlock = 1024;

// Tuning, chosen by measurement on MI355X at the KAT-B shapes.  U = passes
// per workgroup (all of a lane's loads are issued together).  The backward
// prefers small blocks (with ~90 VGPRs a SIMD holds 5 of its waves; 3-wave
// blocks fill those slots in finer steps than 6-wave ones) and 4 passes to
// amortise the block reduction; the bf16 backward, which is bound by its
// arithmetic rather than by memory, and high-degree fp32 backwards, which
// need more registers per element, use 2 passes.
template <class IO> constexpr bool is_f32() { return __is_same(IO, float); }
template <class IO, int M, int N> constexpr int fwd_unroll() { return 2; }
template <class IO, int M, int N> constexpr int bwd_unroll() {
    return (is_f32<IO>() && M + N <= 9) ? 4 : 2;
}
constexpr int kFwdBlock = 384;
constexpr int kBwdBlock = 192;
// One fp32 atomic per coefficient per workgroup serialises on the few cache
// lines of dA and dB in L2, so the atomic mode uses 4x larger workgroups.
constexpr int kAtomicModeBlock = 768;

// Workgroup position: (tile, group, part) from the grid coordinates; false
// for the padding workgroups of the last bundle of 8 tiles.
struct Pos {
    int64_t tile;
    int g;
    int part;
};

__device__ static inline bool pos_of(const Plan &P, int64_t bundle0, Pos &p) {
    const uint32_t b = blockIdx.x;
    const uint32_t k = b >> 3;
    const uint32_t bundle = fastdiv(k, P.div_gp);
    const uint32_t gp = k - bundle * (uint32_t)(P.parts * P.n_groups);
    const uint32_t g = fastdiv(gp, P.div_parts);
    p.g = (int)g;
    p.part = (int)(gp - g * (uint32_t)P.parts);
    p.tile = (bundle0 + (int64_t)bundle) * 8 + (b & 7);
    return p.tile < P.tiles;
}

// Byte offset of the workgroup's first vector (uniform) and the lane's offset
// from it; lanes of a ragged last part that fall outside the segment get an
// offset the range check rejects.
struct Window {
    int64_t base;     // bytes from the tensor start
    int64_t avail;    // bytes from base to the tensor end
    uint32_t lane;    // this lane's byte offset from base, pass 0
    uint32_t stride;  // bytes between passes (rows_per_iter rows)
};

template <int U>
__device__ static inline Window window_of(const Plan &P, const Pos &p) {
    Window w;
    const int64_t row0 = p.tile * (int64_t)(U * P.rows_per_iter);
    w.base = row0 * P.row_bytes + (int64_t)p.g * P.seg_bytes + (int64_t)p.part * P.part_vecs * 16;
    w.avail = P.rows * P.row_bytes - w.base;
    const int col = (int)threadIdx.x;
    const int valid = P.seg_vecs - p.part * P.part_vecs;  // vectors of this part in the segment
    w.lane = (col < valid) ? (uint32_t)threadIdx.y * (uint32_t)P.row_bytes + (uint32_t)col * 16u
                           : kOffsetOutOfRange;
    w.stride = (uint32_t)P.rows_per_iter * (uint32_t)P.row_bytes;
    return w;
}

template <class T>
__device__ static inline T *at(T *p, int64_t bytes) {
    return reinterpret_cast<T *>(reinterpret_cast<char *>(p) + bytes);
}
template <class T>
__device__ static inline const T *at(const T *p, int64_t bytes) {
    return reinterpret_cast<const T *>(reinterpret_cast<const char *>(p) + bytes);
}

// ----------------------------------------------------------------- forward

template <class IO, int M, int N, int U>
__global__ __launch_bounds__(kMaxBlock) void grkan_fwd_kernel(FwdArgs a) {
    using V = Io<IO>;
    constexpr int E = V::kElems;
    const Plan &P = a.plan;
    Pos p;
    if (!pos_of(P, a.bundle0, p)) return;
    const Coefs<M, N> c = load_coefs<M, N>(a.A, a.B, p.g);
    const Window w = window_of<U>(P, p);
    const Span rx = make_span(at(a.x, w.base), w.avail);
    const Span ry = make_span(at(a.y, w.base), w.avail);

    u32x4 in[U];
#pragma unroll
    for (int u = 0; u < U; ++u) in[u] = win_load16(rx, w.lane + u * w.stride);
#pragma unroll
    for (int u = 0; u < U; ++u) {
        float f[E];
        V::unpack(in[u], f);
#pragma unroll
        for (int e = 0; e < E; ++e) f[e] = rational<M, N>(f[e], c);
        win_store16(ry, w.lane + u * w.stride, V::pack(f));
    }
}

// ---------------------------------------------------------------- backward

// One tile's elements: dX stored, this lane's gradient sums in acc.  The rare
// exact-sign fix runs once per tile, before any dX is stored; it re-reads x
// and dy, which is safe even when dx aliases x or dy.
template <class IO, int M, int N, int U, bool QZERO>
__device__ static inline void bwd_tile(Span rx, Span rdy, Span rdx, const Window &w,
                                       const BwdCoefs<M, N> &k, float (&acc)[Deg<M, N>::kNumCoef]) {
    using V = Io<IO>;
    constexpr int E = V::kElems;
    constexpr int K = Deg<M, N>::kTop;

    u32x4 xin[U], din[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        xin[u] = win_load16(rx, w.lane + u * w.stride);
        din[u] = win_load16(rdy, w.lane + u * w.stride);
    }
    float dxf[U][E];
    bool sure = true;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        // The two tile variants start with the same arithmetic; without this
        // empty asm barrier the compiler hoists it above the uniform branch
        // that picks the variant, for all of the tile's elements at once,
        // which costs ~30 registers.
        if constexpr (QZERO && N > 0) asm volatile("" : "+v"(xin[u]), "+v"(din[u]));
        float xf[E], dyf[E];
        V::unpack(xin[u], xf);
        V::unpack(din[u], dyf);
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const Pow<K> X(xf[e]);
            const float dy = dyf[e];
            if constexpr (QZERO) {
                // Q == 0: D = 1, s = 0: dX = dY P', dA terms dY x^i, no dB terms.
                float Pd = (M >= 1) ? k.da[0] : 0.0f;
#pragma unroll
                for (int i = 2; i <= M; ++i) Pd = fmaf(k.da[i - 1], X.p[i - 1], Pd);
                dxf[u][e] = dy * Pd;
                accumulate<M, N>(dy, 0.0f, X, acc);
            } else {
                const ElemBwd eb = backward_element<M, N, K>(X, dy, k);
                accumulate<M, N>(eb.w, eb.sv, X, acc);
                dxf[u][e] = eb.dx;
                sure = sure && eb.sure;
            }
        }
    }
    if constexpr (!QZERO) {
        // Rare: some element's sign of Q was not proven by the fp32 guard.
        // Re-read the tile (dx has not been written yet, so this is safe when
        // dx aliases x or dy) and fix those elements before storing.
        if (__builtin_expect(!sure, 0)) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float xf[E], dyf[E];
                V::unpack(win_reload16(rx, w.lane + u * w.stride), xf);
                V::unpack(win_reload16(rdy, w.lane + u * w.stride), dyf);
#pragma unroll
                for (int e = 0; e < E; ++e) dxf[u][e] = exact_fix<M, N>(xf[e], dyf[e], k, acc);
            }
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) win_store16(rdx, w.lane + u * w.stride, V::pack(dxf[u]));
}

// Slot of a tile's partial within its part: tiles of one XCD side by side.
__device__ static inline int64_t slot_in_part(const Plan &P, int64_t tile) {
    return (tile & 7) * P.bundles + (tile >> 3);
}

template <class IO, int M, int N, int U>
__global__ __launch_bounds__(kMaxBlock) void grkan_bwd_kernel(BwdArgs a) {
    constexpr int NC = Deg<M, N>::kNumCoef;
    const Plan &P = a.plan;
    Pos p;
    if (!pos_of(P, a.bundle0, p)) return;
    const BwdCoefs<M, N> k = derive<M, N>(load_coefs<M, N>(a.A, a.B, p.g));
    const Window w = window_of<U>(P, p);
    const Span rx = make_span(at(a.x, w.base), w.avail);
    const Span rdy = make_span(at(a.dy, w.base), w.avail);
    const Span rdx = make_span(at(a.dx, w.base), w.avail);
    float acc[NC];
#pragma unroll
    for (int i = 0; i < NC; ++i) acc[i] = 0.0f;
    if (k.q_zero) {
        bwd_tile<IO, M, N, U, true>(rx, rdy, rdx, w, k, acc);
    } else {
        if constexpr (N > 0) bwd_tile<IO, M, N, U, false>(rx, rdy, rdx, w, k, acc);
    }

    // Workgroup sum of the NC terms, in a fixed order: transposed through LDS
    // (lane sums -> red[k][lane], zero-padded to whole waves); 16 threads per
    // coefficient add nbp/16 consecutive lanes each in fp32; thread k adds its
    // coefficient's 16 slices in fp64.  About 13 VALU operations per lane for
    // GR-KAN's 10 sums, against 60 for DPP sums of the ten values across each
    // wave (measured faster on MI355X, where the backward's VALU load and
    // power draw matter).
    extern __shared__ float red[];  // [NC][nbp], then [NC][16] slices
    const int nb = (int)(blockDim.x * blockDim.y);
    const int nbp = (nb + 63) & ~63;
    const int t = (int)(threadIdx.y * blockDim.x + threadIdx.x);
#pragma unroll
    for (int i = 0; i < NC; ++i) red[i * nbp + t] = acc[i];
    for (int q = t; q < nbp - nb; q += nb) {
#pragma unroll
        for (int i = 0; i < NC; ++i) red[i * nbp + nb + q] = 0.0f;
    }
    __syncthreads();
    float *slices = red + NC * nbp;
    const int per = nbp / 16;  // a multiple of 4
    for (int idx = t; idx < NC * 16; idx += nb) {
        const int kk = idx >> 4, seg = idx & 15;
        const float4 *src = reinterpret_cast<const float4 *>(red + kk * nbp + seg * per);
        float slice = 0.0f;
        for (int j = 0; j < per / 4; ++j) {
            const float4 q = src[j];
            slice += ((q.x + q.y) + q.z) + q.w;
        }
        slices[idx] = slice;
    }
    __syncthreads();
    if (t < NC) {
        double total = 0.0;
#pragma unroll
        for (int j = 0; j < 16; ++j) total += (double)slices[t * 16 + j];
        if (a.mode == kModePartials) {
            const int64_t slot = (int64_t)p.part * 8 * P.bundles + slot_in_part(P, p.tile);
            a.partials[((int64_t)p.g * NC + t) * plan_slots(P) + slot] = (float)total;
        } else {
            float *dst = (t <= M) ? (a.dA + p.g * (M + 1) + t) : (a.dB + p.g * N + (t - M - 1));
            unsafeAtomicAdd(dst, (float)total);
        }
    }
}

// ------------------------------------------------------ narrow groups
//
// Groups whose row segment is not a whole number of 16-byte vectors (down to
// one function per channel).  Lane (x, y) of a 64 x kNarrowRowLanes block owns
// channel column c = 64 cb + x of the row tile, with that channel's
// coefficients in its own registers, and walks rows y, y + kNarrowRowLanes,
// ... of the tile in batches of U rows (loads issued together).  Each wave
// reads 64 consecutive elements (256 or 128 bytes) per row.  The workgroup
// then sums its lanes' terms over the row lanes and over the channels of
// each group it touches, and writes one partial per (group, coefficient,
// column block, tile).  Tiles are long (kNarrowRowLanes U iters rows) so
// that these partials stay a small fraction of the traffic even with one
// group per channel.

constexpr int kNarrowCols = 64;
constexpr int kNarrowRowLanes = 4;
constexpr int kNarrowThreads = kNarrowCols * kNarrowRowLanes;
constexpr int kNarrowUnroll = 4;
// Tiles of 128 rows (forward) and 512 rows (backward: with one group per
// channel the partials are then below 1% of the backward's traffic).
constexpr int kNarrowFwdIters = 128 / (kNarrowRowLanes * kNarrowUnroll);
constexpr int kNarrowBwdIters = 512 / (kNarrowRowLanes * kNarrowUnroll);

struct NarrowPos {
    int64_t tile;
    int cb;
};

__device__ static inline NarrowPos narrow_pos(const Plan &P, int64_t tile0) {
    const uint32_t b = blockIdx.x;
    const uint32_t t = fastdiv(b, P.div_ncb);
    NarrowPos p;
    p.cb = (int)(b - t * (uint32_t)P.ncb);
    p.tile = tile0 + t;
    return p;
}

template <int U, int K>
__device__ static inline Window narrow_window(const Plan &P, const NarrowPos &p, int64_t &ch) {
    Window w;
    const int64_t row0 = p.tile * (int64_t)(kNarrowRowLanes * U * K);
    w.base = row0 * P.row_bytes + (int64_t)p.cb * kNarrowCols * P.es;
    w.avail = P.rows * P.row_bytes - w.base;
    ch = (int64_t)p.cb * kNarrowCols + threadIdx.x;
    w.lane = (ch < P.d) ? (uint32_t)threadIdx.y * (uint32_t)P.row_bytes + (uint32_t)threadIdx.x * (uint32_t)P.es
                        : kOffsetOutOfRange;
    w.stride = (uint32_t)kNarrowRowLanes * (uint32_t)P.row_bytes;
    return w;
}

// Group of this lane's channel (group 0 for lanes past the row, whose
// accesses are all skipped).
__device__ static inline int narrow_group(const Plan &P, int64_t ch) {
    return ch < P.d ? (int)fastdiv((uint32_t)ch, P.div_dg) : 0;
}

template <class IO, int M, int N, int U, int K>
__global__ __launch_bounds__(kNarrowThreads) void grkan_fwd_narrow_kernel(FwdArgs a) {
    using V = Elem<IO>;
    const Plan &P = a.plan;
    const NarrowPos p = narrow_pos(P, a.bundle0);
    if (p.tile >= P.tiles) return;
    int64_t ch;
    const Window w = narrow_window<U, K>(P, p, ch);
    const Coefs<M, N> c = load_coefs<M, N>(a.A, a.B, narrow_group(P, ch));
    const Span sx = make_span(at(a.x, w.base), w.avail);
    const Span sy = make_span(at(a.y, w.base), w.avail);
    for (int it = 0; it < K; ++it) {
        float f[U];
#pragma unroll
        for (int u = 0; u < U; ++u) f[u] = V::load(sx, w.lane + (it * U + u) * w.stride);
#pragma unroll
        for (int u = 0; u < U; ++u) V::store(sy, w.lane + (it * U + u) * w.stride, rational<M, N>(f[u], c));
    }
}

template <class IO, int M, int N, int U, int K>
__global__ __launch_bounds__(kNarrowThreads) void grkan_bwd_narrow_kernel(BwdArgs a) {
    using V = Elem<IO>;
    constexpr int NC = Deg<M, N>::kNumCoef;
    constexpr int KP = Deg<M, N>::kTop;
    const Plan &P = a.plan;
    const NarrowPos p = narrow_pos(P, a.bundle0);
    if (p.tile >= P.tiles) return;
    int64_t ch;
    const Window w = narrow_window<U, K>(P, p, ch);
    const BwdCoefs<M, N> k = derive<M, N>(load_coefs<M, N>(a.A, a.B, narrow_group(P, ch)));
    const Span sx = make_span(at(a.x, w.base), w.avail);
    const Span sdy = make_span(at(a.dy, w.base), w.avail);
    const Span sdx = make_span(at(a.dx, w.base), w.avail);

    // Sums per channel: fp32 over one batch (U terms), then fp32 across the
    // batches (iters terms): no fp32 chain longer than 32.
    float acc[NC];
#pragma unroll
    for (int i = 0; i < NC; ++i) acc[i] = 0.0f;
    for (int it = 0; it < K; ++it) {
        float xf[U], dyf[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            xf[u] = V::load(sx, w.lane + (it * U + u) * w.stride);
            dyf[u] = V::load(sdy, w.lane + (it * U + u) * w.stride);
        }
        float part[NC];
#pragma unroll
        for (int i = 0; i < NC; ++i) part[i] = 0.0f;
        float dxf[U];
        bool sure = true;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const Pow<KP> X(xf[u]);
            const ElemBwd eb = backward_element<M, N, KP>(X, dyf[u], k);
            accumulate<M, N>(eb.w, eb.sv, X, part);
            dxf[u] = eb.dx;
            sure = sure && eb.sure;
        }
        if constexpr (N > 0) {
            // Rare: an element whose sign of Q the fp32 guard did not prove
            // (x == 0, a root of Q, or b = 0 in its group): fix the batch.
            if (__builtin_expect(!sure, 0)) {
#pragma unroll
                for (int u = 0; u < U; ++u) dxf[u] = exact_fix<M, N>(xf[u], dyf[u], k, part);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) V::store(sdx, w.lane + (it * U + u) * w.stride, dxf[u]);
#pragma unroll
        for (int i = 0; i < NC; ++i) acc[i] += part[i];
    }

    // Workgroup sums in a fixed order: per channel over the row lanes, then
    // per group over its channels in this column block, in fp64.
    __shared__ float red[NC * kNarrowRowLanes * kNarrowCols];
    __shared__ double ct[NC * kNarrowCols];
    const int x = (int)threadIdx.x, y = (int)threadIdx.y;
    const int t = y * kNarrowCols + x;
#pragma unroll
    for (int i = 0; i < NC; ++i) red[(i * kNarrowRowLanes + y) * kNarrowCols + x] = acc[i];
    __syncthreads();
    for (int idx = t; idx < NC * kNarrowCols; idx += kNarrowThreads) {
        const int i = idx / kNarrowCols, xx = idx % kNarrowCols;
        double s = 0.0;
#pragma unroll
        for (int yy = 0; yy < kNarrowRowLanes; ++yy) s += (double)red[(i * kNarrowRowLanes + yy) * kNarrowCols + xx];
        ct[idx] = s;
    }
    __syncthreads();
    const int64_t c0 = (int64_t)p.cb * kNarrowCols;
    const int64_t c1 = (c0 + kNarrowCols < P.d) ? c0 + kNarrowCols : P.d;
    const int64_t g_lo = c0 / P.d_g, g_hi = (c1 - 1) / P.d_g;
    const int nlg = (int)(g_hi - g_lo + 1);
    for (int idx = t; idx < nlg * NC; idx += kNarrowThreads) {
        const int64_t gg = g_lo + idx / NC;
        const int i = idx % NC;
        const int64_t lo = (gg * P.d_g > c0 ? gg * P.d_g : c0) - c0;
        const int64_t hi = ((gg + 1) * P.d_g < c1 ? (gg + 1) * P.d_g : c1) - c0;
        double s = 0.0;
        for (int64_t c = lo; c < hi; ++c) s += ct[i * kNarrowCols + c];
        if (a.mode == kModePartials) {
            const int64_t part = (int64_t)p.cb - gg * P.d_g / P.cpb;
            const int64_t slot = part * 8 * P.bundles + slot_in_part(P, p.tile);
            a.partials[(gg * NC + i) * plan_slots(P) + slot] = (float)s;
        } else {
            float *dst = (i <= M) ? (a.dA + gg * (M + 1) + i) : (a.dB + gg * N + (i - M - 1));
            unsafeAtomicAdd(dst, (float)s);
        }
    }
}

template <class IO, int M, int N>
hipError_t fwd_impl(const FwdArgs &a, dim3 grid, hipStream_t s) {
    if (a.plan.kind == kNarrow) {
        hipLaunchKernelGGL((grkan_fwd_narrow_kernel<IO, M, N, kNarrowUnroll, kNarrowFwdIters>), grid,
                           dim3(kNarrowCols, kNarrowRowLanes), 0, s, a);
        return hipGetLastError();
    }
    const dim3 block((unsigned)a.plan.part_vecs, (unsigned)a.plan.rows_per_iter);
    hipLaunchKernelGGL((grkan_fwd_kernel<IO, M, N, fwd_unroll<IO, M, N>()>), grid, block, 0, s, a);
    return hipGetLastError();
}

template <int M, int N>
size_t bwd_lds_bytes(int block) {
    const int nbp = (block + 63) & ~63;
    return (size_t)Deg<M, N>::kNumCoef * (nbp + 16) * sizeof(float);
}

template <class IO, int M, int N>
hipError_t bwd_impl(const BwdArgs &a, dim3 grid, hipStream_t s) {
    if (a.plan.kind == kNarrow) {
        hipLaunchKernelGGL((grkan_bwd_narrow_kernel<IO, M, N, kNarrowUnroll, kNarrowBwdIters>), grid,
                           dim3(kNarrowCols, kNarrowRowLanes), 0, s, a);
        return hipGetLastError();
    }
    const dim3 block((unsigned)a.plan.part_vecs, (unsigned)a.plan.rows_per_iter);
    const size_t lds = bwd_lds_bytes<M, N>(a.plan.block);
    hipLaunchKernelGGL((grkan_bwd_kernel<IO, M, N, bwd_unroll<IO, M, N>()>), grid, block, lds, s, a);
    return hipGetLastError();
}

}  // namespace

template <int M, int N>
int Kernels<M, N>::unroll(grkan_dtype_t io, int pass) {
    if (io == GRKAN_BF16) return pass ? bwd_unroll<bf16io, M, N>() : fwd_unroll<bf16io, M, N>();
    return pass ? bwd_unroll<float, M, N>() : fwd_unroll<float, M, N>();
}

template <int M, int N>
void Kernels<M, N>::narrow_shape(grkan_dtype_t, int pass, int *row_lanes, int *unroll, int *iters) {
    *row_lanes = kNarrowRowLanes;
    *unroll = kNarrowUnroll;
    *iters = pass ? kNarrowBwdIters : kNarrowFwdIters;
}

template <int M, int N>
int Kernels<M, N>::target_block(grkan_dtype_t, int pass, bool atomic_mode) {
    if (pass == 1 && atomic_mode) return kAtomicModeBlock;
    return pass ? kBwdBlock : kFwdBlock;
}

template <int M, int N>
hipError_t Kernels<M, N>::forward(grkan_dtype_t io, const FwdArgs &a, dim3 grid, hipStream_t s) {
    return io == GRKAN_BF16 ? fwd_impl<bf16io, M, N>(a, grid, s) : fwd_impl<float, M, N>(a, grid, s);
}

template <int M, int N>
hipError_t Kernels<M, N>::backward(grkan_dtype_t io, const BwdArgs &a, dim3 grid, hipStream_t s) {
    return io == GRKAN_BF16 ? bwd_impl<bf16io, M, N>(a, grid, s) : bwd_impl<float, M, N>(a, grid, s);
}

template <int M, int N>
hipError_t Kernels<M, N>::occupancy(grkan_dtype_t io, int pass, int block, int *blocks_per_cu, bool narrow) {
    if (narrow) {
        const void *fn;
        if (io == GRKAN_BF16)
            fn = pass ? (const void *)grkan_bwd_narrow_kernel<bf16io, M, N, kNarrowUnroll, kNarrowBwdIters>
                      : (const void *)grkan_fwd_narrow_kernel<bf16io, M, N, kNarrowUnroll, kNarrowFwdIters>;
        else
            fn = pass ? (const void *)grkan_bwd_narrow_kernel<float, M, N, kNarrowUnroll, kNarrowBwdIters>
                      : (const void *)grkan_fwd_narrow_kernel<float, M, N, kNarrowUnroll, kNarrowFwdIters>;
        return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, fn, kNarrowThreads, 0);
    }
    const void *fn;
    const size_t lds = pass ? bwd_lds_bytes<M, N>(block) : 0;
    if (io == GRKAN_BF16)
        fn = pass ? (const void *)grkan_bwd_kernel<bf16io, M, N, bwd_unroll<bf16io, M, N>()>
                  : (const void *)grkan_fwd_kernel<bf16io, M, N, fwd_unroll<bf16io, M, N>()>;
    else
        fn = pass ? (const void *)grkan_bwd_kernel<float, M, N, bwd_unroll<float, M, N>()>
                  : (const void *)grkan_fwd_kernel<float, M, N, fwd_unroll<float, M, N>()>;
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, fn, block, lds);
}

template struct Kernels<GRKAN_M, GRKAN_N>;

}  // namespace grkan
