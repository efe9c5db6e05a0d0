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
#include <type_traits>

#include "grkan_device.h"
#include "grkan_launch.h"

#ifndef GRKAN_M
#error "compile with -DGRKAN_M=<numerator degree> -DGRKAN_N=<denominator degree>"
#endif

namespace grkan {

namespace {

constexpr int kMaxBlock = 1024;

// Tuning, chosen by measurement on MI355X at the KAT-B shapes.  U = passes
// per workgroup (all of a lane's loads are issued together).  Forward: 2
// passes, 384-lane blocks.  The fp32 backward at GR-KAN-sized degrees: 2
// passes, 384-lane blocks (292 us; 4 passes of 192 lanes -- the same 32-row
// tiles -- 302 us, 2 x 192 303, 2 x 768 293, 3 x 384 295, 1 x 384 327; 4 x 384
// with the passes kept apart 626 against 599 us at KAT-S hidden).  High-degree
// fp32 backwards, which need more registers per element: 2 passes, 192-lane
// blocks.  The bf16 backward, which is bound by its arithmetic rather than by
// memory: 4 passes of 192 lanes (32 elements per lane, so the per-lane work of
// the reduction and set-up is spread over twice as many elements: 749 against
// 771 us at KAT-B hidden), its passes kept apart by a scheduling barrier (80
// VGPRs; 62 at 2 passes, 88 without the barrier).
template <class IO> constexpr bool is_f32() { return __is_same(IO, float); }
template <class IO, int M, int N> constexpr int fwd_unroll() { return 2; }
template <class IO, int M, int N> constexpr int bwd_unroll() { return is_f32<IO>() ? 2 : 4; }
// Small grids (fewer workgroups than kSmallGrid at the passes above, e.g. the
// KAT-T shape with 1,600): half the passes, so that twice as many shorter
// workgroups run in about two rounds and one round's loads overlap the other's
// arithmetic instead of every workgroup loading, then computing, at once.
// KAT-T backward 24.1 against 26.7-29.1 us (the same at KAT-B sizes would be
// 20% slower).
template <class IO, int M, int N> constexpr int fwd_unroll_small() { return 1; }
template <class IO, int M, int N> constexpr int bwd_unroll_small() { return is_f32<IO>() ? 1 : 2; }
template <class IO, int M, int N> constexpr bool bwd_wide_block() { return is_f32<IO>() && M + N <= 9; }
constexpr int kFwdBlock = 384;
constexpr int kBwdBlock = 192;
constexpr int kBwdWideBlock = 384;
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
    bool full;        // every lane's every access is inside the tensor (uniform)
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
    w.full = valid >= P.part_vecs && row0 + U * P.rows_per_iter <= P.rows;
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

// ------------------------------------------------- FLOP-inflation probe
//
// [FlashKAT notes] (section "1. 性能瓶颈诊断", Insight 2) multiply the
// rational's arithmetic by 8 with nested loops and find the run time
// unchanged: the activation's FLOPs are not what limits it.  The same probe
// here: with R > 1 every element is evaluated R - 1 extra times before the
// evaluation whose results are used.  Each extra evaluation starts from a
// copy of x passed through an empty asm statement, so the compiler can
// neither share its arithmetic with the real evaluation nor fold it away, and
// hands its results to another empty asm statement, so it is not dropped as
// dead.  Outputs are those of R = 1 bit for bit; only the arithmetic per
// element grows.  The gradient terms are accumulated once.

template <class T> __device__ static inline T opaque(T v) {
    asm volatile("" : "+v"(v));
    return v;
}

template <int M, int N, int R>
__device__ static inline void burn_forward(float x, const Coefs<M, N> &c) {
#pragma unroll
    for (int r = 1; r < R; ++r) {
        const float y = rational<M, N>(opaque(x), c);
        asm volatile("" ::"v"(y));
    }
}

template <int M, int N, int K, int R, bool QZERO>
__device__ static inline void burn_backward(float x, float dy, const BwdCoefs<M, N> &k, const QWide<N> &kw) {
#pragma unroll
    for (int r = 1; r < R; ++r) {
        const Pow<K> X(opaque(x));
        if constexpr (QZERO) {
            float Pd = (M >= 1) ? k.da[0] : 0.0f;
#pragma unroll
            for (int i = 2; i <= M; ++i) Pd = fmaf(k.da[i - 1], X.p[i - 1], Pd);
            asm volatile("" ::"v"(dy * Pd));
        } else {
            const ElemBwd e = backward_element<M, N, K>(X, dy, k, kw);
            asm volatile("" ::"v"(e.dx), "v"(e.w), "v"(e.sv), "v"(e.sure ? 1 : 0));
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// ----------------------------------------------------------------- forward

template <class IO, int M, int N, int U, bool CHECK, int R = 1>
__device__ static inline void fwd_tile(Span rx, Span ry, const Window &w, const Coefs<M, N> &c) {
    using V = Io<IO>;
    constexpr int E = V::kElems;
    u32x4 in[U];
#pragma unroll
    for (int u = 0; u < U; ++u) in[u] = win_load16<CHECK>(rx, w.lane + u * w.stride);
#pragma unroll
    for (int u = 0; u < U; ++u) {
        float f[E];
        V::unpack(in[u], f);
#pragma unroll
        for (int e = 0; e < E; ++e) {
            if constexpr (R > 1) burn_forward<M, N, R>(f[e], c);
            f[e] = rational<M, N>(f[e], c);
        }
        win_store16<CHECK>(ry, w.lane + u * w.stride, V::pack(f));
    }
}

// R = 1: the plain forward; R = 2, 4, 8: the FLOP-inflation probe.
template <class IO, int M, int N, int U, int R>
__global__ __launch_bounds__(kMaxBlock) void grkan_fwd_kernel(FwdArgs a) {
    const Plan &P = a.plan;
    Pos p;
    if (!pos_of(P, a.bundle0, p)) return;
    const Coefs<M, N> c = load_coefs<M, N>(a.A, a.B, p.g);
    const Window w = window_of<U>(P, p);
    const Span rx = make_span(at(a.x, w.base), w.avail);
    const Span ry = make_span(at(a.y, w.base), w.avail);
    fwd_tile<IO, M, N, U, true, R>(rx, ry, w, c);
}


// ---------------------------------------------------------------- backward

// One tile's elements: dX stored, this lane's gradient sums in acc.  The rare
// sign fix runs once per tile, before any dX is stored; it re-reads x
// and dy, which is safe even when dx aliases x or dy.
// With WY, F(x) is stored too, through ry (which may be rdy: every load
// precedes every store).
template <int U>
__device__ static inline void load_pair(Span ra, Span rb, const Window &w, u32x4 (&a)[U], u32x4 (&b)[U]) {
    // Only the loads and stores differ between full and partial tiles, so only
    // they are branched on (a uniform branch); a second copy of the whole tile
    // for full tiles costs registers.
    if (w.full) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            a[u] = win_load16<false>(ra, w.lane + u * w.stride);
            b[u] = win_load16<false>(rb, w.lane + u * w.stride);
        }
    } else {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            a[u] = win_load16<true>(ra, w.lane + u * w.stride);
            b[u] = win_load16<true>(rb, w.lane + u * w.stride);
        }
    }
}

template <int U>
__device__ static inline void store_all(Span r, const Window &w, const u32x4 (&v)[U]) {
    if (w.full) {
#pragma unroll
        for (int u = 0; u < U; ++u) win_store16<false>(r, w.lane + u * w.stride, v[u]);
    } else {
#pragma unroll
        for (int u = 0; u < U; ++u) win_store16<true>(r, w.lane + u * w.stride, v[u]);
    }
}

template <class IO, int M, int N, int U, bool QZERO, int R = 1, bool WY = false>
__device__ static inline void bwd_tile(Span rx, Span rdy, Span rdx, const Window &w,
                                       const BwdCoefs<M, N> &k, const QWide<N> &kw,
                                       float (&acc)[Deg<M, N>::kNumCoef], Span ry = Span{}) {
    using V = Io<IO>;
    constexpr int E = V::kElems;
    constexpr int K = Deg<M, N>::kTop;

    u32x4 xin[U], din[U];
    load_pair<U>(rx, rdy, w, xin, din);
    float dxf[U][E];
    [[maybe_unused]] u32x4 ypk[WY ? U : 1];  // F, packed to the I/O type as each pass ends
    bool sure = true;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        // The two tile variants start with the same arithmetic; without this
        // empty asm barrier the compiler hoists it above the uniform branch
        // that picks the variant, for all of the tile's elements at once,
        // which costs ~30 registers.
        if constexpr (QZERO && N > 0) asm volatile("" : "+v"(xin[u]), "+v"(din[u]));
        float xf[E], dyf[E];
        [[maybe_unused]] float yf[E];
        V::unpack(xin[u], xf);
        V::unpack(din[u], dyf);
#pragma unroll
        for (int e = 0; e < E; ++e) {
            if constexpr (R > 1) burn_backward<M, N, K, R, QZERO>(xf[e], dyf[e], k, kw);
            const Pow<K> X(xf[e]);
            const float dy = dyf[e];
            if constexpr (QZERO) {
                // Q == 0: D = 1, s = 0: dX = dY P', dA terms dY x^i, no dB terms.
                float Pd = (M >= 1) ? k.da[0] : 0.0f;
#pragma unroll
                for (int i = 2; i <= M; ++i) Pd = fmaf(k.da[i - 1], X.p[i - 1], Pd);
                dxf[u][e] = dy * Pd;
                accumulate<M, N>(dy, 0.0f, X, acc);
                if constexpr (WY) {
                    float P = k.a[0];
#pragma unroll
                    for (int i = 1; i <= M; ++i) P = fmaf(k.a[i], X.p[i], P);
                    yf[e] = P;
                }
            } else {
                const ElemBwd eb = backward_element<M, N, K>(X, dy, k, kw);
                accumulate<M, N>(eb.w, eb.sv, X, acc);
                dxf[u][e] = eb.dx;
                if constexpr (WY) yf[e] = eb.F;
                sure = sure && eb.sure;
            }
        }
        if constexpr (WY) ypk[u] = V::pack(yf);
        if constexpr (!is_f32<IO>()) __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (!QZERO) {
        // Rare: some element's sign of Q was not proven by the fp32 guard.
        // Re-read the tile (dx has not been written yet, so this is safe when
        // dx aliases x or dy) and fix those elements before storing.
        if (__builtin_expect(!sure, 0)) {
            if constexpr (N >= kExactSignMinN) {
                // exact integer sign: one vector at a time, x and dy read
                // again after the sign loop rather than held across it
                const CoefHeld<M, N> src{k, kw};
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    uint32_t unsure, pos, neg;
                    {
                        float xf[E];
                        V::unpack(win_reload16<true>(rx, w.lane + u * w.stride), xf);
                        exact_signs<M, N, E>(xf, src, unsure, pos, neg);
                    }
                    float xf[E], dyf[E];
                    V::unpack(win_reload16<true>(rx, w.lane + u * w.stride), xf);
                    V::unpack(win_reload16<true>(rdy, w.lane + u * w.stride), dyf);
                    exact_apply<M, N, E>(xf, dyf, src, unsure, pos, neg, acc, dxf[u]);
                }
            } else {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    float xf[E], dyf[E];
                    V::unpack(win_reload16<true>(rx, w.lane + u * w.stride), xf);
                    V::unpack(win_reload16<true>(rdy, w.lane + u * w.stride), dyf);
#pragma unroll
                    for (int e = 0; e < E; ++e) dxf[u][e] = compensated_fix<M, N>(xf[e], dyf[e], k, kw, acc);
                }
            }
        }
    }
    u32x4 dxpk[U];
#pragma unroll
    for (int u = 0; u < U; ++u) dxpk[u] = V::pack(dxf[u]);
    store_all<U>(rdx, w, dxpk);
    if constexpr (WY) store_all<U>(ry, w, ypk);
}

// Slot of a tile's partial within its part: tiles of one XCD side by side.
__device__ static inline int64_t slot_in_part(const Plan &P, int64_t tile) {
    return (tile & 7) * P.bundles + (tile >> 3);
}

// Workgroup sum of the NC lane sums, in a fixed order, and its exit: one fp32
// partial per (group, coefficient, part, tile), or one fp32 atomic add per
// coefficient.
//   1. Each wave writes its lanes' sums to its own LDS rows [wave][NC][64]:
//      one base address per lane, the coefficient index in the instruction's
//      immediate offset.  Lanes a partial last wave lacks are zero-filled.
//   2. Slice s (0..15) of a coefficient is lanes 4s..4s+3 of every wave;
//      thread (k, s) adds slice s of coefficient k in fp32, wave by wave, one
//      16-byte LDS read per wave (consecutive threads read consecutive 16-byte
//      words: no bank conflicts).
//   3. Thread k adds its coefficient's 16 slices in fp64.
// About 4 vector instructions and 5 paired LDS writes per lane for step 1 and
// 5 per wave for step 2, against ~60 for DPP sums of ten values across each
// wave; the order
// depends only on the block shape, so the partials are bitwise reproducible.
template <int M, int N>
__device__ static inline void reduce_and_emit(const BwdArgs &a, const Plan &P, const Pos &p,
                                              const float (&acc)[Deg<M, N>::kNumCoef]) {
    constexpr int NC = Deg<M, N>::kNumCoef;
    extern __shared__ float4 red4[];  // [nw][NC][64] lane sums, then [NC][16] slices
    float *red = reinterpret_cast<float *>(red4);
    const int nb = (int)(blockDim.x * blockDim.y);
    const int nw = (nb + 63) >> 6;
    const int t = (int)(threadIdx.y * blockDim.x + threadIdx.x);
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int lane = t & 63;
    float *mine = red + wave * (NC * 64) + lane;
#pragma unroll
    for (int i = 0; i < NC; ++i) mine[i * 64] = acc[i];
    const int tail = nb & 63;  // lanes of a partial last wave (0: none)
    if (tail != 0) {
        const int missing = 64 - tail;
        float *last = red + (nw - 1) * (NC * 64);
        for (int q = t; q < NC * missing; q += nb) last[(q / missing) * 64 + tail + q % missing] = 0.0f;
    }
    __syncthreads();
    float *slices = red + nw * (NC * 64);
    for (int idx = t; idx < NC * 16; idx += nb) {
        // slice s = idx mod 16 of coefficient idx / 16: lanes 4s..4s+3 of every
        // wave, i.e. the 16-byte row element idx + j * NC * 16 for wave j
        const float4 *src = red4 + idx;
        float slice = 0.0f;
        for (int j = 0; j < nw; ++j, src += NC * 16) {
            const float4 q = *src;
            slice += ((q.x + q.y) + q.z) + q.w;
        }
        slices[idx] = slice;
    }
    __syncthreads();
    if (t < NC) {
        double total = 0.0;
#pragma unroll
        for (int j = 0; j < 16; ++j) total += (double)slices[t * 16 + j];
        float *dst = (t <= M) ? (a.dA + p.g * (M + 1) + t) : (a.dB + p.g * N + (t - M - 1));
        if (a.mode != kModeAtomic) {
            const int64_t slot = (int64_t)p.part * 8 * P.bundles + slot_in_part(P, p.tile);
            float *part = a.partials + ((int64_t)p.g * NC + t) * plan_slots(P) + slot;
            *(a.mode == kModeDirect ? dst : part) = (float)total;
        } else {
            unsafeAtomicAdd(dst, (float)total);
        }
    }
}

// R = 1: the plain backward; R = 2, 4, 8: the FLOP-inflation probe.  WY: F(x)
// is stored too (a.y), for the layer backward.
template <class IO, int M, int N, int U, int R, bool WY = false>
__global__ __launch_bounds__(kMaxBlock) void grkan_bwd_kernel(BwdArgs a) {
    constexpr int NC = Deg<M, N>::kNumCoef;
    const Plan &P = a.plan;
    Pos p;
    if (!pos_of(P, a.bundle0, p)) return;
    const Coefs<M, N> c = load_coefs<M, N>(a.A, a.B, p.g);
    const BwdCoefs<M, N> k = derive<M, N>(c);
    const QWide<N> kw = widen<M, N>(c);
    const Window w = window_of<U>(P, p);
    const Span rx = make_span(at(a.x, w.base), w.avail);
    const Span rdy = make_span(at(a.dy, w.base), w.avail);
    const Span rdx = make_span(at(a.dx, w.base), w.avail);
    float acc[NC];
#pragma unroll
    for (int i = 0; i < NC; ++i) acc[i] = 0.0f;
    const Span ry = WY ? make_span(at(a.y, w.base), w.avail) : Span{};
    if (k.q_zero) {
        bwd_tile<IO, M, N, U, true, R, WY>(rx, rdy, rdx, w, k, kw, acc, ry);
    } else {
        if constexpr (N > 0) bwd_tile<IO, M, N, U, false, R, WY>(rx, rdy, rdx, w, k, kw, acc, ry);
    }
    reduce_and_emit<M, N>(a, P, p, acc);
}

// ------------------------------------------------------ narrow groups
//
// Groups whose row segment is not a whole number of 16-byte vectors (down to
// one function per channel).  Lane (x, y) of a 64-column block owns channel
// column c = 64 cb + x of the row tile, with that channel's coefficients in
// its own registers; each wave reads 64 consecutive elements per row.  The
// forward loads all of a lane's rows (y, y + row lanes, ...) at once,
// computes, stores and exits, like the wide kernels; the backward walks its
// rows in batches (register limits, see below).  The backward workgroup then
// sums its lanes' terms over the row lanes and over the channels of each
// group it touches, and writes one partial per (group, coefficient, column
// block, tile).  Workgroup b takes tile 8 (b / (8 ncb)) + (b mod 8) and
// column block (b / 8) mod ncb, so that, as in the wide kernels, XCD (b mod 8)
// takes whole row tiles.
//
// Measured on MI355X with copy probes of this layout at KAT-B: 128-row
// one-shot tiles with that mapping streamed 6.1 TB/s, the same tiles dealt
// column block first 5.6 TB/s, lanes looping over 4-row batches 5.2 TB/s
// (128-row tiles) to 4.5 TB/s (512-row tiles).  The backward's tiles are 256
// rows: with one group per channel the partials are then ~1.3% of its
// traffic, written once and read once by the merge.

constexpr int kNarrowCols = 64;
constexpr int kNarrowRowLanes = 16;  // forward
constexpr int kNarrowThreads = kNarrowCols * kNarrowRowLanes;
// Backward: 4 row lanes, each walking 8 batches of 8 rows (256-row tiles)
// with the next batch's loads in flight.  The one-shot 128-row shape of the
// forward needs 1024-lane blocks, which run one per CU at the backward's
// register count and stall the CU during the workgroup reduction (440-460 us
// with one function per channel at KAT-B).  Batches x rows per batch, with
// the prefetch, at that workload (backward call, merge included): 8 x 4
// 390 us, 4 x 8 383, 16 x 4 372, 8 x 8 361 (chosen), 16 x 8 369, 32 x 4 373,
// 12 x 6 370, 12 x 8 377, 16 x 2 403; without the prefetch 8 x 4 took 396 us.
constexpr int kNarrowBwdRowLanes = 4;
constexpr int kNarrowBwdThreads = kNarrowCols * kNarrowBwdRowLanes;
constexpr int kNarrowBwdIters = 8;
template <int M, int N> constexpr int narrow_bwd_unroll() { return 8; }
// Forward rows per lane: 8 (128-row tiles); 4 for high degrees.
template <int M, int N> constexpr int narrow_unroll() { return M + N <= 9 ? 8 : 4; }

struct NarrowPos {
    int64_t tile;
    int cb;
};

__device__ static inline NarrowPos narrow_pos(const Plan &P, int64_t bundle0) {
    const uint32_t b = blockIdx.x;
    const uint32_t k = b >> 3;
    const uint32_t bundle = fastdiv(k, P.div_ncb);
    NarrowPos p;
    p.cb = (int)(k - bundle * (uint32_t)P.ncb);
    p.tile = (bundle0 + (int64_t)bundle) * 8 + (b & 7);
    return p;
}

// The column block lies wholly inside the row.
__device__ static inline bool c0_full(const Plan &P, const NarrowPos &p) {
    return (int64_t)(p.cb + 1) * kNarrowCols <= P.d;
}

template <int RW, int U, int K>
__device__ static inline Window narrow_window(const Plan &P, const NarrowPos &p, int64_t &ch) {
    Window w;
    const int64_t row0 = p.tile * (int64_t)(RW * U * K);
    w.base = row0 * P.row_bytes + (int64_t)p.cb * kNarrowCols * P.es;
    w.avail = P.rows * P.row_bytes - w.base;
    ch = (int64_t)p.cb * kNarrowCols + threadIdx.x;
    w.lane = (ch < P.d) ? (uint32_t)threadIdx.y * (uint32_t)P.row_bytes + (uint32_t)threadIdx.x * (uint32_t)P.es
                        : kOffsetOutOfRange;
    w.stride = (uint32_t)RW * (uint32_t)P.row_bytes;
    w.full = c0_full(P, p) && row0 + RW * U * K <= P.rows;
    return w;
}

// Group of this lane's channel (group 0 for lanes past the row, whose
// accesses are all skipped).
__device__ static inline int narrow_group(const Plan &P, int64_t ch) {
    return ch < P.d ? (int)fastdiv((uint32_t)ch, P.div_dg) : 0;
}

template <class IO, int M, int N, int U, bool CHECK>
__device__ static inline void narrow_fwd_rows(Span sx, Span sy, const Window &w, const Coefs<M, N> &c) {
    using V = Elem<IO>;
    float f[U];
#pragma unroll
    for (int u = 0; u < U; ++u) f[u] = V::template load<CHECK>(sx, w.lane + u * w.stride);
#pragma unroll
    for (int u = 0; u < U; ++u) V::template store<CHECK>(sy, w.lane + u * w.stride, rational<M, N>(f[u], c));
}

template <class IO, int M, int N>
__global__ __launch_bounds__(kNarrowThreads) void grkan_fwd_narrow_kernel(FwdArgs a) {
    using V = Elem<IO>;
    constexpr int U = narrow_unroll<M, N>();
    const Plan &P = a.plan;
    const NarrowPos p = narrow_pos(P, a.bundle0);
    if (p.tile >= P.tiles) return;
    int64_t ch;
    const Window w = narrow_window<kNarrowRowLanes, U, 1>(P, p, ch);
    const Coefs<M, N> c = load_coefs<M, N>(a.A, a.B, narrow_group(P, ch));
    const Span sx = make_span(at(a.x, w.base), w.avail);
    const Span sy = make_span(at(a.y, w.base), w.avail);
    if (w.full) narrow_fwd_rows<IO, M, N, U, false>(sx, sy, w, c);
    else narrow_fwd_rows<IO, M, N, U, true>(sx, sy, w, c);
}

// One lane's rows of a narrow tile, K batches of U rows: dX stored, the terms
// added to acc.  The next batch's loads are issued before the current batch
// is computed, so two batches (2 x U x 2 loads) are in flight per wave: a
// lane moves only one channel per row, and the reads in flight, not the
// arithmetic, decide this kernel's rate.
template <class IO, int M, int N, int U, int K, bool CHECK>
__device__ static inline void narrow_bwd_rows(Span sx, Span sdy, Span sdx, const Window &w,
                                              const BwdCoefs<M, N> &k, const QWide<N> &kw,
                                              float (&acc)[Deg<M, N>::kNumCoef]) {
    using V = Elem<IO>;
    constexpr int KP = Deg<M, N>::kTop;
    float xf[U], dyf[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        xf[u] = V::template load<CHECK>(sx, w.lane + u * w.stride);
        dyf[u] = V::template load<CHECK>(sdy, w.lane + u * w.stride);
        // keeps the two variants' arithmetic from being hoisted above the
        // branch between them (see bwd_tile)
        if constexpr (CHECK) asm volatile("" : "+v"(xf[u]), "+v"(dyf[u]));
    }
#pragma unroll
    for (int it = 0; it < K; ++it) {
        const uint32_t lane = w.lane + (uint32_t)(it * U) * w.stride;
        float xn[U], dyn[U];
        if (it + 1 < K) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                xn[u] = V::template load<CHECK>(sx, lane + (U + u) * w.stride);
                dyn[u] = V::template load<CHECK>(sdy, lane + (U + u) * w.stride);
                if constexpr (CHECK) asm volatile("" : "+v"(xn[u]), "+v"(dyn[u]));
            }
        }
        float dxf[U];
        bool sure = true;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const Pow<KP> X(xf[u]);
            const ElemBwd eb = backward_element<M, N, KP>(X, dyf[u], k, kw);
            accumulate<M, N>(eb.w, eb.sv, X, acc);
            dxf[u] = eb.dx;
            sure = sure && eb.sure;
        }
        if constexpr (N > 0) {
            // Rare: an element whose sign of Q the fp32 guard did not prove
            // (x == 0, a root of Q, or b = 0 in its group): fix this lane's rows.
            if (__builtin_expect(!sure, 0)) {
                if constexpr (N >= kExactSignMinN) {
                    uint32_t unsure, pos, neg;
                    const CoefHeld<M, N> src{k, kw};
                    exact_signs<M, N, U>(xf, src, unsure, pos, neg);
                    exact_apply<M, N, U>(xf, dyf, src, unsure, pos, neg, acc, dxf);
                } else {
#pragma unroll
                    for (int u = 0; u < U; ++u) dxf[u] = compensated_fix<M, N>(xf[u], dyf[u], k, kw, acc);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) V::template store<CHECK>(sdx, lane + u * w.stride, dxf[u]);
        if (it + 1 < K) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                xf[u] = xn[u];
                dyf[u] = dyn[u];
            }
        }
        // one batch ahead, no further: the scheduler would otherwise pull
        // later batches' loads up and hold them all in registers
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <class IO, int M, int N>
__global__ __launch_bounds__(kNarrowBwdThreads) void grkan_bwd_narrow_kernel(BwdArgs a) {
    using V = Elem<IO>;
    constexpr int U = narrow_bwd_unroll<M, N>();
    constexpr int K = kNarrowBwdIters;
    constexpr int RW = kNarrowBwdRowLanes;
    constexpr int NC = Deg<M, N>::kNumCoef;
    const Plan &P = a.plan;
    const NarrowPos p = narrow_pos(P, a.bundle0);
    if (p.tile >= P.tiles) return;
    int64_t ch;
    const Window w = narrow_window<RW, U, K>(P, p, ch);
    const Coefs<M, N> c = load_coefs<M, N>(a.A, a.B, narrow_group(P, ch));
    const BwdCoefs<M, N> k = derive<M, N>(c);
    const QWide<N> kw = widen<M, N, false>(c);
    const Span sx = make_span(at(a.x, w.base), w.avail);
    const Span sdy = make_span(at(a.dy, w.base), w.avail);
    const Span sdx = make_span(at(a.dx, w.base), w.avail);

    float acc[NC];
#pragma unroll
    for (int i = 0; i < NC; ++i) acc[i] = 0.0f;
    if (w.full) narrow_bwd_rows<IO, M, N, U, K, false>(sx, sdy, sdx, w, k, kw, acc);
    else narrow_bwd_rows<IO, M, N, U, K, true>(sx, sdy, sdx, w, k, kw, acc);

    // Workgroup sums in a fixed order: per channel over the row lanes, then
    // per group over its channels in this column block, in fp64.
    __shared__ float red[NC * RW * kNarrowCols];
    __shared__ double ct[NC * kNarrowCols];
    const int x = (int)threadIdx.x, y = (int)threadIdx.y;
    const int t = y * kNarrowCols + x;
#pragma unroll
    for (int i = 0; i < NC; ++i) red[(i * RW + y) * kNarrowCols + x] = acc[i];
    __syncthreads();
    for (int idx = t; idx < NC * kNarrowCols; idx += kNarrowBwdThreads) {
        const int i = idx / kNarrowCols, xx = idx % kNarrowCols;
        double s = 0.0;
#pragma unroll
        for (int yy = 0; yy < RW; ++yy) s += (double)red[(i * RW + yy) * kNarrowCols + xx];
        ct[idx] = s;
    }
    __syncthreads();
    const int64_t c0 = (int64_t)p.cb * kNarrowCols;
    const int64_t c1 = (c0 + kNarrowCols < P.d) ? c0 + kNarrowCols : P.d;
    const int64_t g_lo = c0 / P.d_g, g_hi = (c1 - 1) / P.d_g;
    const int nlg = (int)(g_hi - g_lo + 1);
    for (int idx = t; idx < nlg * NC; idx += kNarrowBwdThreads) {
        const int64_t gg = g_lo + idx / NC;
        const int i = idx % NC;
        const int64_t lo = (gg * P.d_g > c0 ? gg * P.d_g : c0) - c0;
        const int64_t hi = ((gg + 1) * P.d_g < c1 ? (gg + 1) * P.d_g : c1) - c0;
        double s = 0.0;
        for (int64_t c = lo; c < hi; ++c) s += ct[i * kNarrowCols + c];
        float *dst = (i <= M) ? (a.dA + gg * (M + 1) + i) : (a.dB + gg * N + (i - M - 1));
        if (a.mode != kModeAtomic) {
            const int64_t part = (int64_t)p.cb - gg * P.d_g / P.cpb;
            const int64_t slot = part * 8 * P.bundles + slot_in_part(P, p.tile);
            float *pp = a.partials + (gg * NC + i) * plan_slots(P) + slot;
            *(a.mode == kModeDirect ? dst : pp) = (float)s;
        } else {
            unsafeAtomicAdd(dst, (float)s);
        }
    }
}

template <class IO, int M, int N>
hipError_t fwd_impl(const FwdArgs &a, int repeat, dim3 grid, hipStream_t s) {
    if (a.plan.kind == kNarrow) {
        if (repeat != 1) return hipErrorInvalidValue;
        hipLaunchKernelGGL((grkan_fwd_narrow_kernel<IO, M, N>), grid,
                           dim3(kNarrowCols, kNarrowRowLanes), 0, s, a);
        return hipGetLastError();
    }
    const dim3 block((unsigned)a.plan.part_vecs, (unsigned)a.plan.rows_per_iter);
    constexpr int U = fwd_unroll<IO, M, N>();
    constexpr int US = fwd_unroll_small<IO, M, N>();
    if (a.plan.unroll == US && US != U) {
        if (repeat != 1) {
            if constexpr (M == 5 && N == 4) {
                switch (repeat) {
                case 2: hipLaunchKernelGGL((grkan_fwd_kernel<IO, M, N, US, 2>), grid, block, 0, s, a); break;
                case 4: hipLaunchKernelGGL((grkan_fwd_kernel<IO, M, N, US, 4>), grid, block, 0, s, a); break;
                case 8: hipLaunchKernelGGL((grkan_fwd_kernel<IO, M, N, US, 8>), grid, block, 0, s, a); break;
                default: return hipErrorInvalidValue;
                }
                return hipGetLastError();
            }
            return hipErrorInvalidValue;
        }
        hipLaunchKernelGGL((grkan_fwd_kernel<IO, M, N, US, 1>), grid, block, 0, s, a);
        return hipGetLastError();
    }
    if (a.plan.unroll != U) return hipErrorInvalidValue;
    if (repeat != 1) {
        if constexpr (M == 5 && N == 4) {
            switch (repeat) {
            case 2: hipLaunchKernelGGL((grkan_fwd_kernel<IO, M, N, U, 2>), grid, block, 0, s, a); break;
            case 4: hipLaunchKernelGGL((grkan_fwd_kernel<IO, M, N, U, 4>), grid, block, 0, s, a); break;
            case 8: hipLaunchKernelGGL((grkan_fwd_kernel<IO, M, N, U, 8>), grid, block, 0, s, a); break;
            default: return hipErrorInvalidValue;
            }
            return hipGetLastError();
        }
        return hipErrorInvalidValue;
    }
    hipLaunchKernelGGL((grkan_fwd_kernel<IO, M, N, U, 1>), grid, block, 0, s, a);
    return hipGetLastError();
}

template <int M, int N>
size_t bwd_lds_bytes(int block) {
    const int nw = (block + 63) / 64;
    return (size_t)Deg<M, N>::kNumCoef * (nw * 64 + 16) * sizeof(float);
}

template <class IO, int M, int N>
hipError_t bwd_impl(const BwdArgs &a, int repeat, dim3 grid, hipStream_t s) {
    if (a.y && repeat != 1) return hipErrorInvalidValue;
    if (a.plan.kind == kNarrow) {
        if (repeat != 1 || a.y) return hipErrorInvalidValue;
        hipLaunchKernelGGL((grkan_bwd_narrow_kernel<IO, M, N>), grid,
                           dim3(kNarrowCols, kNarrowBwdRowLanes), 0, s, a);
        return hipGetLastError();
    }
    const dim3 block((unsigned)a.plan.part_vecs, (unsigned)a.plan.rows_per_iter);
    const size_t lds = bwd_lds_bytes<M, N>(a.plan.block);
    constexpr int U = bwd_unroll<IO, M, N>();
    constexpr int US = bwd_unroll_small<IO, M, N>();
    if (a.plan.unroll == US && US != U) {
        if (repeat != 1) {
            if constexpr (M == 5 && N == 4) {
                if (a.y) return hipErrorInvalidValue;
                switch (repeat) {
                case 2: hipLaunchKernelGGL((grkan_bwd_kernel<IO, M, N, US, 2>), grid, block, lds, s, a); break;
                case 4: hipLaunchKernelGGL((grkan_bwd_kernel<IO, M, N, US, 4>), grid, block, lds, s, a); break;
                case 8: hipLaunchKernelGGL((grkan_bwd_kernel<IO, M, N, US, 8>), grid, block, lds, s, a); break;
                default: return hipErrorInvalidValue;
                }
                return hipGetLastError();
            }
            return hipErrorInvalidValue;
        }
        if (a.y) {
            if constexpr (std::is_same<IO, bf16io>::value && M == 5 && N == 4) {
                hipLaunchKernelGGL((grkan_bwd_kernel<IO, M, N, US, 1, true>), grid, block, lds, s, a);
                return hipGetLastError();
            }
            return hipErrorInvalidValue;
        }
        hipLaunchKernelGGL((grkan_bwd_kernel<IO, M, N, US, 1>), grid, block, lds, s, a);
        return hipGetLastError();
    }
    if (a.plan.unroll != U) return hipErrorInvalidValue;
    if (repeat != 1) {
        if constexpr (M == 5 && N == 4) {
            switch (repeat) {
            case 2: hipLaunchKernelGGL((grkan_bwd_kernel<IO, M, N, U, 2>), grid, block, lds, s, a); break;
            case 4: hipLaunchKernelGGL((grkan_bwd_kernel<IO, M, N, U, 4>), grid, block, lds, s, a); break;
            case 8: hipLaunchKernelGGL((grkan_bwd_kernel<IO, M, N, U, 8>), grid, block, lds, s, a); break;
            default: return hipErrorInvalidValue;
            }
            return hipGetLastError();
        }
        return hipErrorInvalidValue;
    }
    // F(x) as a second output (the GR-KAN bf16 layer backward) takes the
    // small pass count at every size (plan_shape's with_f)
    if (a.y) return hipErrorInvalidValue;
    hipLaunchKernelGGL((grkan_bwd_kernel<IO, M, N, U, 1>), grid, block, lds, s, a);
    return hipGetLastError();
}

}  // namespace

template <int M, int N>
int Kernels<M, N>::unroll(grkan_dtype_t io, int pass, bool small) {
    if (io == GRKAN_BF16) {
        if (small) return pass ? bwd_unroll_small<bf16io, M, N>() : fwd_unroll_small<bf16io, M, N>();
        return pass ? bwd_unroll<bf16io, M, N>() : fwd_unroll<bf16io, M, N>();
    }
    if (small) return pass ? bwd_unroll_small<float, M, N>() : fwd_unroll_small<float, M, N>();
    return pass ? bwd_unroll<float, M, N>() : fwd_unroll<float, M, N>();
}

template <int M, int N>
void Kernels<M, N>::narrow_shape(grkan_dtype_t, int pass, int *row_lanes, int *unroll, int *iters) {
    *row_lanes = pass ? kNarrowBwdRowLanes : kNarrowRowLanes;
    *unroll = pass ? narrow_bwd_unroll<M, N>() : narrow_unroll<M, N>();
    *iters = pass ? kNarrowBwdIters : 1;
}

template <int M, int N>
int Kernels<M, N>::target_block(grkan_dtype_t io, int pass, bool atomic_mode) {
    if (pass == 1 && atomic_mode) return kAtomicModeBlock;
    if (pass == 0) return kFwdBlock;
    const bool wide = io == GRKAN_BF16 ? bwd_wide_block<bf16io, M, N>() : bwd_wide_block<float, M, N>();
    return wide ? kBwdWideBlock : kBwdBlock;
}

template <int M, int N>
hipError_t Kernels<M, N>::forward(grkan_dtype_t io, const FwdArgs &a, int repeat, dim3 grid, hipStream_t s) {
    return io == GRKAN_BF16 ? fwd_impl<bf16io, M, N>(a, repeat, grid, s) : fwd_impl<float, M, N>(a, repeat, grid, s);
}

template <int M, int N>
hipError_t Kernels<M, N>::backward(grkan_dtype_t io, const BwdArgs &a, int repeat, dim3 grid, hipStream_t s) {
    return io == GRKAN_BF16 ? bwd_impl<bf16io, M, N>(a, repeat, grid, s) : bwd_impl<float, M, N>(a, repeat, grid, s);
}

template <int M, int N>
hipError_t Kernels<M, N>::occupancy(grkan_dtype_t io, int pass, int block, int *blocks_per_cu, bool narrow) {
    if (narrow) {
        const void *fn;
        if (io == GRKAN_BF16)
            fn = pass ? (const void *)grkan_bwd_narrow_kernel<bf16io, M, N>
                      : (const void *)grkan_fwd_narrow_kernel<bf16io, M, N>;
        else
            fn = pass ? (const void *)grkan_bwd_narrow_kernel<float, M, N>
                      : (const void *)grkan_fwd_narrow_kernel<float, M, N>;
        return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, fn,
                                                            pass ? kNarrowBwdThreads : kNarrowThreads, 0);
    }
    const void *fn;
    const size_t lds = pass ? bwd_lds_bytes<M, N>(block) : 0;
    if (io == GRKAN_BF16)
        fn = pass ? (const void *)grkan_bwd_kernel<bf16io, M, N, bwd_unroll<bf16io, M, N>(), 1>
                  : (const void *)grkan_fwd_kernel<bf16io, M, N, fwd_unroll<bf16io, M, N>(), 1>;
    else
        fn = pass ? (const void *)grkan_bwd_kernel<float, M, N, bwd_unroll<float, M, N>(), 1>
                  : (const void *)grkan_fwd_kernel<float, M, N, fwd_unroll<float, M, N>(), 1>;
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, fn, block, lds);
}

template struct Kernels<GRKAN_M, GRKAN_N>;

}  // namespace grkan
