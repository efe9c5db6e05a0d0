// grkan_layer.hip -- the GR-KAN layer's linear map on MFMA (gfx950): the
// forward z = F(x) W^T with the group-rational activation F applied while the
// A operand is staged (F fused into the GEMM prologue), and the plain GEMM
// z = y W^T it replaces when F is applied by its own kernel.
//
// Pages cited
//   [FlashKAT notes]  "FlashKAT: Understanding and Addressing Performance
//                     Bottlenecks in the Kolmogorov-Arnold Transformer",
//                     Paper-Notes page (AAAI 2026), arXiv 2505.13813.
//
// A GR-KAN layer applies the group-rational F to its d_in inputs and maps the
// result linearly to d_out outputs: (2m + 2n + 3) d_in FLOPs of rational
// against 2 d_in d_out of linear map per row ([FlashKAT notes], section
// "1. 性能瓶颈诊断", Insight 2).  The pages print no bias; none is applied.
// Precision: x, W and z are bf16, F is evaluated in fp32 exactly as the
// activation kernels do and rounded to nearest-even bf16 as the MFMA operand,
// products accumulate in fp32, z is rounded to nearest-even bf16.
//
// Kernel shape (both variants).  C[M][N] = A[M][K] B[N][K]^T with both
// operands K-contiguous (x row-major [rows][d_in], W row-major
// [d_out][d_in]).  Workgroup tile 256 x 256, 8 waves as 4 x 2, wave tile
// 64 x 128 = 2 x 4 blocks of v_mfma_f32_32x32x16_bf16 (128 fp32 accumulators
// per lane, 2 waves per SIMD).  K advances 64 at a time through two LDS
// stages of [256 + 256][64 + 8] bf16 (rows padded by 16 bytes so that a
// fragment read by 8 consecutive rows touches 8 distinct bank groups; 144 KB
// in all).  The tiles of step k + 1 arrive in registers during step k - 1
// (their loads are issued at the end of the previous step, so a whole step
// of MFMAs covers their latency) and are written to the other stage one
// 16-byte chunk per thread after each of step k's four MFMA sub-steps; each
// lane's MFMA fragments (8 consecutive k of one row) are read one sub-step
// ahead.  Fused variant: the activation runs on each staged x chunk between
// the registers and the LDS write -- a thread's chunks lie in one channel
// group (d_in / n_groups a multiple of 8), whose coefficients come from an
// LDS table -- interleaved with the MFMAs.
// Workgroup order: XCD (b mod 8) takes whole 256-row panels, N tiles of a
// panel back to back, so a panel of x is fetched into one XCD's L2 once.
// Output: with 16-byte aligned rows of z, each wave stages its bf16 tile in
// the idle LDS and writes 16-byte row chunks; otherwise one bf16 per store.
//
// Measured on MI355X (KAT-B MLP shapes, 201,728 rows, 951.9 GFLOP per
// call): the plain GEMM runs at 900-1,040 TFLOP/s; the fused prologue costs
// 0.45 ms (d_out = 3072) and 0.48 ms (d_out = 768) more than the plain GEMM,
// because evaluating F costs ~15 VALU instructions per element and every
// 256-wide N tile evaluates it again: at this tile width the activation's
// vector work is as large as the tile's matrix work (a CU issues ~4,000 bf16
// MFMA FLOPs but only 64 vector lanes per cycle), and the two overlap only in
// part.  Wider N tiles need more accumulator registers than a SIMD holds at
// 256 rows.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "grkan_device.h"
#include "grkan_launch.h"

namespace grkan {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 256, kBN = 256, kBK = 64;
constexpr int kWavesM = 4, kWavesN = 2;
constexpr int kThreads = kWavesM * kWavesN * 64;
constexpr int kLdk = kBK + 8;                         // padded LDS row, bf16 elements
constexpr int kWTM = kBM / kWavesM, kWTN = kBN / kWavesN;
constexpr int kTM = kWTM / 32, kTN = kWTN / 32;       // MFMA blocks per wave
constexpr int kChunksPerRow = kBK / 8;                // 16-byte chunks per tile row
constexpr int kCA = kBM * kChunksPerRow / kThreads;   // A chunks per thread per step
constexpr int kCB = kBN * kChunksPerRow / kThreads;
constexpr int kStage = (kBM + kBN) * kLdk;            // bf16 elements per LDS stage
constexpr size_t kLdsBytes = 2 * (size_t)kStage * 2;
constexpr int kKSteps = kBK / 16;
constexpr int kInterleave = 14;                       // VALU instructions scheduled per MFMA (fused)
static_assert(kBM * kChunksPerRow % kThreads == 0 && kBN * kChunksPerRow % kThreads == 0, "chunks");
static_assert(kCA == kKSteps && kCB == kKSteps, "one chunk of each tile is staged per K sub-step");
static_assert(kThreads % kChunksPerRow == 0, "a thread's chunks share one column");
static_assert((kThreads / 64) * (kWTM / 2) * kWTN * 4 <= (int)kLdsBytes && kWTN == 128 && kWTM % 32 == 0,
              "the bf16 output staging fits in the operand stages");

// What the A operand is made of.
enum Prologue : int {
    kPlain = 0,     // A = x itself (bf16 [M][K])
    kRational = 1,  // A = bf16(F(x)), F the group-rational activation (x bf16 [M][K])
    kChebyshev = 2, // A = bf16(T_k(tanh(x_i))) at K position 8 i + k, k = 0..7 (x bf16 [M][K / 8])
    kChebyDx = 3    // A = x itself; the bf16 result G is not stored but turned into the
                    // Chebyshev layer's dx (cheby_dx8) in the epilogue
};

struct LayerArgs {
    const uint16_t *x;  // A's source (see Prologue)
    const uint16_t *w;  // [N][K] bf16
    uint16_t *z;        // [M][N] bf16
    const float *A;     // [n_groups][6] (kRational)
    const float *B;     // [n_groups][4]
    int32_t M, N, K, d_g, n_groups;
    const uint16_t *xc; // kChebyDx: the layer input x, bf16 [M][N / 8]
    uint16_t *dxc;      // kChebyDx: dx, bf16 [M][N / 8]
};

// The coefficient table: group g at [g * 12]: a_0..a_5, b_1..b_4.
constexpr int kMaxLayerGroups = 64;

__device__ static inline u32x4 activate8(u32x4 v, const Coefs<5, 4> &c) {
    float f[8];
    Io<bf16io>::unpack(v, f);
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = rational<5, 4>(f[e], c);
    return Io<bf16io>::pack(f);
}

// tanh in fp32, absolute error below 2^-21: for |x| < 0.55 its odd Taylor
// series through x^15 (the next term is below 3e-8 there); above, 1 - 2 /
// (e^(2|x|) + 1) with the sign of x, from the hardware base-2 exponential
// and reciprocal (no cancellation: the fraction is below 0.55).
__device__ static inline float tanh_f32(float x) {
    const float ax = fabsf(x), x2 = x * x;
    float p = -929569.0f / 638512875.0f;
    p = fmaf(p, x2, 21844.0f / 6081075.0f);
    p = fmaf(p, x2, -1382.0f / 155925.0f);
    p = fmaf(p, x2, 62.0f / 2835.0f);
    p = fmaf(p, x2, -17.0f / 315.0f);
    p = fmaf(p, x2, 2.0f / 15.0f);
    p = fmaf(p, x2, -1.0f / 3.0f);
    const float series = fmaf(p * x2, x, x);
    const float e = __builtin_amdgcn_exp2f(ax * 2.8853900817779268f);  // e^(2|x|)
    const float q = 1.0f - 2.0f * __builtin_amdgcn_rcpf(e + 1.0f);
    return ax < 0.55f ? series : __builtin_copysignf(q, x);
}

// The Chebyshev basis T_0..T_7 of t = tanh(x) as 8 bf16 (the order of the K
// positions 8 i .. 8 i + 7), by the three-term recurrence.
__device__ static inline u32x4 chebyshev8(uint32_t xbits) {
    const float t = tanh_f32(__uint_as_float(xbits << 16)), t2 = t + t;
    float T[8];
    T[0] = 1.0f;
    T[1] = t;
#pragma unroll
    for (int k = 1; k < 7; ++k) T[k + 1] = fmaf(t2, T[k], -T[k - 1]);
    return Io<bf16io>::pack(T);
}

// The Chebyshev layer's dx of one input from its 8 values g_k = (dy C)[8 i + k]
// (bf16) and x (bf16): dx = (1 - t^2) sum_k k U_{k-1}(t) g_k, t = tanh(x), with
// U the second-kind polynomials by their recurrence; rounded to bf16.
__device__ static inline uint16_t cheby_dx8(u32x4 gbits, uint32_t xbits) {
    float g[8];
    Io<bf16io>::unpack(gbits, g);
    const float t = tanh_f32(__uint_as_float(xbits << 16)), t2 = t + t;
    float um = 1.0f, u = t2;                   // U_0, U_1
    float sum = g[1];                          // T_1' = 1 U_0
    sum = fmaf(2.0f * u, g[2], sum);           // T_2' = 2 U_1
#pragma unroll
    for (int k = 3; k <= 7; ++k) {
        const float un = fmaf(t2, u, -um);     // U_{k-1}
        um = u;
        u = un;
        sum = fmaf((float)k * u, g[k], sum);
    }
    const __bf16 h = (__bf16)(fmaf(-t, t, 1.0f) * sum);
    return __builtin_bit_cast(uint16_t, h);
}

template <int PRO>
__global__ __launch_bounds__(kThreads) void grkan_layer_gemm_kernel(LayerArgs a) {
    constexpr bool FUSED = PRO == kRational;
    constexpr bool CHEBY_DX = PRO == kChebyDx;
    extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
    __shared__ float coef[kMaxLayerGroups * 12];
    const int t = (int)threadIdx.x, lane = t & 63, wv = t >> 6;
    const int wm = wv / kWavesN, wn = wv % kWavesN;
    const int nb_count = (a.N + kBN - 1) / kBN;
    const int b = (int)blockIdx.x, xcd = b & 7, idx = b >> 3;
    const int m0 = ((idx / nb_count) * 8 + xcd) * kBM, n0 = (idx % nb_count) * kBN;
    if (m0 >= a.M) return;
    if (FUSED) {
        for (int i = t; i < a.n_groups * 12; i += kThreads) {
            const int g = i / 12, k = i % 12;
            coef[i] = k < 6 ? a.A[g * 6 + k] : (k < 10 ? a.B[g * 4 + k - 6] : 0.0f);
        }
    }

    // Source rows of this thread's chunks.  Rows past the end are clamped to
    // the last row: they only feed outputs that are never stored.  A
    // Chebyshev chunk is the basis of one x value: x index 8 k-step + cc.
    const int cc = t % kChunksPerRow;
    const uint16_t *pa[kCA];
    const uint16_t *pb[kCB];
#pragma unroll
    for (int j = 0; j < kCA; ++j) {
        const int r = (t + kThreads * j) / kChunksPerRow;
        if constexpr (PRO == kChebyshev)
            pa[j] = a.x + (size_t)min(m0 + r, a.M - 1) * (a.K / 8) + cc;
        else
            pa[j] = a.x + (size_t)min(m0 + r, a.M - 1) * a.K + cc * 8;
    }
#pragma unroll
    for (int j = 0; j < kCB; ++j) {
        const int r = (t + kThreads * j) / kChunksPerRow;
        pb[j] = a.w + (size_t)min(n0 + r, a.N - 1) * a.K + cc * 8;
    }
    u32x4 ra[kCA], rb[kCB];
    uint32_t rx[kCA];
    auto load_tiles = [&](int kt) {
#pragma unroll
        for (int j = 0; j < kCA; ++j) {
            if constexpr (PRO == kChebyshev)
                rx[j] = pa[j][kt * (kBK / 8)];
            else
                ra[j] = *reinterpret_cast<const u32x4 *>(pa[j] + kt * kBK);
        }
#pragma unroll
        for (int j = 0; j < kCB; ++j) rb[j] = *reinterpret_cast<const u32x4 *>(pb[j] + kt * kBK);
    };
    Coefs<5, 4> c;
    auto load_coefs_of = [&](int kt) {
        const int g = (kt * kBK + cc * 8) / a.d_g;
#pragma unroll
        for (int i = 0; i < 6; ++i) c.a[i] = coef[g * 12 + i];
#pragma unroll
        for (int i = 0; i < 4; ++i) c.b[i] = coef[g * 12 + 6 + i];
    };
    // Chunk j of this thread's share of both tiles -> LDS stage buf.
    auto stage_chunk = [&](int buf, int j) {
        if constexpr (FUSED) ra[j] = activate8(ra[j], c);
        if constexpr (PRO == kChebyshev) ra[j] = chebyshev8(rx[j]);
        uint16_t *s = lds + buf * kStage;
        const int r = (t + kThreads * j) / kChunksPerRow;
        *reinterpret_cast<u32x4 *>(s + r * kLdk + cc * 8) = ra[j];
        *reinterpret_cast<u32x4 *>(s + (kBM + r) * kLdk + cc * 8) = rb[j];
    };

    f32x16 acc[kTM][kTN];
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN; ++j) acc[i][j] = f32x16{};
    bf16x8 fa[2][kTM], fb[2][kTN];
    auto load_fragments = [&](int buf, int ks, int set) {
        const uint16_t *s = lds + buf * kStage;
        const int ko = ks * 16 + 8 * (lane >> 5);
#pragma unroll
        for (int i = 0; i < kTM; ++i)
            fa[set][i] = *reinterpret_cast<const bf16x8 *>(s + (wm * kWTM + i * 32 + (lane & 31)) * kLdk + ko);
#pragma unroll
        for (int j = 0; j < kTN; ++j)
            fb[set][j] = *reinterpret_cast<const bf16x8 *>(s + (kBM + wn * kWTN + j * 32 + (lane & 31)) * kLdk + ko);
    };

    const int nk = a.K / kBK;
    load_tiles(0);
    __syncthreads();  // coefficient table
    if (FUSED) load_coefs_of(0);
#pragma unroll
    for (int j = 0; j < kKSteps; ++j) stage_chunk(0, j);
    if (nk > 1) load_tiles(1);
    __syncthreads();
    load_fragments(0, 0, 0);
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < nk;
        if (FUSED && more) load_coefs_of(kt + 1);
#pragma unroll
        for (int ks = 0; ks < kKSteps; ++ks) {
            const int set = ks & 1;
            if (ks + 1 < kKSteps) load_fragments(cur, ks + 1, set ^ 1);
#pragma unroll
            for (int i = 0; i < kTM; ++i)
#pragma unroll
                for (int j = 0; j < kTN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[set][i], fb[set][j], acc[i][j], 0, 0, 0);
            if (more) stage_chunk(cur ^ 1, ks);
            if (FUSED) {
#pragma unroll
                for (int q = 0; q < kTM * kTN; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);            // one MFMA
                    __builtin_amdgcn_sched_group_barrier(0x002, kInterleave, 0);  // then VALU
                }
            }
        }
        if (kt + 2 < nk) load_tiles(kt + 2);
        __syncthreads();
        if (more) load_fragments(cur ^ 1, 0, 0);
    }

    // bf16 results.  When rows of z are 16-byte aligned (N a multiple of 8),
    // each wave stages its 64 x 128 tile in 16 KB of the (now idle) LDS and
    // writes it back as 16-byte row chunks: an accumulator lane holds one
    // column of 4-row runs, so pairs of rows are packed into one dword
    // ([row pair][column], columns of row pairs 2, 3 mod 4 offset by 32 so
    // the two lane halves of a write use different banks), then each lane
    // reads 8 columns of a row pair and splits them into the two rows.
    if (CHEBY_DX || ((a.N & 7) == 0 && (reinterpret_cast<uintptr_t>(a.z) & 15) == 0)) {
        __syncthreads();  // every wave is done with the operand stages
        uint32_t *rd = reinterpret_cast<uint32_t *>(lds) + wv * (kWTM / 2) * kWTN;
#pragma unroll
        for (int i = 0; i < kTM; ++i)
#pragma unroll
            for (int j = 0; j < kTN; ++j)
#pragma unroll
                for (int v = 0; v < 16; v += 2) {
                    const int p = i * 16 + 4 * (v >> 2) + 2 * (lane >> 5) + ((v & 3) >> 1);
                    const int col = j * 32 + (lane & 31);
                    const uint32_t lo = __builtin_bit_cast(uint16_t, (__bf16)acc[i][j][v]);
                    const uint32_t hi = __builtin_bit_cast(uint16_t, (__bf16)acc[i][j][v + 1]);
                    rd[p * kWTN + (col ^ (((p >> 1) & 1) << 5))] = lo | (hi << 16);
                }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        constexpr int kGroups = (kWTM / 2) * (kWTN / 8);  // (row pair, 8 columns) per wave
#pragma unroll
        for (int u = 0; u < kGroups / 64; ++u) {
            const int g = u * 64 + lane, p = g / (kWTN / 8), c8 = (g % (kWTN / 8)) * 8;
            const uint32_t *src = rd + p * kWTN + (c8 ^ (((p >> 1) & 1) << 5));
            const u32x4 d0 = *reinterpret_cast<const u32x4 *>(src);
            const u32x4 d1 = *reinterpret_cast<const u32x4 *>(src + 4);
            u32x4 r0, r1;  // rows 2 p and 2 p + 1: low and high halves of the dwords
            r0[0] = __builtin_amdgcn_perm(d0[1], d0[0], 0x05040100u);
            r0[1] = __builtin_amdgcn_perm(d0[3], d0[2], 0x05040100u);
            r0[2] = __builtin_amdgcn_perm(d1[1], d1[0], 0x05040100u);
            r0[3] = __builtin_amdgcn_perm(d1[3], d1[2], 0x05040100u);
            r1[0] = __builtin_amdgcn_perm(d0[1], d0[0], 0x07060302u);
            r1[1] = __builtin_amdgcn_perm(d0[3], d0[2], 0x07060302u);
            r1[2] = __builtin_amdgcn_perm(d1[1], d1[0], 0x07060302u);
            r1[3] = __builtin_amdgcn_perm(d1[3], d1[2], 0x07060302u);
            const int row = m0 + wm * kWTM + 2 * p, col = n0 + wn * kWTN + c8;
            if constexpr (CHEBY_DX) {
                // the 8 columns are the 8 basis values of input col / 8
                const int d_in = a.N >> 3;
                const size_t e = (size_t)row * d_in + (col >> 3);
                if (col < a.N) {
                    if (row < a.M) a.dxc[e] = cheby_dx8(r0, a.xc[e]);
                    if (row + 1 < a.M) a.dxc[e + d_in] = cheby_dx8(r1, a.xc[e + d_in]);
                }
            } else if (col < a.N) {
                if (row < a.M) *reinterpret_cast<u32x4 *>(a.z + (size_t)row * a.N + col) = r0;
                if (row + 1 < a.M) *reinterpret_cast<u32x4 *>(a.z + (size_t)(row + 1) * a.N + col) = r1;
            }
        }
        return;
    }
    // Otherwise one bf16 per store; full tiles skip the range checks.
    const bool full = m0 + kBM <= a.M && n0 + kBN <= a.N;
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN; ++j) {
            const int col = n0 + wn * kWTN + j * 32 + (lane & 31);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = m0 + wm * kWTM + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                if (full || (row < a.M && col < a.N)) {
                    const __bf16 h = (__bf16)acc[i][j][v];
                    a.z[(size_t)row * a.N + col] = __builtin_bit_cast(uint16_t, h);
                }
            }
        }
}

// ------------------------------------------------------------ backward
//
// Weight gradient dW = dZ^T Y: P[s][m][n] = sum over the rows r of split s of
// A[r][m] B[r][n] (A = dZ [rows][d_out], B = Y [rows][d_in], bf16), then a
// fixed-order sum over the splits.  Here K = rows runs down the columns of
// both operands, while an MFMA fragment wants 8 consecutive k of one m (or
// n).  Each thread loads one 16-byte chunk (8 consecutive m) from each of 4
// consecutive rows -- a wave reads 2 rows x 512 contiguous bytes per
// instruction -- and stages it in one of two ways:
//   transposed writes (dW): for each of its 8 m, the 4 rows as one 8-byte
//     LDS write.  LDS rows are [m][64 k] without padding, their eight
//     16-byte chunks permuted by chunk ^ ((m + m / 8) mod 8): fragment reads
//     (8 consecutive m, one chunk) and the transposed writes (m = 8 cc + i
//     for 32 chunk columns cc) both spread over the banks;
//   transposed reads (the Chebyshev dC, whose B chunks are built in
//     registers): the tiles are stored as they lie, [64 k][256 m] with rows
//     padded to 288 elements (rows k .. k + 3 start in four different
//     quarters of the bank space), and fragments are read with gfx950's
//     ds_read_b64_tr_b16 -- in each group of 16 lanes, lane i receives value
//     j = i mod 4 of lane 4 j + i / 4's 8-byte read, so lanes 4 j + q
//     pointing at row k0 + j, columns m0 + 4 q leave lane i with rows
//     k0 .. k0 + 3 of column m0 + i; two such reads give the 8 k of a
//     32 x 32 x 16 fragment.  Twice the LDS read instructions of the first
//     way, but no packing and half the write instructions: faster where the
//     basis already takes vector work, slower for the plain dW.
// The rows are cut
// into splits so that the few output tiles (36 at the KAT-B shapes) still
// fill the GPU in whole rounds of one workgroup per CU (14 splits, 504
// workgroups = 2 rounds at KAT-B); each workgroup writes its fp32 tile of partial sums, and
// grkan_wgrad_reduce_kernel adds the splits in order (bitwise reproducible).
constexpr int kWgSlots = 256;          // workgroups resident at once on MI355X (one per CU)
constexpr int64_t kWgMaxSplitRows = 16384;  // rows summed in fp32 by one workgroup at most
constexpr int kWgRow = kBK;            // transposed writes: bf16 per LDS row [m][64 k] (unpadded)
constexpr int kWgPitch = kBM + 32;     // transposed reads: bf16 per LDS row [k][m] (padded)
template <bool TR>
constexpr int kWgStage = TR ? 2 * kBK * kWgPitch : (kBM + kBN) * kWgRow;
template <bool TR>
constexpr size_t kWgLdsBytes = 2 * (size_t)kWgStage<TR> * 2;
static_assert(kBM == kBN, "A and B tiles share one layout");

struct WgradArgs {
    const uint16_t *a;   // [rows][M] bf16 (dZ)
    const uint16_t *b;   // [rows][N] bf16 (Y = F(x)); with CHEBY_B x [rows][N / 8], whose
                         // Chebyshev basis (chebyshev8) is the operand
    float *partials;     // [splits][M][N]
    int32_t rows, M, N, splits, rows_per_split;
};

__device__ static inline uint32_t pack2(uint32_t lo, uint32_t hi, int odd) {
    // the bf16 at position odd (0 = low half) of lo and of hi, as (lo's, hi's)
    return odd ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
}

// bf16 offset of 16-byte chunk `chunk` of LDS row m.
__device__ static inline int wg_chunk(int m, int chunk) {
    return m * kWgRow + ((chunk ^ ((m + (m >> 3)) & 7)) << 3);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Transposing read: 4 consecutive rows of one column per lane (see above).
__device__ static inline s16x4 read_tr(const uint16_t *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p));
}

template <bool CHEBY_B>
__global__ __launch_bounds__(kThreads) void grkan_wgrad_kernel(WgradArgs a) {
    constexpr bool TR = CHEBY_B;  // staging by transposed reads (else transposed writes)
    constexpr int kStg = kWgStage<TR>;
    extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
    const int t = (int)threadIdx.x, lane = t & 63, wv = t >> 6;
    const int wm = wv / kWavesN, wn = wv % kWavesN;
    const int mb_count = (a.M + kBM - 1) / kBM, nb_count = (a.N + kBN - 1) / kBN;
    const int tiles = mb_count * nb_count;
    const int b = (int)blockIdx.x;
    const int split = b / tiles, tile = b % tiles;
    const int m0 = (tile / nb_count) * kBM, n0 = (tile % nb_count) * kBN;
    const int r_begin = split * a.rows_per_split;
    const int r_end = min(a.rows, r_begin + a.rows_per_split);

    // This thread's chunks: 8 consecutive columns (cc), rows 4 rg .. 4 rg + 3
    // of each 64-row step.  Columns past the end are clamped (their outputs
    // are not stored); rows past the split's end read as zero.
    constexpr int kColChunks = kBM / 8;                 // 32
    static_assert(kThreads / kColChunks * 4 == kBK && kBM == kBN, "one 64-row step per thread set");
    const int cc = t % kColChunks, rg = t / kColChunks;
    const uint16_t *pa = a.a + min(m0 + cc * 8, a.M - 8);
    const int bld = CHEBY_B ? a.N / 8 : a.N;  // elements per row of b
    const uint16_t *pb = CHEBY_B ? a.b + min(n0 / 8 + cc, bld - 1) : a.b + min(n0 + cc * 8, a.N - 8);
    u32x4 ra[4], rb[4];
    uint32_t rx[4];
    bool rin[4];
    auto load_tiles = [&](int kt) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = r_begin + kt * kBK + rg * 4 + q;
            const bool in = r < r_end;
            const size_t rr = (size_t)(in ? r : r_begin);
            const u32x4 va = *reinterpret_cast<const u32x4 *>(pa + rr * a.M);
            ra[q] = in ? va : u32x4{0u, 0u, 0u, 0u};
            if constexpr (CHEBY_B) {
                rx[q] = pb[rr * bld];
                rin[q] = in;
            } else {
                const u32x4 vb = *reinterpret_cast<const u32x4 *>(pb + rr * a.N);
                rb[q] = in ? vb : u32x4{0u, 0u, 0u, 0u};
            }
        }
    };
    // Sub-step h's share of the staging.  Transposed reads: row 4 rg + h of
    // this thread's chunks, as it lies.  Transposed writes: columns 2h and
    // 2h + 1 of the chunks -> LDS rows cc*8 + 2h (+ 1), k = 4 rg .. 4 rg + 3.
    auto stage_part = [&](int buf, int h) {
        if constexpr (TR) {
            if constexpr (CHEBY_B) rb[h] = rin[h] ? chebyshev8(rx[h]) : u32x4{0u, 0u, 0u, 0u};
            uint16_t *s = lds + buf * kStg + (rg * 4 + h) * kWgPitch + cc * 8;
            *reinterpret_cast<u32x4 *>(s) = ra[h];
            *reinterpret_cast<u32x4 *>(s + kBK * kWgPitch) = rb[h];
            return;
        }
        if constexpr (CHEBY_B) {
            if (h == 0) {
#pragma unroll
                for (int q = 0; q < 4; ++q) rb[q] = rin[q] ? chebyshev8(rx[q]) : u32x4{0u, 0u, 0u, 0u};
            }
        }
        uint16_t *s = lds + buf * kStg;
        const int sub = (rg & 1) * 4;
#pragma unroll
        for (int odd = 0; odd < 2; ++odd) {
            const int col = cc * 8 + 2 * h + odd;
            uint2 va, vb;
            va.x = pack2(ra[0][h], ra[1][h], odd);
            va.y = pack2(ra[2][h], ra[3][h], odd);
            vb.x = pack2(rb[0][h], rb[1][h], odd);
            vb.y = pack2(rb[2][h], rb[3][h], odd);
            *reinterpret_cast<uint2 *>(s + wg_chunk(col, rg >> 1) + sub) = va;
            *reinterpret_cast<uint2 *>(s + wg_chunk(kBM + col, rg >> 1) + sub) = vb;
        }
    };

    f32x16 acc[kTM][kTN];
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN; ++j) acc[i][j] = f32x16{};
    bf16x8 fa[2][kTM], fb[2][kTN];
    // Transposed reads: lane l (group g = l / 16, i = l mod 16) points its two
    // reads at rows 16 ks + 8 (g / 2) + 4 r + i / 4, columns base + 16 (g mod
    // 2) + 4 (i mod 4).
    const int frow = 8 * (lane >> 5) + ((lane & 15) >> 2), fcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    auto load_fragments = [&](int buf, int ks, int set) {
        if constexpr (TR) {
            const uint16_t *s = lds + buf * kStg + (16 * ks + frow) * kWgPitch + fcol;
#pragma unroll
            for (int i = 0; i < kTM; ++i) {
                const uint16_t *p = s + wm * kWTM + i * 32;
                const s16x4 lo = read_tr(p), hi = read_tr(p + 4 * kWgPitch);
                fa[set][i] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            }
#pragma unroll
            for (int j = 0; j < kTN; ++j) {
                const uint16_t *p = s + kBK * kWgPitch + wn * kWTN + j * 32;
                const s16x4 lo = read_tr(p), hi = read_tr(p + 4 * kWgPitch);
                fb[set][j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            }
            return;
        }
        const uint16_t *s = lds + buf * kStg;
        const int chunk = 2 * ks + (lane >> 5);
#pragma unroll
        for (int i = 0; i < kTM; ++i)
            fa[set][i] = *reinterpret_cast<const bf16x8 *>(s + wg_chunk(wm * kWTM + i * 32 + (lane & 31), chunk));
#pragma unroll
        for (int j = 0; j < kTN; ++j)
            fb[set][j] = *reinterpret_cast<const bf16x8 *>(s + wg_chunk(kBM + wn * kWTN + j * 32 + (lane & 31), chunk));
    };

    const int nk = (r_end - r_begin + kBK - 1) / kBK;
    if (nk > 0) {
        load_tiles(0);
#pragma unroll
        for (int h = 0; h < 4; ++h) stage_part(0, h);
        if (nk > 1) load_tiles(1);
        __syncthreads();
        load_fragments(0, 0, 0);
    }
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < nk;
#pragma unroll
        for (int ks = 0; ks < kKSteps; ++ks) {
            const int set = ks & 1;
            if (ks + 1 < kKSteps) load_fragments(cur, ks + 1, set ^ 1);
#pragma unroll
            for (int i = 0; i < kTM; ++i)
#pragma unroll
                for (int j = 0; j < kTN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[set][i], fb[set][j], acc[i][j], 0, 0, 0);
            if (more) stage_part(cur ^ 1, ks);
        }
        if (kt + 2 < nk) load_tiles(kt + 2);
        __syncthreads();
        if (more) load_fragments(cur ^ 1, 0, 0);
    }

    float *out = a.partials + (size_t)split * a.M * a.N;
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN; ++j) {
            const int col = n0 + wn * kWTN + j * 32 + (lane & 31);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = m0 + wm * kWTM + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                if (row < a.M && col < a.N) out[(size_t)row * a.N + col] = acc[i][j][v];
            }
        }
}

// dW[i] = sum over s of partials[s][i], in split order, in fp64.
__global__ __launch_bounds__(256) void grkan_wgrad_reduce_kernel(const float *__restrict__ partials,
                                                                 float *__restrict__ dW, int64_t n, int splits) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    double s = 0.0;
    for (int k = 0; k < splits; ++k) s += (double)partials[(size_t)k * n + i];
    dW[i] = (float)s;
}

// out[c][r] = in[r][c] for a [R][C] bf16 matrix, 32 x 32 tiles through LDS.
__global__ __launch_bounds__(256) void grkan_transpose16_kernel(const uint16_t *__restrict__ in,
                                                                uint16_t *__restrict__ out, int R, int C) {
    __shared__ uint16_t tile[32][33];
    const int c0 = blockIdx.x * 32, r0 = blockIdx.y * 32;
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
    for (int k = ty; k < 32; k += 8) {
        const int r = r0 + k, c = c0 + tx;
        if (r < R && c < C) tile[k][tx] = in[(size_t)r * C + c];
    }
    __syncthreads();
    for (int k = ty; k < 32; k += 8) {
        const int c = c0 + k, r = r0 + tx;
        if (r < R && c < C) out[(size_t)c * R + r] = tile[tx][k];
    }
}


std::once_flag g_attr_once[4];
hipError_t g_attr_err[4];

template <int PRO>
hipError_t launch(const LayerArgs &a, hipStream_t s) {
    auto kern = grkan_layer_gemm_kernel<PRO>;
    std::call_once(g_attr_once[PRO], [&] {
        g_attr_err[PRO] = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytes);
    });
    if (g_attr_err[PRO] != hipSuccess) return g_attr_err[PRO];
    const int64_t mb = (a.M + kBM - 1) / kBM, nb = (a.N + kBN - 1) / kBN;
    const int64_t grid = (mb + 7) / 8 * 8 * nb;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreads), kLdsBytes, s, a);
    return hipGetLastError();
}

}  // namespace

int layer_max_groups() { return kMaxLayerGroups; }
int layer_k_step() { return kBK; }

hipError_t launch_layer_forward(const void *x, const float *A, const float *B, const void *W, void *z,
                                int64_t rows, int64_t d_in, int64_t d_out, int32_t n_groups, hipStream_t s) {
    LayerArgs a{static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(W), static_cast<uint16_t *>(z),
                A, B, (int32_t)rows, (int32_t)d_out, (int32_t)d_in, (int32_t)(d_in / n_groups), n_groups};
    return launch<kRational>(a, s);
}

int wgrad_splits(int64_t rows, int64_t M, int64_t N) {
    // A workgroup holds one CU (its LDS), so workgroups run in rounds of
    // kWgSlots.  Take the fewest splits of at most kWgMaxSplitRows rows each
    // whose rounds are at least 95% full (else the fullest within 64 more);
    // a fixed rule, so the summation order does not depend on the device.
    const int64_t tiles = ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
    const int64_t steps = (rows + kBK - 1) / kBK;
    int64_t lo = (rows + kWgMaxSplitRows - 1) / kWgMaxSplitRows;
    if (lo < 1) lo = 1;
    if (lo >= steps) return (int)(steps < 1 ? 1 : steps);
    int64_t best = lo;
    double best_fill = 0.0;
    for (int64_t sp = lo; sp <= steps && sp < lo + 64; ++sp) {
        const int64_t wgs = tiles * sp, rounds = (wgs + kWgSlots - 1) / kWgSlots;
        const double fill = (double)wgs / (double)(rounds * kWgSlots);
        if (fill >= 0.95) return (int)sp;
        if (fill > best_fill) best_fill = fill, best = sp;
    }
    return (int)best;
}

size_t wgrad_partials_bytes(int64_t rows, int64_t M, int64_t N) {
    return (size_t)wgrad_splits(rows, M, N) * (size_t)M * (size_t)N * sizeof(float);
}

template <bool CHEBY_B>
hipError_t launch_wgrad_impl(const void *dz, const void *y, float *partials, float *dW, int64_t rows, int64_t M,
                             int64_t N, hipStream_t s) {
    auto kern = grkan_wgrad_kernel<CHEBY_B>;
    static std::once_flag once;
    static hipError_t err;
    std::call_once(once, [&] {
        err = hipFuncSetAttribute(reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (int)kWgLdsBytes<CHEBY_B>);
    });
    if (err != hipSuccess) return err;
    const int splits = wgrad_splits(rows, M, N);
    const int64_t steps = (rows + kBK - 1) / kBK;
    const int rps = (int)((steps + splits - 1) / splits) * kBK;
    WgradArgs a{static_cast<const uint16_t *>(dz), static_cast<const uint16_t *>(y), partials, (int32_t)rows,
                (int32_t)M, (int32_t)N, splits, rps};
    const int64_t tiles = ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
    hipLaunchKernelGGL(kern, dim3((unsigned)(tiles * splits)), dim3(kThreads), kWgLdsBytes<CHEBY_B>, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n = M * N;
    hipLaunchKernelGGL(grkan_wgrad_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, partials, dW,
                       n, splits);
    return hipGetLastError();
}

hipError_t launch_wgrad(const void *dz, const void *y, float *partials, float *dW, int64_t rows, int64_t M,
                        int64_t N, hipStream_t s) {
    return launch_wgrad_impl<false>(dz, y, partials, dW, rows, M, N, s);
}

hipError_t launch_cheby_wgrad(const void *dy, const void *x, float *partials, float *dC, int64_t rows,
                              int64_t d_out, int64_t d_in, hipStream_t s) {
    return launch_wgrad_impl<true>(dy, x, partials, dC, rows, d_out, d_in * 8, s);
}

hipError_t launch_cheby_g_dx(const void *dy, const void *Ct, const void *x, void *dx, int64_t rows,
                             int64_t d_out, int64_t d_in, hipStream_t s) {
    LayerArgs a{static_cast<const uint16_t *>(dy), static_cast<const uint16_t *>(Ct), nullptr, nullptr, nullptr,
                (int32_t)rows, (int32_t)(d_in * 8), (int32_t)d_out, 1, 1, static_cast<const uint16_t *>(x),
                static_cast<uint16_t *>(dx)};
    return launch<kChebyDx>(a, s);
}

hipError_t launch_transpose16(const void *in, void *out, int64_t R, int64_t C, hipStream_t s) {
    hipLaunchKernelGGL(grkan_transpose16_kernel, dim3((unsigned)((C + 31) / 32), (unsigned)((R + 31) / 32)),
                       dim3(256), 0, s, static_cast<const uint16_t *>(in), static_cast<uint16_t *>(out), (int)R,
                       (int)C);
    return hipGetLastError();
}

hipError_t launch_cheby_forward(const void *x, const void *C, void *y, int64_t rows, int64_t d_in, int64_t d_out,
                                hipStream_t s) {
    LayerArgs a{static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(C), static_cast<uint16_t *>(y),
                nullptr, nullptr, (int32_t)rows, (int32_t)d_out, (int32_t)(d_in * 8), 1, 1};
    return launch<kChebyshev>(a, s);
}

hipError_t launch_linear_forward(const void *y, const void *W, void *z, int64_t rows, int64_t d_in,
                                 int64_t d_out, hipStream_t s) {
    LayerArgs a{static_cast<const uint16_t *>(y), static_cast<const uint16_t *>(W), static_cast<uint16_t *>(z),
                nullptr, nullptr, (int32_t)rows, (int32_t)d_out, (int32_t)d_in, 1, 1};
    return launch<kPlain>(a, s);
}

}  // namespace grkan
