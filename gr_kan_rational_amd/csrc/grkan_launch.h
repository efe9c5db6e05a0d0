// grkan_launch.h -- internal interface between the C ABI (grkan_api.hip) and
// the kernel translation units.  Not installed; callers use include/grkan.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "grkan.h"
#include "grkan_fastdiv.h"

namespace grkan {

// Launch plan of one pass over a [rows][d] tensor split into n_groups groups
// of d_g = d / n_groups contiguous channels, where a group's row segment is a
// whole number of 16-byte vectors (seg_vecs of them).
//
// A segment is cut into `parts` column parts of at most part_vecs vectors (one
// part unless the segment is wider than the kernel's target block).  The rows
// are cut into tiles of unroll x rows_per_iter rows.  One workgroup handles
// one (tile, group, part): a 2D block of part_vecs x rows_per_iter lanes, each
// lane one 16-byte vector column of its part, `unroll` rows apart.
//
// Grid: one dimension, 8 * parts * n_groups workgroups per bundle of 8 row
// tiles.  Workgroup b takes tile 8 (b / (8 parts n_groups)) + (b mod 8), and
// (group, part) from (b / 8) mod (parts n_groups), group-major.  The
// dispatcher deals workgroups to the 8 XCDs round-robin, so XCD (b mod 8)
// takes whole row tiles.  (A 3D grid with the same linear order measured
// ~2% slower on MI355X.)  Grids too large for one launch are split into
// launches of whole bundles.
enum PlanKind : int32_t { kSegment = 0, kNarrow = 1 };

struct Plan {
    int32_t kind;           // kSegment, or kNarrow (below)
    int64_t rows;
    int64_t d;
    int32_t n_groups;
    int32_t m, n;           // numerator / denominator degree
    int32_t es;             // bytes per I/O element
    int64_t row_bytes;      // d * es
    int64_t seg_bytes;      // d_g * es
    int32_t seg_vecs;       // 16-byte vectors per group row segment
    int32_t parts;          // column parts per segment
    int32_t part_vecs;      // vectors per part (the last part may be ragged)
    int32_t rows_per_iter;  // rows covered by one pass of a workgroup's lanes
    int32_t unroll;         // passes per tile
    int32_t block;          // part_vecs * rows_per_iter threads
    int64_t tiles;          // ceil(rows / (unroll * rows_per_iter))
    int64_t bundles;        // ceil(tiles / 8)
    int32_t ncoef;          // m + 1 + n gradient sums per group
    int64_t bundles_per_launch;
    FastDiv div_gp;         // division by parts * n_groups
    FastDiv div_parts;      // division by parts
    // Narrow groups (a group row segment that is not a whole number of
    // 16-byte vectors, e.g. one function per channel): each lane owns one
    // channel column (with its own coefficients); a workgroup is 64 channel
    // columns x row_lanes rows, loading `unroll` rows per lane at once (a
    // tile of row_lanes * unroll rows; iters = 1).  `parts` is then the most
    // column blocks one group spans; workgroups per bundle of 8 tiles:
    // 8 * ncb.
    int64_t row_words;      // channels per row
    int32_t ncb;            // column blocks of 64 channels
    int32_t cpb;            // channels per column block
    int32_t d_g;            // channels per group
    int32_t row_lanes;
    int32_t iters;
    FastDiv div_ncb;        // division by ncb
    FastDiv div_dg;         // channel -> group
};

// Workgroups of a plan (padding workgroups of the last bundle included).
__host__ __device__ inline int64_t plan_grid(const Plan &P) { return 8 * (int64_t)P.parts * P.n_groups * P.bundles; }

// Partial-sum slots of the deterministic backward: one per (part, tile),
// [parts][8 * bundles]; within a part, tile t sits at slot
// (t mod 8) * bundles + t / 8, so the tiles of one XCD are adjacent.
__host__ __device__ inline int64_t plan_slots(const Plan &P) { return (int64_t)P.parts * 8 * P.bundles; }

struct FwdArgs {
    const void *x;
    void *y;
    const float *A;
    const float *B;
    Plan plan;
    int64_t bundle0;  // first bundle (segment plans) or first tile (narrow plans) of this launch
};

// kModeDirect: the plan has one tile and one part, so each workgroup's sum is
// its group's whole sum and is stored to dA / dB (no merge; the bits are the
// merge's, which would add that one value to nothing).
enum BwdMode : int32_t { kModeAtomic = 0, kModePartials = 1, kModeDirect = 2 };

struct BwdArgs {
    const void *x;
    const void *dy;
    void *dx;
    const float *A;
    const float *B;
    float *dA;
    float *dB;
    float *partials;  // [n_groups][ncoef][plan_slots] in kModePartials
    int32_t mode;
    Plan plan;
    int64_t bundle0;
    // Optional second output of the GR-KAN bf16 segment backward: F(x) in the
    // I/O type (the layer backward's operand of the weight gradient; may be
    // dy itself, each element being read before it is overwritten).
    void *y = nullptr;
};

// Kernels of one degree pair, defined in grkan_kernels.hip (compiled once per
// supported pair).  pass 0 = forward, 1 = backward.  `repeat` is the number
// of evaluations per element: 1, or 2 / 4 / 8 for the FLOP-inflation probe,
// whose kernels exist for GR-KAN's degrees (5, 4) and segment plans only
// (forward / backward return hipErrorInvalidValue for anything else).
template <int M, int N> struct Kernels {
    // passes per tile; `small`: the count for grids under kSmallGrid workgroups
    static int unroll(grkan_dtype_t io, int pass, bool small);
    static int target_block(grkan_dtype_t io, int pass, bool atomic_mode);
    static hipError_t forward(grkan_dtype_t io, const FwdArgs &a, int repeat, dim3 grid, hipStream_t s);
    static hipError_t backward(grkan_dtype_t io, const BwdArgs &a, int repeat, dim3 grid, hipStream_t s);
    static hipError_t occupancy(grkan_dtype_t io, int pass, int block, int *blocks_per_cu, bool narrow);
    // Narrow-group launch shape: row lanes per block, rows loaded together,
    // batches per tile.
    static void narrow_shape(grkan_dtype_t io, int pass, int *row_lanes, int *unroll, int *iters);
};

// Segment plans whose grid at the usual pass count has fewer workgroups than
// this take the kernels' small-grid pass count (a function of the shape only,
// so the summation order is still the same on every device).
constexpr int64_t kSmallGrid = 4096;

// Forward workgroups on grids that are not small: one wave (a segment's
// vectors per row, times as many rows as fit), 2 passes.  Measured on MI355X
// (forward call): KAT-B 195.5 against 197.5 us for 384-lane workgroups,
// KAT-S hidden 401 against 409, KAT-B hidden bf16 397.5 against 412-415; on
// the small KAT-T grid it was 16 against 12.7 us, which keeps 384 lanes and 1
// pass.  The 2-read / 1-write streaming probe peaks with one-wave
// workgroups too.
constexpr int kFwdWaveBlock = 64;

// Degree pairs compiled into the library: (m, n) with a_0..a_m, b_1..b_n.
// GR-KAN's (5, 4) first.
#define GRKAN_FOR_EACH_DEGREE(X) X(5, 4) X(3, 2) X(4, 3) X(6, 5) X(7, 6) X(2, 1) X(4, 4) X(5, 0)

// Degree-independent kernels (grkan_merge.hip).  The merge adds each
// (group, coefficient)'s partials in one workgroup up to 16384 slots, else in
// chunks of 8192 slots; with more than one chunk it needs merge_chunks(slots)
// fp64 chunk sums per (group, coefficient) of scratch, after the partials in
// the workspace.
// For narrow plans the merge skips the parts a group does not span (d_g,
// cpb > 0); segment plans pass 0, 0.
uint32_t merge_chunks(int64_t slots);
hipError_t launch_merge(const float *partials, double *chunk_sums, int32_t n_groups, int32_t m,
                        int32_t n, int64_t tiles, int64_t bundles, int32_t parts, int32_t narrow_dg,
                        int32_t narrow_cpb, float *dA, float *dB, hipStream_t s);
hipError_t launch_zero(float *dA, float *dB, int64_t na, int64_t nb, hipStream_t s);

// The GR-KAN layer's linear map on MFMA (grkan_layer.hip), bf16 x / W / z:
// z = F(x) W^T with F fused into the GEMM prologue (GR-KAN degrees), and the
// plain z = y W^T.  Callers check: rows, d_out < 2^31, d_in a multiple of
// layer_k_step(), d_in / n_groups a multiple of 8, n_groups at most
// layer_max_groups(), 16-byte aligned x, y, W.
int layer_max_groups();
int layer_k_step();
hipError_t launch_layer_forward(const void *x, const float *A, const float *B, const void *W, void *z,
                                int64_t rows, int64_t d_in, int64_t d_out, int32_t n_groups, hipStream_t s);
hipError_t launch_linear_forward(const void *y, const void *W, void *z, int64_t rows, int64_t d_in,
                                 int64_t d_out, hipStream_t s);
// Weight gradient dW [M][N] (fp32) = dz^T y for bf16 dz [rows][M], y [rows][N]
// (M, N multiples of 8, 16-byte aligned rows), through fp32 split partials
// [wgrad_splits][M][N] (wgrad_partials_bytes of scratch) and a fixed-order sum.
int wgrad_splits(int64_t rows, int64_t M, int64_t N);
size_t wgrad_partials_bytes(int64_t rows, int64_t M, int64_t N);
hipError_t launch_wgrad(const void *dz, const void *y, float *partials, float *dW, int64_t rows, int64_t M,
                        int64_t N, hipStream_t s);
// Chebyshev-KAN layer (degree 7, 8 basis functions per input): forward
// y = bf16(basis(x)) C^T with the basis built while staging (x bf16
// [rows][d_in], C bf16 [d_out][8 d_in]); dC = dy^T basis(x) through the
// weight-gradient kernel (fp32 partials as launch_wgrad with M = d_out,
// N = 8 d_in); dx from G = dy C, computed by the plain GEMM over C^T
// (Ct bf16 [8 d_in][d_out]) whose epilogue turns each bf16 row chunk of G
// (the 8 values of one input) into that input's dx without storing G.
hipError_t launch_cheby_forward(const void *x, const void *C, void *y, int64_t rows, int64_t d_in, int64_t d_out,
                                hipStream_t s);
hipError_t launch_cheby_wgrad(const void *dy, const void *x, float *partials, float *dC, int64_t rows,
                              int64_t d_out, int64_t d_in, hipStream_t s);
hipError_t launch_cheby_g_dx(const void *dy, const void *Ct, const void *x, void *dx, int64_t rows,
                             int64_t d_out, int64_t d_in, hipStream_t s);
// out [C][R] = in [R][C]^T, bf16.
hipError_t launch_transpose16(const void *in, void *out, int64_t R, int64_t C, hipStream_t s);

// Streaming ceiling probe (grkan_probe.hip): c = a XOR b over `bytes` bytes
// (a multiple of 16; 16-byte aligned pointers; checked by the caller).
hipError_t launch_stream_probe(const void *a, const void *b, void *c, int64_t bytes, hipStream_t s);

// Per-element-atomic baseline, GR-KAN degrees only (grkan_naive.hip).
hipError_t launch_naive(grkan_dtype_t io, const void *x, const void *dy, void *dx, const float *A,
                        const float *B, float *dA, float *dB, int64_t rows, int64_t d,
                        int32_t n_groups, hipStream_t s);

}  // namespace grkan
