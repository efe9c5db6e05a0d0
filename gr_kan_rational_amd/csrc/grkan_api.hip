// grkan_api.hip -- the C ABI of libgrkan.so (declared in include/grkan.h):
// argument validation, launch planning and kernel dispatch.
//
// Pages cited
//   [FlashKAT notes]  "FlashKAT: Understanding and Addressing Performance
//                     Bottlenecks in the Kolmogorov-Arnold Transformer",
//                     Paper-Notes page (AAAI 2026), arXiv 2505.13813.
//
// Launch plan.  The pages' Algorithm 2 (section "3. FlashKAT 核函数重构
// （Algorithm 2）") uses a grid of ceil(rows / S_block) row tiles x n_g groups.
// Here likewise: tiles of unroll x rows_per_iter rows, one workgroup per
// (tile, group, column part).  The plan depends only on the shape, dtype and
// degrees, never on the device, so the deterministic mode gives the same bits
// on every device.
#include <limits.h>
#include <stdint.h>

#include <cstdlib>
#include <mutex>

#include "grkan.h"
#include "grkan_launch.h"

using namespace grkan;

namespace {

// ------------------------------------------------------- degree dispatch

struct DegreeOps {
    int m, n;
    int (*unroll)(grkan_dtype_t, int, bool);
    int (*target_block)(grkan_dtype_t, int, bool);
    hipError_t (*forward)(grkan_dtype_t, const FwdArgs &, int, dim3, hipStream_t);
    hipError_t (*backward)(grkan_dtype_t, const BwdArgs &, int, dim3, hipStream_t);
    hipError_t (*occupancy)(grkan_dtype_t, int, int, int *, bool);
    void (*narrow_shape)(grkan_dtype_t, int, int *, int *, int *);
};

#define GRKAN_DEGREE_ENTRY(M, N)                                                                \
    {M, N, &Kernels<M, N>::unroll, &Kernels<M, N>::target_block, &Kernels<M, N>::forward,      \
     &Kernels<M, N>::backward, &Kernels<M, N>::occupancy, &Kernels<M, N>::narrow_shape},
const DegreeOps kDegrees[] = {GRKAN_FOR_EACH_DEGREE(GRKAN_DEGREE_ENTRY)};
#undef GRKAN_DEGREE_ENTRY

const DegreeOps *find_degree(int32_t m, int32_t n) {
    for (const DegreeOps &d : kDegrees)
        if (d.m == m && d.n == n) return &d;
    return nullptr;
}

constexpr int32_t kGrkanM = 5, kGrkanN = 4;

// ------------------------------------------------------------ validation

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Half-open byte ranges overlap (both non-empty).
bool overlap(const void *p, size_t pn, const void *q, size_t qn) {
    if (!p || !q || pn == 0 || qn == 0) return false;
    uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
    return a < b + qn && b < a + pn;
}

// Overlap that is not exact aliasing of equal ranges.
bool bad_alias(const void *p, const void *q, size_t n) { return p != q && overlap(p, n, q, n); }

int io_bytes(grkan_dtype_t io) { return io == GRKAN_BF16 ? 2 : 4; }

constexpr int kMaxBlockThreads = 1024;
constexpr int64_t kMaxGroups = 65535;
constexpr int64_t kMaxLaneSpan = int64_t(1) << 31;  // bytes a workgroup's lanes may span

// Plan for groups whose row segment is not a whole number of 16-byte vectors:
// one channel column per lane, 64 columns per workgroup, long row tiles.
grkan_status_t plan_narrow(int64_t rows, int64_t d, int32_t n_groups, const DegreeOps &deg,
                           grkan_dtype_t io, int pass, Plan *P) {
    const int es = io_bytes(io);
    const int64_t row_bytes = d * es;
    if (d >= (int64_t(1) << 31)) return GRKAN_ERR_UNSUPPORTED;
    int rl = 0, u = 0, it = 0;
    deg.narrow_shape(io, pass, &rl, &u, &it);
    const int64_t tile_rows = (int64_t)rl * u * it;
    if (tile_rows * row_bytes > kMaxLaneSpan) return GRKAN_ERR_UNSUPPORTED;
    *P = Plan{};
    P->kind = kNarrow;
    P->rows = rows;
    P->d = d;
    P->n_groups = n_groups;
    P->m = deg.m;
    P->n = deg.n;
    P->es = es;
    P->row_bytes = row_bytes;
    P->seg_bytes = (d / n_groups) * es;
    P->row_words = d;
    P->cpb = 64;
    P->ncb = (int32_t)((d + 63) / 64);
    P->d_g = (int32_t)(d / n_groups);
    // the most column blocks a run of d_g consecutive channels can touch
    P->parts = (int32_t)((P->d_g - 1 + P->cpb - 1) / P->cpb + 1);
    P->part_vecs = 64;
    P->rows_per_iter = rl;
    P->row_lanes = rl;
    P->unroll = u;
    P->iters = it;
    P->block = 64 * rl;
    P->tiles = (rows + tile_rows - 1) / tile_rows;
    P->bundles = (P->tiles + 7) / 8;
    P->ncoef = deg.m + 1 + deg.n;
    if (plan_slots(*P) > (int64_t)65535 * 8192) return GRKAN_ERR_UNSUPPORTED;
    // Whole bundles of 8 tiles per launch: workgroup indices below 2^31 and
    // work-items below 2^32.
    const int64_t per_bundle = 8 * (int64_t)P->ncb;
    int64_t bpl = (int64_t(1) << 31) / per_bundle;
    const int64_t by_items = ((int64_t(1) << 32) - 1) / (per_bundle * P->block);
    if (by_items < bpl) bpl = by_items;
    if (bpl < 1) return GRKAN_ERR_UNSUPPORTED;
    P->bundles_per_launch = bpl;
    P->div_ncb = make_fastdiv((uint32_t)P->ncb);
    P->div_dg = make_fastdiv((uint32_t)P->d_g);
    return GRKAN_OK;
}

// Shape checks and the launch plan (a function of the shape, dtype and degrees).
// with_f: the backward that also stores F(x) (the layer backward).  Its
// kernel holds every pass's F until the tile's end (F may overwrite dy,
// which the rare sign-fix path re-reads), so it takes the small-grid pass
// count at every size: 96 VGPRs with 2 bf16 passes, against 128 and spills
// with 4 (KAT-B layer 2: 840 against 896 us).
grkan_status_t plan_shape(int64_t rows, int64_t d, int32_t n_groups, const DegreeOps &deg,
                          grkan_dtype_t io, int pass, bool atomic_mode, Plan *P, bool with_f = false) {
    if (io != GRKAN_F32 && io != GRKAN_BF16) return GRKAN_ERR_INVALID_ARG;
    if (rows < 0 || d <= 0 || n_groups <= 0 || d % n_groups != 0) return GRKAN_ERR_INVALID_ARG;
    const int es = io_bytes(io);
    if (d > INT64_MAX / es || (rows > 0 && rows > INT64_MAX / (d * es))) return GRKAN_ERR_INVALID_ARG;
    const int64_t seg_bytes = (d / n_groups) * es;
    if (seg_bytes % 16 != 0) return plan_narrow(rows, d, n_groups, deg, io, pass, P);
    if (n_groups > kMaxGroups) return GRKAN_ERR_UNSUPPORTED;
    const int64_t seg_vecs = seg_bytes / 16;
    const int64_t row_bytes = d * es;

    // Column parts: a segment wider than the target block is split into
    // parts of at most target lanes.  Rows per pass: for a one-part segment,
    // the k with k * seg_vecs a whole number of waves closest to the target
    // (partial waves otherwise).
    const int target = deg.target_block(io, pass, atomic_mode);
    int64_t parts = 1, part_vecs = seg_vecs;
    int rpi = 1;
    if (seg_vecs > target) {
        parts = (seg_vecs + target - 1) / target;
        part_vecs = (seg_vecs + parts - 1) / parts;
        parts = (seg_vecs + part_vecs - 1) / part_vecs;
    } else {
        rpi = 0;
        for (int k = 1; k * seg_vecs <= kMaxBlockThreads; ++k) {
            const int w = k * (int)seg_vecs;
            if (w % 64 != 0) continue;
            if (rpi == 0 || std::abs(w - target) < std::abs(rpi * (int)seg_vecs - target)) rpi = k;
        }
        if (rpi == 0) rpi = target / (int)seg_vecs > 0 ? target / (int)seg_vecs : 1;
    }
    int u = deg.unroll(io, pass, false);
    bool small = false;
    {
        // fewer passes for small grids (see kSmallGrid)
        const int64_t tiles0 = (rows + (int64_t)u * rpi - 1) / ((int64_t)u * rpi);
        const int64_t grid0 = 8 * parts * n_groups * ((tiles0 + 7) / 8);
        small = grid0 < kSmallGrid;
        if (small || with_f) u = deg.unroll(io, pass, true);
    }
    if (pass == 0 && !small) {
        // Large forward grids: one-wave workgroups, as many whole segments as
        // fit in a wave (partial waves allowed) -- the shape that streams best
        // (see kFwdWaveBlock).
        if (seg_vecs > kFwdWaveBlock) {
            parts = (seg_vecs + kFwdWaveBlock - 1) / kFwdWaveBlock;
            part_vecs = (seg_vecs + parts - 1) / parts;
            parts = (seg_vecs + part_vecs - 1) / part_vecs;
            rpi = 1;
        } else {
            parts = 1;
            part_vecs = seg_vecs;
            rpi = kFwdWaveBlock / (int)seg_vecs;
        }
    }
    if ((int64_t)u * rpi * row_bytes > kMaxLaneSpan) return GRKAN_ERR_UNSUPPORTED;
    *P = Plan{};
    P->kind = kSegment;
    P->rows = rows;
    P->d = d;
    P->n_groups = n_groups;
    P->m = deg.m;
    P->n = deg.n;
    P->es = es;
    P->row_bytes = row_bytes;
    P->seg_bytes = seg_bytes;
    P->seg_vecs = (int32_t)seg_vecs;
    P->parts = (int32_t)parts;
    P->part_vecs = (int32_t)part_vecs;
    P->rows_per_iter = rpi;
    P->unroll = u;
    P->block = (int32_t)part_vecs * rpi;
    const int64_t tile_rows = (int64_t)u * rpi;
    P->tiles = (rows + tile_rows - 1) / tile_rows;
    P->bundles = (P->tiles + 7) / 8;
    P->ncoef = deg.m + 1 + deg.n;
    // The merge indexes slots in 32 bits and puts their 8192-slot chunks on a grid dimension.
    if (plan_slots(*P) > (int64_t)65535 * 8192) return GRKAN_ERR_UNSUPPORTED;
    // Whole bundles per launch: workgroup indices below 2^31 and work-items
    // (workgroups x block) below 2^32.
    const int64_t per_bundle = 8 * parts * n_groups;
    int64_t bpl = (int64_t(1) << 31) / per_bundle;
    const int64_t by_items = ((int64_t(1) << 32) - 1) / (per_bundle * P->block);
    if (by_items < bpl) bpl = by_items;
    if (bpl < 1) return GRKAN_ERR_UNSUPPORTED;
    P->bundles_per_launch = bpl;
    P->div_gp = make_fastdiv((uint32_t)(parts * n_groups));
    P->div_parts = make_fastdiv((uint32_t)parts);
    return GRKAN_OK;
}

// Workspace of the deterministic backward: fp32 partials
// [n_groups][ncoef][slots], then (when the merge needs more than one chunk
// per coefficient) fp64 chunk sums [n_groups][ncoef][chunks], 16-byte aligned.
size_t partials_bytes(const Plan &P) {
    return (size_t)P.n_groups * P.ncoef * (size_t)plan_slots(P) * sizeof(float);
}
size_t chunk_sums_offset(const Plan &P) { return (partials_bytes(P) + 15) / 16 * 16; }
size_t workspace_need(const Plan &P) {
    const uint32_t chunks = merge_chunks(plan_slots(P));
    if (chunks <= 1) return partials_bytes(P);
    return chunk_sums_offset(P) + (size_t)P.n_groups * P.ncoef * chunks * sizeof(double);
}

// Per-device CU count, for grkan_query_launch only.
constexpr int kMaxDev = 64;
std::mutex g_mu;
int g_cus[kMaxDev];

grkan_status_t from_hip(hipError_t e) { return e == hipSuccess ? GRKAN_OK : GRKAN_ERR_HIP; }

// Launches cover whole bundles of 8 tiles.
int64_t launch_units(const Plan &P) { return P.bundles; }
int64_t units_per_launch(const Plan &P) { return P.bundles_per_launch; }

// Grid of one launch covering nz bundles.
dim3 grid_of(const Plan &P, int64_t nz) {
    if (P.kind == kNarrow) return dim3((unsigned)(8 * (int64_t)P.ncb * nz));
    return dim3((unsigned)(8 * (int64_t)P.parts * P.n_groups * nz));
}

bool valid_repeat(int32_t repeat) { return repeat == 1 || repeat == 2 || repeat == 4 || repeat == 8; }

grkan_status_t forward_impl(const void *x, void *y, const float *A, const float *B, int64_t rows,
                            int64_t d, int32_t n_groups, int32_t m, int32_t n, grkan_dtype_t io,
                            hipStream_t stream, int32_t repeat = 1) {
    const DegreeOps *deg = find_degree(m, n);
    if (!deg) return (m < 0 || n < 0) ? GRKAN_ERR_INVALID_ARG : GRKAN_ERR_UNSUPPORTED;
    if (!valid_repeat(repeat)) return GRKAN_ERR_INVALID_ARG;
    Plan P;
    grkan_status_t st = plan_shape(rows, d, n_groups, *deg, io, 0, false, &P);
    if (st != GRKAN_OK) return st;
    if (repeat != 1 && (P.kind == kNarrow || m != kGrkanM || n != kGrkanN)) return GRKAN_ERR_UNSUPPORTED;
    if (!A || (n > 0 && !B)) return GRKAN_ERR_INVALID_ARG;
    if (!aligned(A, 4) || !aligned(B, 4)) return GRKAN_ERR_UNSUPPORTED;
    if (rows == 0) return GRKAN_OK;
    if (!x || !y) return GRKAN_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(y, 16)) return GRKAN_ERR_UNSUPPORTED;
    const size_t bytes = (size_t)rows * (size_t)d * io_bytes(io);
    if (bad_alias(x, y, bytes)) return GRKAN_ERR_INVALID_ARG;
    const size_t ab = (size_t)n_groups * (m + 1) * 4, bb = (size_t)n_groups * n * 4;
    if (overlap(y, bytes, A, ab) || overlap(y, bytes, B, bb)) return GRKAN_ERR_INVALID_ARG;

    // ---- validation done; HIP calls from here on
    for (int64_t b0 = 0; b0 < launch_units(P); b0 += units_per_launch(P)) {
        const int64_t nz = (launch_units(P) - b0 < units_per_launch(P)) ? launch_units(P) - b0 : units_per_launch(P);
        FwdArgs a{x, y, A, B, P, b0};
        st = from_hip(deg->forward(io, a, repeat, grid_of(P, nz), stream));
        if (st != GRKAN_OK) return st;
    }
    return GRKAN_OK;
}

// The reduction scheme a flags word asks for: 0 deterministic, 1 per-block
// atomics, 2 per-element atomics, -1 an invalid word (two schemes, or a bit
// that names none).  flags = 0 is the deterministic default.
constexpr uint32_t kSchemeBits = GRKAN_DETERMINISTIC | GRKAN_BLOCK_ATOMIC | GRKAN_NAIVE_ATOMIC;
int scheme_of(uint32_t flags) {
    if (flags & ~kSchemeBits) return -1;
    if (flags & (flags - 1)) return -1;  // more than one bit
    if (flags == GRKAN_BLOCK_ATOMIC) return 1;
    if (flags == GRKAN_NAIVE_ATOMIC) return 2;
    return 0;
}

size_t workspace_impl(int64_t rows, int64_t d, int32_t n_groups, int32_t m, int32_t n,
                      grkan_dtype_t io, uint32_t flags) {
    if (scheme_of(flags) != 0) return 0;
    const DegreeOps *deg = find_degree(m, n);
    if (!deg) return 0;
    Plan P;
    if (plan_shape(rows, d, n_groups, *deg, io, 1, false, &P) != GRKAN_OK) return 0;
    return workspace_need(P);
}

grkan_status_t backward_impl(const void *x, const void *dy, const float *A, const float *B, void *dx,
                             float *dA, float *dB, int64_t rows, int64_t d, int32_t n_groups,
                             int32_t m, int32_t n, grkan_dtype_t io, uint32_t flags,
                             void *workspace, size_t workspace_bytes, hipStream_t stream,
                             int32_t repeat = 1, void *y = nullptr, bool validate_only = false) {
    const int scheme = scheme_of(flags);
    if (scheme < 0) return GRKAN_ERR_INVALID_ARG;
    const bool det = scheme == 0, naive = scheme == 2;
    const DegreeOps *deg = find_degree(m, n);
    if (!deg) return (m < 0 || n < 0) ? GRKAN_ERR_INVALID_ARG : GRKAN_ERR_UNSUPPORTED;
    if (!valid_repeat(repeat)) return GRKAN_ERR_INVALID_ARG;
    if (naive && (m != kGrkanM || n != kGrkanN)) return GRKAN_ERR_UNSUPPORTED;
    Plan P;
    grkan_status_t st = plan_shape(rows, d, n_groups, *deg, io, 1, !det, &P, y != nullptr);
    if (st != GRKAN_OK) return st;
    if (repeat != 1 && (P.kind == kNarrow || m != kGrkanM || n != kGrkanN || naive))
        return GRKAN_ERR_UNSUPPORTED;
    if (!A || !dA || (n > 0 && (!B || !dB))) return GRKAN_ERR_INVALID_ARG;
    if (!aligned(A, 4) || !aligned(B, 4) || !aligned(dA, 4) || !aligned(dB, 4))
        return GRKAN_ERR_UNSUPPORTED;
    const size_t bytes = (size_t)rows * (size_t)d * io_bytes(io);
    const size_t ab = (size_t)n_groups * (m + 1) * 4, bb = (size_t)n_groups * n * 4;
    if (rows > 0) {
        if (!x || !dy || !dx) return GRKAN_ERR_INVALID_ARG;
        if (!aligned(x, 16) || !aligned(dy, 16) || !aligned(dx, 16)) return GRKAN_ERR_UNSUPPORTED;
        if (bad_alias(dx, x, bytes) || bad_alias(dx, dy, bytes)) return GRKAN_ERR_INVALID_ARG;
        if (overlap(dx, bytes, A, ab) || overlap(dx, bytes, B, bb)) return GRKAN_ERR_INVALID_ARG;
    }
    const void *others[] = {x, dy, dx, A, B};
    const size_t sizes[] = {rows > 0 ? bytes : 0, rows > 0 ? bytes : 0, rows > 0 ? bytes : 0, ab, bb};
    if (overlap(dA, ab, dB, bb)) return GRKAN_ERR_INVALID_ARG;
    for (int i = 0; i < 5; ++i)
        if (overlap(dA, ab, others[i], sizes[i]) || overlap(dB, bb, others[i], sizes[i]))
            return GRKAN_ERR_INVALID_ARG;
    if (det && rows > 0 && !validate_only) {
        const size_t need = workspace_need(P);
        if (!workspace || workspace_bytes < need) return GRKAN_ERR_INVALID_ARG;
        if (!aligned(workspace, 16)) return GRKAN_ERR_UNSUPPORTED;
        for (int i = 0; i < 5; ++i)
            if (overlap(workspace, need, others[i], sizes[i])) return GRKAN_ERR_INVALID_ARG;
        if (overlap(workspace, need, dA, ab) || overlap(workspace, need, dB, bb))
            return GRKAN_ERR_INVALID_ARG;
    }

    if (validate_only) return GRKAN_OK;

    // ---- validation done; HIP calls from here on
    const int64_t na = (int64_t)n_groups * (m + 1), nb = (int64_t)n_groups * n;
    if (rows == 0) return from_hip(launch_zero(dA, dB, na, nb, stream));
    if (naive) {
        st = from_hip(launch_zero(dA, dB, na, nb, stream));
        if (st != GRKAN_OK) return st;
        return from_hip(launch_naive(io, x, dy, dx, A, B, dA, dB, rows, d, n_groups, stream));
    }
    if (!det) {
        st = from_hip(launch_zero(dA, dB, na, nb, stream));
        if (st != GRKAN_OK) return st;
    }
    float *partials = static_cast<float *>(workspace);
    // One tile and one part: each workgroup holds its group's whole sum (no merge).
    const bool direct = det && P.tiles == 1 && P.parts == 1;
    const int32_t mode = direct ? kModeDirect : (det ? kModePartials : kModeAtomic);
    for (int64_t b0 = 0; b0 < launch_units(P); b0 += units_per_launch(P)) {
        const int64_t nz = (launch_units(P) - b0 < units_per_launch(P)) ? launch_units(P) - b0 : units_per_launch(P);
        BwdArgs a{x, dy, dx, A, B, dA, dB, partials, mode, P, b0, y};
        st = from_hip(deg->backward(io, a, repeat, grid_of(P, nz), stream));
        if (st != GRKAN_OK) return st;
    }
    if (!det || direct) return GRKAN_OK;
    double *chunk_sums = reinterpret_cast<double *>(static_cast<char *>(workspace) + chunk_sums_offset(P));
    const bool narrow = P.kind == kNarrow;
    return from_hip(launch_merge(partials, chunk_sums, n_groups, m, n, P.tiles, P.bundles, P.parts,
                                 narrow ? P.d_g : 0, narrow ? P.cpb : 0, dA, dB, stream));
}

grkan_status_t query_impl(int64_t rows, int64_t d, int32_t n_groups, int32_t m, int32_t n,
                          grkan_dtype_t io, int32_t pass, grkan_launch_t *out) {
    if (!out || pass < 0 || pass > 2) return GRKAN_ERR_INVALID_ARG;
    const DegreeOps *deg = find_degree(m, n);
    if (!deg) return (m < 0 || n < 0) ? GRKAN_ERR_INVALID_ARG : GRKAN_ERR_UNSUPPORTED;
    Plan P;
    grkan_status_t st = plan_shape(rows, d, n_groups, *deg, io, pass ? 1 : 0, pass == 2, &P);
    if (st != GRKAN_OK) return st;
    int dev = 0, cus = 0, occ = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return GRKAN_ERR_HIP;
    {
        std::lock_guard<std::mutex> lock(g_mu);
        cus = g_cus[dev];
    }
    if (cus == 0) {
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return GRKAN_ERR_HIP;
        std::lock_guard<std::mutex> lock(g_mu);
        g_cus[dev] = cus;
    }
    if (deg->occupancy(io, pass ? 1 : 0, P.block, &occ, P.kind == kNarrow) != hipSuccess) return GRKAN_ERR_HIP;
    out->block = P.block;
    out->rows_per_iter = P.rows_per_iter;
    out->unroll = P.unroll;
    out->tiles = P.tiles;
    out->grid = P.kind == kNarrow ? 8 * P.bundles * P.ncb : plan_grid(P);
    out->cus = cus;
    out->blocks_per_cu = occ;
    out->parts = P.parts;
    out->part_vecs = P.part_vecs;
    return GRKAN_OK;
}

}  // namespace

extern "C" const char *grkan_status_string(grkan_status_t status) {
    switch (status) {
    case GRKAN_OK: return "GRKAN_OK: success";
    case GRKAN_ERR_INVALID_ARG: return "GRKAN_ERR_INVALID_ARG: invalid argument";
    case GRKAN_ERR_UNSUPPORTED: return "GRKAN_ERR_UNSUPPORTED: unsupported shape, degree or alignment";
    case GRKAN_ERR_HIP: return "GRKAN_ERR_HIP: HIP runtime error";
    }
    return "GRKAN: unknown status";
}

// ----------------------------------------------------------------- GR-KAN

extern "C" grkan_status_t grkan_forward(const void *x, void *y, const float *A, const float *B,
                                        int64_t rows, int64_t d, int32_t n_groups,
                                        grkan_dtype_t io, hipStream_t stream) {
    return forward_impl(x, y, A, B, rows, d, n_groups, kGrkanM, kGrkanN, io, stream);
}

extern "C" size_t grkan_backward_workspace_size(int64_t rows, int64_t d, int32_t n_groups,
                                                grkan_dtype_t io, uint32_t flags) {
    return workspace_impl(rows, d, n_groups, kGrkanM, kGrkanN, io, flags);
}

extern "C" grkan_status_t grkan_backward(const void *x, const void *dy, const float *A,
                                         const float *B, void *dx, float *dA, float *dB,
                                         int64_t rows, int64_t d, int32_t n_groups,
                                         grkan_dtype_t io, uint32_t flags, void *workspace,
                                         size_t workspace_bytes, hipStream_t stream) {
    return backward_impl(x, dy, A, B, dx, dA, dB, rows, d, n_groups, kGrkanM, kGrkanN, io, flags,
                         workspace, workspace_bytes, stream);
}

// --------------------------------------------------- streaming ceiling

extern "C" grkan_status_t grkan_stream_probe(const void *a, const void *b, void *c, int64_t bytes,
                                             hipStream_t stream) {
    if (bytes < 0) return GRKAN_ERR_INVALID_ARG;
    if (bytes == 0) return GRKAN_OK;
    if (!a || !b || !c) return GRKAN_ERR_INVALID_ARG;
    if (bytes % 16 != 0 || !aligned(a, 16) || !aligned(b, 16) || !aligned(c, 16)) return GRKAN_ERR_UNSUPPORTED;
    if (bad_alias(c, a, (size_t)bytes) || bad_alias(c, b, (size_t)bytes)) return GRKAN_ERR_INVALID_ARG;
    // ---- validation done; HIP calls from here on
    return from_hip(launch_stream_probe(a, b, c, bytes, stream));
}

// ------------------------------------------- backward without allocation
//
// For callers that cannot allocate (code under HIP graph capture, tight
// serving loops, harnesses that forbid allocation): the deterministic
// backward with its partial sums in a fixed device array of this library
// instead of a caller's workspace.  The array lives as long as the process,
// one copy per device the library runs on.  In host code its name is only a
// stand-in for the symbol: the device address is asked of the runtime once
// per device (hipGetSymbolAddress) and that address is what the kernels get.

namespace {

static __device__ __align__(256) unsigned char scratch[GRKAN_NOALLOC_SCRATCH_BYTES];

void *g_scratch[kMaxDev];

// The device address of `scratch` on the current device; looked up on the
// first call on each device.
grkan_status_t scratch_ptr(void **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return GRKAN_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return GRKAN_ERR_HIP;
        g_scratch[dev] = ptr;
    }
    *out = g_scratch[dev];
    return GRKAN_OK;
}

}  // namespace

extern "C" grkan_status_t grkan_backward_noalloc(const void *x, const void *dy, const float *A,
                                                 const float *B, void *dx, float *dA, float *dB,
                                                 int64_t rows, int64_t d, int32_t n_groups,
                                                 grkan_dtype_t io, hipStream_t stream) {
    const DegreeOps *deg = find_degree(kGrkanM, kGrkanN);
    Plan P;
    grkan_status_t st = plan_shape(rows, d, n_groups, *deg, io, 1, false, &P);
    if (st != GRKAN_OK) return st;
    const size_t need = rows > 0 ? workspace_need(P) : 0;
    if (need > (size_t)GRKAN_NOALLOC_SCRATCH_BYTES) return GRKAN_ERR_UNSUPPORTED;
    // Every other check is backward_impl's, which runs before any HIP call;
    // a null workspace with rows > 0 would be reported as INVALID_ARG there,
    // so the lookup is only skipped when nothing needs the scratch.
    void *ws = nullptr;
    if (need > 0) {
        // validate first with a stand-in (never dereferenced), so that an
        // invalid call makes no HIP call at all
        st = backward_impl(x, dy, A, B, dx, dA, dB, rows, d, n_groups, kGrkanM, kGrkanN, io,
                           GRKAN_DETERMINISTIC, nullptr, 0, stream, 1, nullptr, /*validate_only=*/true);
        if (st != GRKAN_OK) return st;
        st = scratch_ptr(&ws);
        if (st != GRKAN_OK) return st;
    }
    return backward_impl(x, dy, A, B, dx, dA, dB, rows, d, n_groups, kGrkanM, kGrkanN, io,
                         GRKAN_DETERMINISTIC, ws, need, stream);
}

extern "C" grkan_status_t grkan_query_launch(int64_t rows, int64_t d, int32_t n_groups,
                                             grkan_dtype_t io, int32_t pass,
                                             grkan_launch_t *out) {
    return query_impl(rows, d, n_groups, kGrkanM, kGrkanN, io, pass, out);
}

// ------------------------------------------------------------- PAU family

extern "C" int grkan_pau_supported(int32_t m, int32_t n) { return find_degree(m, n) != nullptr; }

extern "C" grkan_status_t grkan_pau_forward(const void *x, void *y, const float *A, const float *B,
                                            int64_t rows, int64_t d, int32_t n_groups, int32_t m,
                                            int32_t n, grkan_dtype_t io, hipStream_t stream) {
    return forward_impl(x, y, A, B, rows, d, n_groups, m, n, io, stream);
}

extern "C" size_t grkan_pau_backward_workspace_size(int64_t rows, int64_t d, int32_t n_groups,
                                                    int32_t m, int32_t n, grkan_dtype_t io,
                                                    uint32_t flags) {
    return workspace_impl(rows, d, n_groups, m, n, io, flags);
}

extern "C" grkan_status_t grkan_pau_backward(const void *x, const void *dy, const float *A,
                                             const float *B, void *dx, float *dA, float *dB,
                                             int64_t rows, int64_t d, int32_t n_groups, int32_t m,
                                             int32_t n, grkan_dtype_t io, uint32_t flags,
                                             void *workspace, size_t workspace_bytes,
                                             hipStream_t stream) {
    return backward_impl(x, dy, A, B, dx, dA, dB, rows, d, n_groups, m, n, io, flags, workspace,
                         workspace_bytes, stream);
}

extern "C" grkan_status_t grkan_pau_query_launch(int64_t rows, int64_t d, int32_t n_groups,
                                                 int32_t m, int32_t n, grkan_dtype_t io,
                                                 int32_t pass, grkan_launch_t *out) {
    return query_impl(rows, d, n_groups, m, n, io, pass, out);
}

// ------------------------------------------------------------ the layer

namespace {

grkan_status_t layer_shape(int64_t rows, int64_t d_in, int64_t d_out) {
    if (rows < 0 || d_in <= 0 || d_out <= 0) return GRKAN_ERR_INVALID_ARG;
    if (rows > INT32_MAX || d_in > INT32_MAX || d_out > INT32_MAX) return GRKAN_ERR_UNSUPPORTED;
    if (d_in % layer_k_step() != 0) return GRKAN_ERR_UNSUPPORTED;
    return GRKAN_OK;
}

}  // namespace

extern "C" grkan_status_t grkan_layer_forward(const void *x, const float *A, const float *B,
                                              const void *W, void *z, int64_t rows, int64_t d_in,
                                              int64_t d_out, int32_t n_groups, hipStream_t stream) {
    grkan_status_t st = layer_shape(rows, d_in, d_out);
    if (st != GRKAN_OK) return st;
    if (n_groups <= 0 || d_in % n_groups != 0) return GRKAN_ERR_INVALID_ARG;
    if (n_groups > layer_max_groups() || (d_in / n_groups) % 8 != 0) return GRKAN_ERR_UNSUPPORTED;
    if (!A || !B || !W) return GRKAN_ERR_INVALID_ARG;
    if (!aligned(A, 4) || !aligned(B, 4) || !aligned(W, 16)) return GRKAN_ERR_UNSUPPORTED;
    if (rows == 0) return GRKAN_OK;
    if (!x || !z) return GRKAN_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(z, 2)) return GRKAN_ERR_UNSUPPORTED;
    const size_t xb = (size_t)rows * d_in * 2, zb = (size_t)rows * d_out * 2, wb = (size_t)d_out * d_in * 2;
    if (overlap(z, zb, x, xb) || overlap(z, zb, W, wb) || overlap(z, zb, A, (size_t)n_groups * 24) ||
        overlap(z, zb, B, (size_t)n_groups * 16))
        return GRKAN_ERR_INVALID_ARG;
    // ---- validation done; HIP calls from here on
    return from_hip(launch_layer_forward(x, A, B, W, z, rows, d_in, d_out, n_groups, stream));
}

// The layer forward with a workspace: the fused form re-evaluates F for every
// 256-column tile of z, so it only pays while z has one such tile; beyond
// that F is evaluated once into the workspace (bf16, the operand the fused
// form rounds to) and the plain product follows (measured on MI355X at the
// KAT-B layers, d_out 3072 / 768: 1.16 / 1.33 ms against 1.56 / 1.48 ms fused).
namespace {

constexpr int64_t kFusedMaxDout = 256;

bool layer_takes_unfused(int64_t d_out) { return d_out > kFusedMaxDout; }

}  // namespace

extern "C" size_t grkan_layer_forward_workspace_size(int64_t rows, int64_t d_in, int64_t d_out,
                                                     int32_t n_groups) {
    if (layer_shape(rows, d_in, d_out) != GRKAN_OK) return 0;
    if (n_groups <= 0 || d_in % n_groups != 0 || n_groups > layer_max_groups() || (d_in / n_groups) % 8 != 0)
        return 0;
    if (rows == 0 || !layer_takes_unfused(d_out)) return 0;
    return (size_t)rows * (size_t)d_in * 2;
}

extern "C" grkan_status_t grkan_layer_forward_ws(const void *x, const float *A, const float *B, const void *W,
                                                 void *z, int64_t rows, int64_t d_in, int64_t d_out,
                                                 int32_t n_groups, void *workspace, size_t workspace_bytes,
                                                 hipStream_t stream) {
    const size_t need = grkan_layer_forward_workspace_size(rows, d_in, d_out, n_groups);
    if (need == 0)  // the fused form, or an argument error that it reports
        return grkan_layer_forward(x, A, B, W, z, rows, d_in, d_out, n_groups, stream);
    // everything grkan_layer_forward checks, then the workspace
    if (!A || !B || !W || !x || !z) return GRKAN_ERR_INVALID_ARG;
    if (!aligned(A, 4) || !aligned(B, 4) || !aligned(W, 16) || !aligned(x, 16) || !aligned(z, 2))
        return GRKAN_ERR_UNSUPPORTED;
    const size_t xb = (size_t)rows * d_in * 2, zb = (size_t)rows * d_out * 2, wb = (size_t)d_out * d_in * 2;
    const size_t ab = (size_t)n_groups * 24, bb = (size_t)n_groups * 16;
    if (overlap(z, zb, x, xb) || overlap(z, zb, W, wb) || overlap(z, zb, A, ab) || overlap(z, zb, B, bb))
        return GRKAN_ERR_INVALID_ARG;
    if (!workspace || workspace_bytes < need) return GRKAN_ERR_INVALID_ARG;
    if (!aligned(workspace, 16)) return GRKAN_ERR_UNSUPPORTED;
    const void *ins[] = {x, W, A, B, z};
    const size_t insz[] = {xb, wb, ab, bb, zb};
    for (int i = 0; i < 5; ++i)
        if (overlap(workspace, need, ins[i], insz[i])) return GRKAN_ERR_INVALID_ARG;
    // ---- validation done; HIP calls from here on
    grkan_status_t st = forward_impl(x, workspace, A, B, rows, d_in, n_groups, kGrkanM, kGrkanN, GRKAN_BF16, stream);
    if (st != GRKAN_OK) return st;
    return from_hip(launch_linear_forward(workspace, W, z, rows, d_in, d_out, stream));
}

extern "C" grkan_status_t grkan_linear_forward(const void *y, const void *W, void *z, int64_t rows,
                                               int64_t d_in, int64_t d_out, hipStream_t stream) {
    grkan_status_t st = layer_shape(rows, d_in, d_out);
    if (st != GRKAN_OK) return st;
    if (!W) return GRKAN_ERR_INVALID_ARG;
    if (!aligned(W, 16)) return GRKAN_ERR_UNSUPPORTED;
    if (rows == 0) return GRKAN_OK;
    if (!y || !z) return GRKAN_ERR_INVALID_ARG;
    if (!aligned(y, 16) || !aligned(z, 2)) return GRKAN_ERR_UNSUPPORTED;
    const size_t yb = (size_t)rows * d_in * 2, zb = (size_t)rows * d_out * 2, wb = (size_t)d_out * d_in * 2;
    if (overlap(z, zb, y, yb) || overlap(z, zb, W, wb)) return GRKAN_ERR_INVALID_ARG;
    // ---- validation done; HIP calls from here on
    return from_hip(launch_linear_forward(y, W, z, rows, d_in, d_out, stream));
}

// Layer backward workspace: W^T, one bf16 [rows][d_in] buffer (dY, then
// Y = F(x) written over it by the activation backward), the activation
// backward's partials, the weight gradient's split partials; each 256-byte
// aligned.
namespace {

struct LayerBwdPlan {
    Plan act;
    size_t off_wt, off_buf, off_act, off_wg, total;
};

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

grkan_status_t layer_bwd_plan(int64_t rows, int64_t d_in, int64_t d_out, int32_t n_groups, LayerBwdPlan *lp) {
    grkan_status_t st = layer_shape(rows, d_in, d_out);
    if (st != GRKAN_OK) return st;
    if (n_groups <= 0 || d_in % n_groups != 0) return GRKAN_ERR_INVALID_ARG;
    if (n_groups > layer_max_groups() || (d_in / n_groups) % 8 != 0) return GRKAN_ERR_UNSUPPORTED;
    if (d_out % layer_k_step() != 0) return GRKAN_ERR_UNSUPPORTED;
    const DegreeOps *deg = find_degree(kGrkanM, kGrkanN);
    st = plan_shape(rows > 0 ? rows : 1, d_in, n_groups, *deg, GRKAN_BF16, 1, false, &lp->act, true);
    if (st != GRKAN_OK) return st;
    lp->off_wt = 0;
    lp->off_buf = align256((size_t)d_in * d_out * 2);
    lp->off_act = lp->off_buf + align256((size_t)rows * d_in * 2);
    lp->off_wg = lp->off_act + align256(workspace_need(lp->act));
    lp->total = lp->off_wg + align256(wgrad_partials_bytes(rows, d_out, d_in));
    return GRKAN_OK;
}

}  // namespace

extern "C" size_t grkan_layer_backward_workspace_size(int64_t rows, int64_t d_in, int64_t d_out,
                                                      int32_t n_groups) {
    LayerBwdPlan lp;
    if (rows <= 0 || layer_bwd_plan(rows, d_in, d_out, n_groups, &lp) != GRKAN_OK) return 0;
    return lp.total;
}

extern "C" grkan_status_t grkan_layer_backward(const void *x, const void *dz, const float *A, const float *B,
                                               const void *W, void *dx, float *dA, float *dB, float *dW,
                                               int64_t rows, int64_t d_in, int64_t d_out, int32_t n_groups,
                                               void *workspace, size_t workspace_bytes, hipStream_t stream) {
    LayerBwdPlan lp;
    grkan_status_t st = layer_bwd_plan(rows, d_in, d_out, n_groups, &lp);
    if (st != GRKAN_OK) return st;
    if (!A || !B || !W || !dA || !dB || !dW) return GRKAN_ERR_INVALID_ARG;
    if (!aligned(A, 4) || !aligned(B, 4) || !aligned(dA, 4) || !aligned(dB, 4) || !aligned(dW, 4) ||
        !aligned(W, 16))
        return GRKAN_ERR_UNSUPPORTED;
    const size_t ab = (size_t)n_groups * 24, bb = (size_t)n_groups * 16, wb = (size_t)d_out * d_in * 2;
    const size_t wgb = (size_t)d_out * d_in * 4;
    const size_t xb = rows > 0 ? (size_t)rows * d_in * 2 : 0, zb = rows > 0 ? (size_t)rows * d_out * 2 : 0;
    if (rows > 0) {
        if (!x || !dz || !dx) return GRKAN_ERR_INVALID_ARG;
        if (!aligned(x, 16) || !aligned(dz, 16) || !aligned(dx, 16)) return GRKAN_ERR_UNSUPPORTED;
        // dx may be x itself (x is last read by the step that writes dx)
        if (bad_alias(dx, x, xb) || overlap(dx, xb, dz, zb) || overlap(dx, xb, W, wb) ||
            overlap(dx, xb, A, ab) || overlap(dx, xb, B, bb))
            return GRKAN_ERR_INVALID_ARG;
    }
    const void *ins[] = {x, dz, W, A, B, dx};
    const size_t insz[] = {xb, zb, wb, ab, bb, xb};
    const void *outs[] = {dA, dB, dW};
    const size_t outsz[] = {ab, bb, wgb};
    for (int o = 0; o < 3; ++o) {
        for (int i = 0; i < 6; ++i)
            if (overlap(outs[o], outsz[o], ins[i], insz[i])) return GRKAN_ERR_INVALID_ARG;
        for (int q = o + 1; q < 3; ++q)
            if (overlap(outs[o], outsz[o], outs[q], outsz[q])) return GRKAN_ERR_INVALID_ARG;
    }
    if (rows > 0) {
        if (!workspace || workspace_bytes < lp.total) return GRKAN_ERR_INVALID_ARG;
        if (!aligned(workspace, 256)) return GRKAN_ERR_UNSUPPORTED;
        for (int i = 0; i < 6; ++i)
            if (overlap(workspace, lp.total, ins[i], insz[i])) return GRKAN_ERR_INVALID_ARG;
        for (int o = 0; o < 3; ++o)
            if (overlap(workspace, lp.total, outs[o], outsz[o])) return GRKAN_ERR_INVALID_ARG;
    }

    // ---- validation done; HIP calls from here on
    if (rows == 0) {
        st = from_hip(launch_zero(dA, dB, (int64_t)n_groups * 6, (int64_t)n_groups * 4, stream));
        if (st != GRKAN_OK) return st;
        return from_hip(launch_zero(dW, dW, (int64_t)d_out * d_in, 0, stream));
    }
    char *ws = static_cast<char *>(workspace);
    void *wt = ws + lp.off_wt, *buf = ws + lp.off_buf;
    // dY = dz W (bf16, over W^T so that both operands are K-contiguous)
    st = from_hip(launch_transpose16(W, wt, d_out, d_in, stream));
    if (st != GRKAN_OK) return st;
    st = from_hip(launch_linear_forward(dz, wt, buf, rows, d_out, d_in, stream));
    if (st != GRKAN_OK) return st;
    // dx, dA, dB: the activation's backward on (x, dY), deterministic scheme; it
    // also stores Y = F(x) (bf16) over dY, from the P and 1/D it forms anyway,
    // so that x is read once.  dx may be x: nothing after this reads x.
    st = backward_impl(x, buf, A, B, dx, dA, dB, rows, d_in, n_groups, kGrkanM, kGrkanN, GRKAN_BF16, 0,
                       ws + lp.off_act, workspace_need(lp.act), stream, 1, buf);
    if (st != GRKAN_OK) return st;
    // dW = dz^T Y
    return from_hip(launch_wgrad(dz, buf, reinterpret_cast<float *>(ws + lp.off_wg), dW, rows, d_out, d_in, stream));
}

// ------------------------------------------------------- Chebyshev KAN

namespace {

constexpr int32_t kChebyDegree = 7;

grkan_status_t cheby_shape(int64_t rows, int64_t d_in, int64_t d_out, int32_t degree) {
    if (rows < 0 || d_in <= 0 || d_out <= 0 || degree < 0) return GRKAN_ERR_INVALID_ARG;
    if (degree != kChebyDegree) return GRKAN_ERR_UNSUPPORTED;
    if (rows > INT32_MAX || d_out > INT32_MAX || d_in > INT32_MAX / 8) return GRKAN_ERR_UNSUPPORTED;
    if ((d_in * 8) % layer_k_step() != 0) return GRKAN_ERR_UNSUPPORTED;
    return GRKAN_OK;
}

struct ChebyBwdPlan {
    size_t off_ct, off_wg, total;
};

grkan_status_t cheby_bwd_plan(int64_t rows, int64_t d_in, int64_t d_out, int32_t degree, ChebyBwdPlan *cp) {
    grkan_status_t st = cheby_shape(rows, d_in, d_out, degree);
    if (st != GRKAN_OK) return st;
    if (d_out % layer_k_step() != 0) return GRKAN_ERR_UNSUPPORTED;
    const int64_t kb = d_in * 8;
    cp->off_ct = 0;
    cp->off_wg = align256((size_t)kb * d_out * 2);
    cp->total = cp->off_wg + align256(wgrad_partials_bytes(rows, d_out, kb));
    return GRKAN_OK;
}

}  // namespace

extern "C" grkan_status_t grkan_chebykan_forward(const void *x, const void *C, void *y, int64_t rows,
                                                 int64_t d_in, int64_t d_out, int32_t degree,
                                                 hipStream_t stream) {
    grkan_status_t st = cheby_shape(rows, d_in, d_out, degree);
    if (st != GRKAN_OK) return st;
    if (!C) return GRKAN_ERR_INVALID_ARG;
    if (!aligned(C, 16)) return GRKAN_ERR_UNSUPPORTED;
    if (rows == 0) return GRKAN_OK;
    if (!x || !y) return GRKAN_ERR_INVALID_ARG;
    if (!aligned(x, 2) || !aligned(y, 2)) return GRKAN_ERR_UNSUPPORTED;
    const size_t xb = (size_t)rows * d_in * 2, yb = (size_t)rows * d_out * 2, cb = (size_t)d_out * d_in * 16;
    if (overlap(y, yb, x, xb) || overlap(y, yb, C, cb)) return GRKAN_ERR_INVALID_ARG;
    // ---- validation done; HIP calls from here on
    return from_hip(launch_cheby_forward(x, C, y, rows, d_in, d_out, stream));
}

extern "C" size_t grkan_chebykan_backward_workspace_size(int64_t rows, int64_t d_in, int64_t d_out,
                                                         int32_t degree) {
    ChebyBwdPlan cp;
    if (rows <= 0 || cheby_bwd_plan(rows, d_in, d_out, degree, &cp) != GRKAN_OK) return 0;
    return cp.total;
}

extern "C" grkan_status_t grkan_chebykan_backward(const void *x, const void *dy, const void *C, void *dx,
                                                  float *dC, int64_t rows, int64_t d_in, int64_t d_out,
                                                  int32_t degree, void *workspace, size_t workspace_bytes,
                                                  hipStream_t stream) {
    ChebyBwdPlan cp;
    grkan_status_t st = cheby_bwd_plan(rows, d_in, d_out, degree, &cp);
    if (st != GRKAN_OK) return st;
    if (d_in % 8 != 0) return GRKAN_ERR_UNSUPPORTED;
    if (!C || !dC) return GRKAN_ERR_INVALID_ARG;
    if (!aligned(C, 16) || !aligned(dC, 4)) return GRKAN_ERR_UNSUPPORTED;
    const size_t xb = rows > 0 ? (size_t)rows * d_in * 2 : 0, yb = rows > 0 ? (size_t)rows * d_out * 2 : 0;
    const size_t cb = (size_t)d_out * d_in * 16, dcb = (size_t)d_out * d_in * 32;
    if (rows > 0) {
        if (!x || !dy || !dx) return GRKAN_ERR_INVALID_ARG;
        if (!aligned(x, 16) || !aligned(dy, 16) || !aligned(dx, 16)) return GRKAN_ERR_UNSUPPORTED;
        // dx may be x itself (each thread reads its x before writing the same bytes of dx,
        // and x is read by the dC step before dx is written)
        if (bad_alias(dx, x, xb) || overlap(dx, xb, dy, yb) || overlap(dx, xb, C, cb)) return GRKAN_ERR_INVALID_ARG;
    }
    const void *ins[] = {x, dy, C, dx};
    const size_t insz[] = {xb, yb, cb, xb};
    for (int i = 0; i < 4; ++i)
        if (overlap(dC, dcb, ins[i], insz[i])) return GRKAN_ERR_INVALID_ARG;
    if (rows > 0) {
        if (!workspace || workspace_bytes < cp.total) return GRKAN_ERR_INVALID_ARG;
        if (!aligned(workspace, 256)) return GRKAN_ERR_UNSUPPORTED;
        for (int i = 0; i < 4; ++i)
            if (overlap(workspace, cp.total, ins[i], insz[i])) return GRKAN_ERR_INVALID_ARG;
        if (overlap(workspace, cp.total, dC, dcb)) return GRKAN_ERR_INVALID_ARG;
    }
    // ---- validation done; HIP calls from here on
    if (rows == 0) return from_hip(launch_zero(dC, dC, d_out * d_in * 8, 0, stream));
    char *ws = static_cast<char *>(workspace);
    const int64_t kb = d_in * 8;
    // dC = dy^T basis(x), the basis built while staging
    st = from_hip(launch_cheby_wgrad(dy, x, reinterpret_cast<float *>(ws + cp.off_wg), dC, rows, d_out, d_in,
                                     stream));
    if (st != GRKAN_OK) return st;
    // G = dy C (bf16), over C^T so that both operands are K-contiguous, turned
    // into dx in the matrix kernel's epilogue (G is never stored)
    st = from_hip(launch_transpose16(C, ws + cp.off_ct, d_out, kb, stream));
    if (st != GRKAN_OK) return st;
    return from_hip(launch_cheby_g_dx(dy, ws + cp.off_ct, x, dx, rows, d_out, d_in, stream));
}

extern "C" grkan_status_t grkan_inflated_forward(const void *x, void *y, const float *A,
                                                 const float *B, int64_t rows, int64_t d,
                                                 int32_t n_groups, grkan_dtype_t io, int32_t repeat,
                                                 hipStream_t stream) {
    return forward_impl(x, y, A, B, rows, d, n_groups, kGrkanM, kGrkanN, io, stream, repeat);
}

extern "C" grkan_status_t grkan_inflated_backward(const void *x, const void *dy, const float *A,
                                                  const float *B, void *dx, float *dA, float *dB,
                                                  int64_t rows, int64_t d, int32_t n_groups,
                                                  grkan_dtype_t io, uint32_t flags, int32_t repeat,
                                                  void *workspace, size_t workspace_bytes,
                                                  hipStream_t stream) {
    return backward_impl(x, dy, A, B, dx, dA, dB, rows, d, n_groups, kGrkanM, kGrkanN, io, flags,
                         workspace, workspace_bytes, stream, repeat);
}
