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
// (tile, group).  The plan depends only on the shape and dtype, never on the
// device, so the deterministic mode gives the same bits on every device.
#include <limits.h>
#include <stdint.h>

#include <cstdlib>
#include <mutex>

#include "grkan.h"
#include "grkan_launch.h"

using namespace grkan;

namespace {

constexpr int kCoefs = 10;

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

// Shape checks and the launch plan (a function of the shape and dtype only).
grkan_status_t plan_shape(int64_t rows, int64_t d, int32_t n_groups, grkan_dtype_t io, int pass,
                          bool atomic_mode, Geometry *G) {
    if (io != GRKAN_F32 && io != GRKAN_BF16) return GRKAN_ERR_INVALID_ARG;
    if (rows < 0 || d <= 0 || n_groups <= 0 || d % n_groups != 0) return GRKAN_ERR_INVALID_ARG;
    const int es = io_bytes(io);
    if (d > INT64_MAX / es || (rows > 0 && rows > INT64_MAX / (d * es))) return GRKAN_ERR_INVALID_ARG;
    const int64_t seg_bytes = (d / n_groups) * es;
    if (seg_bytes % 16 != 0) return GRKAN_ERR_UNSUPPORTED;
    const int64_t seg_vecs = seg_bytes / 16;
    if (seg_vecs > 1024) return GRKAN_ERR_UNSUPPORTED;

    // Rows per pass: the whole-wave block (a multiple of 64 lanes, so the DPP
    // wave sums see only real lanes) closest to the kernel's target size; if
    // no multiple of seg_vecs up to 1024 is a multiple of 64, pad the block
    // with idle lanes instead.
    const int kTargetBlock = target_block(io, pass, atomic_mode);
    int rpi = 0;
    for (int k = 1; k * seg_vecs <= 1024; ++k) {
        const int w = k * (int)seg_vecs;
        if (w % 64 != 0) continue;
        if (rpi == 0 || std::abs(w - kTargetBlock) < std::abs(rpi * (int)seg_vecs - kTargetBlock)) rpi = k;
    }
    if (rpi == 0) {
        rpi = kTargetBlock / (int)seg_vecs;
        if (rpi < 1) rpi = 1;
    }
    const int lanes = rpi * (int)seg_vecs;
    const int u = unroll(io, pass);
    G->rows = rows;
    G->row_vecs = d * es / 16;
    G->seg_vecs = (int32_t)seg_vecs;
    G->rows_per_iter = rpi;
    G->lanes = lanes;
    G->block = (lanes + 63) / 64 * 64;
    G->n_groups = n_groups;
    G->unroll = u;
    const int64_t tile_rows = (int64_t)u * rpi;
    G->tiles = (rows + tile_rows - 1) / tile_rows;
    G->grid = 8 * (int64_t)n_groups * ((G->tiles + 7) / 8);
    if (G->grid > INT32_MAX) return GRKAN_ERR_UNSUPPORTED;
    return GRKAN_OK;
}

// fp32 partials [n_groups][10][8 * ceil(tiles / 8)] (one slot per tile, grouped by XCD).
size_t partials_bytes(const Geometry &G) {
    return (size_t)G.n_groups * kCoefs * (size_t)(8 * ((G.tiles + 7) / 8)) * sizeof(float);
}

// Per-device CU count and occupancy, for grkan_query_launch only.
constexpr int kMaxDev = 64;
std::mutex g_mu;
int g_cus[kMaxDev];

grkan_status_t from_hip(hipError_t e) { return e == hipSuccess ? GRKAN_OK : GRKAN_ERR_HIP; }

}  // namespace

extern "C" const char *grkan_status_string(grkan_status_t status) {
    switch (status) {
    case GRKAN_OK: return "GRKAN_OK: success";
    case GRKAN_ERR_INVALID_ARG: return "GRKAN_ERR_INVALID_ARG: invalid argument";
    case GRKAN_ERR_UNSUPPORTED: return "GRKAN_ERR_UNSUPPORTED: unsupported shape or alignment";
    case GRKAN_ERR_HIP: return "GRKAN_ERR_HIP: HIP runtime error";
    }
    return "GRKAN: unknown status";
}

extern "C" grkan_status_t grkan_forward(const void *x, void *y, const float *A, const float *B,
                                        int64_t rows, int64_t d, int32_t n_groups,
                                        grkan_dtype_t io, hipStream_t stream) {
    Geometry G;
    grkan_status_t st = plan_shape(rows, d, n_groups, io, 0, false, &G);
    if (st != GRKAN_OK) return st;
    if (!A || !B) return GRKAN_ERR_INVALID_ARG;
    if (!aligned(A, 4) || !aligned(B, 4)) return GRKAN_ERR_UNSUPPORTED;
    if (rows == 0) return GRKAN_OK;
    if (!x || !y) return GRKAN_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(y, 16)) return GRKAN_ERR_UNSUPPORTED;
    const size_t bytes = (size_t)rows * (size_t)d * io_bytes(io);
    if (bad_alias(x, y, bytes)) return GRKAN_ERR_INVALID_ARG;
    const size_t cb = (size_t)n_groups * 6 * 4, bb = (size_t)n_groups * 4 * 4;
    if (overlap(y, bytes, A, cb) || overlap(y, bytes, B, bb)) return GRKAN_ERR_INVALID_ARG;

    FwdArgs a{x, y, A, B, G};
    return from_hip(launch_forward(io, a, stream));
}

extern "C" size_t grkan_backward_workspace_size(int64_t rows, int64_t d, int32_t n_groups,
                                                grkan_dtype_t io, uint32_t flags) {
    if (flags != 0) return 0;
    Geometry G;
    if (plan_shape(rows, d, n_groups, io, 1, false, &G) != GRKAN_OK) return 0;
    return partials_bytes(G);
}

extern "C" grkan_status_t grkan_backward(const void *x, const void *dy, const float *A,
                                         const float *B, void *dx, float *dA, float *dB,
                                         int64_t rows, int64_t d, int32_t n_groups,
                                         grkan_dtype_t io, uint32_t flags, void *workspace,
                                         size_t workspace_bytes, hipStream_t stream) {
    Geometry G;
    if (flags & ~(uint32_t)(GRKAN_BLOCK_ATOMIC | GRKAN_NAIVE_ATOMIC)) return GRKAN_ERR_INVALID_ARG;
    if ((flags & GRKAN_BLOCK_ATOMIC) && (flags & GRKAN_NAIVE_ATOMIC)) return GRKAN_ERR_INVALID_ARG;
    grkan_status_t st = plan_shape(rows, d, n_groups, io, 1, flags != 0, &G);
    if (st != GRKAN_OK) return st;
    if (!A || !B || !dA || !dB) return GRKAN_ERR_INVALID_ARG;
    if (!aligned(A, 4) || !aligned(B, 4) || !aligned(dA, 4) || !aligned(dB, 4))
        return GRKAN_ERR_UNSUPPORTED;
    const size_t bytes = (size_t)rows * (size_t)d * io_bytes(io);
    const size_t ab = (size_t)n_groups * 6 * 4, bb = (size_t)n_groups * 4 * 4;
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
    const bool det = flags == 0;
    if (det && rows > 0) {
        const size_t need = partials_bytes(G);
        if (!workspace || workspace_bytes < need) return GRKAN_ERR_INVALID_ARG;
        if (!aligned(workspace, 16)) return GRKAN_ERR_UNSUPPORTED;
        for (int i = 0; i < 5; ++i)
            if (overlap(workspace, need, others[i], sizes[i])) return GRKAN_ERR_INVALID_ARG;
        if (overlap(workspace, need, dA, ab) || overlap(workspace, need, dB, bb))
            return GRKAN_ERR_INVALID_ARG;
    }

    // ---- validation done; HIP calls from here on
    if (rows == 0) return from_hip(launch_zero(dA, dB, n_groups, stream));
    if (flags & GRKAN_NAIVE_ATOMIC) {
        st = from_hip(launch_zero(dA, dB, n_groups, stream));
        if (st != GRKAN_OK) return st;
        return from_hip(launch_naive(io, x, dy, dx, A, B, dA, dB, rows, d, n_groups, stream));
    }
    BwdArgs a{x, dy, dx, A, B, dA, dB, static_cast<float *>(workspace),
              det ? kModePartials : kModeAtomic, G};
    if (!det) {
        st = from_hip(launch_zero(dA, dB, n_groups, stream));
        if (st != GRKAN_OK) return st;
        return from_hip(launch_backward(io, a, stream));
    }
    st = from_hip(launch_backward(io, a, stream));
    if (st != GRKAN_OK) return st;
    return from_hip(launch_merge(a.partials, n_groups, G.tiles, dA, dB, stream));
}

extern "C" grkan_status_t grkan_query_launch(int64_t rows, int64_t d, int32_t n_groups,
                                             grkan_dtype_t io, int32_t pass,
                                             grkan_launch_t *out) {
    if (!out || pass < 0 || pass > 2) return GRKAN_ERR_INVALID_ARG;
    Geometry G;
    grkan_status_t st = plan_shape(rows, d, n_groups, io, pass ? 1 : 0, pass == 2, &G);
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
    if (occupancy(io, pass ? 1 : 0, G.block, &occ) != hipSuccess) return GRKAN_ERR_HIP;
    out->block = G.block;
    out->rows_per_iter = G.rows_per_iter;
    out->unroll = G.unroll;
    out->tiles = G.tiles;
    out->grid = G.grid;
    out->cus = cus;
    out->blocks_per_cu = occ;
    return GRKAN_OK;
}
