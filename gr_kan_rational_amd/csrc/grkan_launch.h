// grkan_launch.h -- internal interface between the C ABI (grkan_api.hip) and
// the kernel translation units.  Not installed; callers use include/grkan.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "grkan.h"

namespace grkan {

// Geometry of one launch over a [rows][d] tensor split into n_groups groups.
// The tensor is cut into tiles of unroll * rows_per_iter rows; one workgroup
// handles one (tile, group) pair: its `lanes` threads cover rows_per_iter
// rows x the group's seg_vecs 16-byte vectors, `unroll` times over.  The
// block is `lanes` rounded up to whole waves (the extra lanes idle).
struct Geometry {
    int64_t rows;
    int64_t row_vecs;       // 16-byte vectors per row (d * bytes / 16)
    int32_t seg_vecs;       // 16-byte vectors per group per row
    int32_t rows_per_iter;  // rows covered by one pass of a workgroup's lanes
    int32_t lanes;          // rows_per_iter * seg_vecs
    int32_t block;          // lanes rounded up to a multiple of 64
    int32_t n_groups;
    int32_t unroll;         // passes per tile
    int64_t tiles;          // ceil(rows / (unroll * rows_per_iter))
    int64_t grid;           // 8 * n_groups * ceil(tiles / 8)
};

struct FwdArgs {
    const void *x;
    void *y;
    const float *A;
    const float *B;
    Geometry geo;
};

enum BwdMode : int32_t { kModeAtomic = 0, kModePartials = 1 };

struct BwdArgs {
    const void *x;
    const void *dy;
    void *dx;
    const float *A;
    const float *B;
    float *dA;
    float *dB;
    float *partials;  // [n_groups][10][8 * ceil(tiles / 8)] in kModePartials
    int32_t mode;
    Geometry geo;
};

// Passes per workgroup and target workgroup size of a kernel (pass 0 =
// forward, 1 = backward; the backward's atomic mode has its own block size).
int unroll(grkan_dtype_t io, int pass);
int target_block(grkan_dtype_t io, int pass, bool atomic_mode);

hipError_t launch_forward(grkan_dtype_t io, const FwdArgs &a, hipStream_t s);
hipError_t launch_backward(grkan_dtype_t io, const BwdArgs &a, hipStream_t s);
hipError_t launch_merge(const float *partials, int32_t n_groups, int64_t tiles, float *dA,
                        float *dB, hipStream_t s);
hipError_t launch_zero(float *dA, float *dB, int32_t n_groups, hipStream_t s);
hipError_t launch_naive(grkan_dtype_t io, const void *x, const void *dy, void *dx, const float *A,
                        const float *B, float *dA, float *dB, int64_t rows, int64_t d,
                        int32_t n_groups, hipStream_t s);

// Resident workgroups per CU for the kernel of (io, pass) at this block size.
hipError_t occupancy(grkan_dtype_t io, int pass, int block, int *blocks_per_cu);

}  // namespace grkan
