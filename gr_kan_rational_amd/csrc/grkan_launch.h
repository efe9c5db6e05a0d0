// grkan_launch.h -- internal interface between the C ABI (grkan_api.hip) and
// the kernel translation units.  Not installed; callers use include/grkan.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "grkan.h"

namespace grkan {

// Geometry of one launch over a [rows][d] tensor split into n_groups groups.
// A workgroup (group g, slice p) walks "steps" of rows_per_iter rows; its
// lanes tile those rows x the group's seg_vecs 16-byte vectors, so a lane
// always touches the same column of the group and only the row changes.
struct Geometry {
    int64_t rows;
    int64_t row_vecs;       // 16-byte vectors per row (d * bytes / 16)
    int32_t seg_vecs;       // 16-byte vectors per group per row
    int32_t rows_per_iter;  // rows covered by one step of a workgroup
    int32_t block;          // threads per workgroup = rows_per_iter * seg_vecs
    int32_t n_groups;
    int32_t slices;         // workgroups per group
    int64_t steps;          // ceil(rows / rows_per_iter)
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
    double *partials;  // [n_groups][slices][10] in kModePartials
    int32_t mode;
    Geometry geo;
};

// Compile-time loop unroll (steps whose loads are issued together).
int unroll(grkan_dtype_t io, int pass);

hipError_t launch_forward(grkan_dtype_t io, const FwdArgs &a, hipStream_t s);
hipError_t launch_backward(grkan_dtype_t io, const BwdArgs &a, hipStream_t s);
hipError_t launch_merge(const double *partials, int32_t n_groups, int32_t slices, float *dA,
                        float *dB, hipStream_t s);
hipError_t launch_zero(float *dA, float *dB, int32_t n_groups, hipStream_t s);
hipError_t launch_naive(grkan_dtype_t io, const void *x, const void *dy, void *dx, const float *A,
                        const float *B, float *dA, float *dB, int64_t rows, int64_t d,
                        int32_t n_groups, hipStream_t s);

// Resident workgroups per CU for the kernel of (io, pass) at this block size.
hipError_t occupancy(grkan_dtype_t io, int pass, int block, int *blocks_per_cu);

}  // namespace grkan
