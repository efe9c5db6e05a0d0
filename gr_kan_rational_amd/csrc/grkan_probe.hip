// grkan_probe.hip -- the streaming ceiling the activation kernels are rated
// against: a kernel with the backward's memory traffic (two tensors read,
// one written, 16-byte non-temporal accesses) and no arithmetic beyond one
// bitwise XOR per word, launched as a one-shot grid of short workgroups in
// the same style.  What it sustains on a device is the most a kernel of this
// access pattern can expect there; the benchmark reports the backward's
// bandwidth as a fraction of it next to the fraction of the published HBM
// peak.
#include "grkan_launch.h"

namespace grkan {

namespace {

constexpr int kProbeBlock = 256;
constexpr int kProbeUnroll = 4;  // 16-byte vectors per lane per tensor
constexpr int64_t kProbeChunk = (int64_t)kProbeBlock * kProbeUnroll * 16;  // bytes per workgroup per tensor

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kProbeBlock) void grkan_stream_probe_kernel(const u32x4 *__restrict__ a,
                                                                         const u32x4 *__restrict__ b,
                                                                         u32x4 *__restrict__ c, int64_t nvec,
                                                                         int64_t block0) {
    // workgroup w covers vectors [w * 1024, (w + 1) * 1024): lane l takes
    // vectors l, l + 256, l + 512, l + 768 of it, so each wave reads whole
    // 1 KB runs per access
    const int64_t base = (block0 + (int64_t)blockIdx.x) * (kProbeBlock * kProbeUnroll) + threadIdx.x;
    u32x4 va[kProbeUnroll], vb[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) {
        const int64_t i = base + (int64_t)u * kProbeBlock;
        if (i < nvec) {
            va[u] = __builtin_nontemporal_load(a + i);
            vb[u] = __builtin_nontemporal_load(b + i);
        }
    }
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) {
        const int64_t i = base + (int64_t)u * kProbeBlock;
        if (i < nvec) __builtin_nontemporal_store(va[u] ^ vb[u], c + i);
    }
}

}  // namespace

hipError_t launch_stream_probe(const void *a, const void *b, void *c, int64_t bytes, hipStream_t s) {
    const int64_t nvec = bytes / 16;
    const int64_t blocks = (bytes + kProbeChunk - 1) / kProbeChunk;
    const int64_t per_launch = ((int64_t(1) << 32) - 1) / kProbeBlock;  // work-items below 2^32
    for (int64_t b0 = 0; b0 < blocks; b0 += per_launch) {
        const int64_t nb = blocks - b0 < per_launch ? blocks - b0 : per_launch;
        hipLaunchKernelGGL(grkan_stream_probe_kernel, dim3((unsigned)nb), dim3(kProbeBlock), 0, s,
                           static_cast<const u32x4 *>(a), static_cast<const u32x4 *>(b),
                           static_cast<u32x4 *>(c), nvec, b0);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace grkan
