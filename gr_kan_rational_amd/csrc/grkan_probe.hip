// grkan_probe.hip -- the streaming ceiling the activation kernels are rated
// against: a kernel with the backward's memory traffic (two tensors read,
// one written, 16-byte non-temporal accesses) and no arithmetic beyond one
// bitwise XOR per word, launched as a one-shot grid of the shortest
// workgroups: one wave, one 16-byte vector per lane and tensor.  That shape
// streamed fastest in a sweep on MI355X at the KAT-B backward's size (1.86 GB
// moved; block x vectors per lane): 64 x 1 6.66-6.68 TB/s, 128 x 1 6.60,
// 256 x 1 6.48-6.57, 1024 x 1 6.53-6.56, 64 x 2 6.40-6.42, 256 x 4 6.44-6.46,
// 512 x 4 5.85, 1024 x 4 5.75; default-policy instead of non-temporal loads
// or stores 3-9% slower; each XCD taking a contiguous run of blocks no
// better.  What it sustains on a device is the most a kernel of this access
// pattern can expect there; the benchmark reports the backward's bandwidth as
// a fraction of it next to the fraction of the published HBM peak.
#include "grkan_launch.h"

namespace grkan {

namespace {

constexpr int kProbeBlock = 64;
constexpr int kProbeUnroll = 1;  // 16-byte vectors per lane per tensor
constexpr int64_t kProbeChunk = (int64_t)kProbeBlock * kProbeUnroll * 16;  // bytes per workgroup per tensor

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kProbeBlock) void grkan_stream_probe_kernel(const char *__restrict__ a,
                                                                         const char *__restrict__ b,
                                                                         char *__restrict__ c, int64_t bytes,
                                                                         int64_t block0) {
    // workgroup w covers bytes [w * kProbeChunk, (w + 1) * kProbeChunk): lane l
    // takes the 16-byte vectors l, l + kProbeBlock, ... of it, so each wave
    // reads whole 1 KB runs per access; all loads are issued before the first
    // store, and only the last, ragged workgroup checks bounds
    const int64_t base = (block0 + (int64_t)blockIdx.x) * kProbeChunk;
    const u32x4 *pa = reinterpret_cast<const u32x4 *>(a + base);
    const u32x4 *pb = reinterpret_cast<const u32x4 *>(b + base);
    u32x4 *pc = reinterpret_cast<u32x4 *>(c + base);
    const int64_t avail = bytes - base;
    const int t = (int)threadIdx.x;
    if (avail >= kProbeChunk) {
        u32x4 va[kProbeUnroll], vb[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) {
            va[u] = __builtin_nontemporal_load(pa + t + u * kProbeBlock);
            vb[u] = __builtin_nontemporal_load(pb + t + u * kProbeBlock);
        }
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) __builtin_nontemporal_store(va[u] ^ vb[u], pc + t + u * kProbeBlock);
    } else {
        const int nv = (int)(avail / 16);
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) {
            const int i = t + u * kProbeBlock;
            if (i < nv) __builtin_nontemporal_store(pa[i] ^ pb[i], pc + i);
        }
    }
}

}  // namespace

hipError_t launch_stream_probe(const void *a, const void *b, void *c, int64_t bytes, hipStream_t s) {
    const int64_t blocks = (bytes + kProbeChunk - 1) / kProbeChunk;
    const int64_t per_launch = ((int64_t(1) << 32) - 1) / kProbeBlock;  // work-items below 2^32
    for (int64_t b0 = 0; b0 < blocks; b0 += per_launch) {
        const int64_t nb = blocks - b0 < per_launch ? blocks - b0 : per_launch;
        hipLaunchKernelGGL(grkan_stream_probe_kernel, dim3((unsigned)nb), dim3(kProbeBlock), 0, s,
                           static_cast<const char *>(a), static_cast<const char *>(b), static_cast<char *>(c),
                           bytes, b0);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace grkan
