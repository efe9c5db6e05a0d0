// grkan_fastdiv.h -- division of 31-bit unsigned integers by a divisor fixed
// at launch time, as a multiply-high, an add and a shift (Granlund &
// Montgomery, "Division by invariant integers using multiplication", 1994).
// The kernels divide their workgroup index this way: on gfx950 all three
// operations exist as scalar instructions, whereas a plain integer division
// expands to a float-reciprocal sequence on the vector unit.
//
// For a divisor 1 <= d <= 2^31 let l = ceil(log2 d) and
// m = floor(2^32 (2^l - d) / d) + 1 (which fits in 32 bits).  Then for every
// 0 <= n < 2^31, n / d = (mulhi(n, m) + n) >> l; mulhi(n, m) < n keeps the
// sum below 2^32.
#pragma once

#include <stdint.h>

#ifdef __HIPCC__
#define GRKAN_HD __host__ __device__
#else
#define GRKAN_HD
#endif

namespace grkan {

struct FastDiv {
    uint32_t mul;
    uint32_t shift;
};

inline FastDiv make_fastdiv(uint32_t d) {
    uint32_t l = 0;
    while ((uint64_t(1) << l) < d) ++l;
    const uint64_t m = ((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1;
    return FastDiv{(uint32_t)m, l};
}

GRKAN_HD inline uint32_t fastdiv(uint32_t n, FastDiv f) {
    const uint32_t t = (uint32_t)(((uint64_t)n * f.mul) >> 32);
    return (t + n) >> f.shift;
}

}  // namespace grkan
