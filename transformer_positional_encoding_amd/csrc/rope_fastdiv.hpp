// Division of 32-bit unsigned integers by a divisor fixed at launch time,
// with one multiply-high, one add and one shift (the round-up method of
// Granlund and Montgomery, "Division by invariant integers using
// multiplication", 1994). Exact for every dividend below 2^31 and every
// divisor in [1, 2^31); the host builds the magic numbers once per launch.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define ROPE_HD __host__ __device__
#else
#define ROPE_HD
#endif

namespace rope {

struct FastDiv {
    uint32_t d = 1;      // divisor
    uint32_t mul = 1;    // low 32 bits of the 33-bit magic 2^32 + mul
    uint32_t shift = 0;  // ceil(log2(d))
};

inline FastDiv make_fastdiv(uint32_t d)
{
    FastDiv f;
    f.d = d;
    uint32_t s = 0;
    while ((1ull << s) < d) ++s;
    f.shift = s;
    // m = floor(2^32 * (2^s - d) / d) + 1 fits in 32 bits for s <= 31
    f.mul = (uint32_t)(((1ull << 32) * ((1ull << s) - d)) / d + 1);
    return f;
}

ROPE_HD inline uint32_t umulhi32(uint32_t a, uint32_t b)
{
#if defined(__HIP_DEVICE_COMPILE__)
    return __umulhi(a, b);
#else
    return (uint32_t)(((uint64_t)a * b) >> 32);
#endif
}

// n / f.d for n < 2^31
ROPE_HD inline uint32_t fast_div(uint32_t n, const FastDiv& f)
{
    return (uint32_t)(((uint64_t)umulhi32(n, f.mul) + n) >> f.shift);
}

}  // namespace rope
