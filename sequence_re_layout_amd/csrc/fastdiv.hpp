// fastdiv.hpp -- division of 31-bit unsigned integers by a run-time invariant
// divisor with one high multiply, an add and a shift.
//
// Method: T. Granlund and P. L. Montgomery, "Division by invariant integers
// using multiplication", PLDI 1994, Sec. 4 (unsigned division, N = 32):
//   l = ceil(log2 d),  m = floor(2^32 * (2^l - d) / d) + 1,
//   q = (mulhi(m, n) + n) >> l.
// The add cannot overflow 32 bits because n < 2^31 and mulhi(m, n) <= n.
// Callers guarantee 1 <= d < 2^31 and n < 2^31.
//
// BASP_HD marks the functions usable in kernels; the including translation
// unit defines it (to "__host__ __device__" in HIP sources).
#pragma once

#include <cstdint>

#ifndef BASP_HD
#error "define BASP_HD before including fastdiv.hpp"
#endif

namespace basp {

struct FastDiv {
    uint32_t d;     // divisor
    uint32_t m;     // magic multiplier
    uint32_t l;     // post-shift
};

inline FastDiv make_fastdiv(uint32_t d)
{
    FastDiv f;
    f.d = d;
    uint32_t l = 0;
    while ((uint64_t{1} << l) < d)
        ++l;
    f.l = l;
    f.m = static_cast<uint32_t>(((uint64_t{1} << 32) * ((uint64_t{1} << l) - d)) / d + 1);
    return f;
}

BASP_HD inline uint32_t fastdiv(uint32_t n, const FastDiv &f)
{
    const uint32_t hi = static_cast<uint32_t>((static_cast<uint64_t>(n) * f.m) >> 32);
    return (hi + n) >> f.l;
}

}  // namespace basp
