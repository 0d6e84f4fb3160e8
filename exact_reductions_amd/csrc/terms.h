// The per-sample terms of the reductions, shared by every kernel of libvqx
// so that all of them add the same integers.
//
// Sources (web pages, cited by title and section):
//   [PSNR]   "ADR-1440: float_psnr_hip adds its squared differences as
//            integers and returns the CPU's score bit for bit"
//   [MOMENT] "ADR-1447: float_moment_hip adds the float squares the CPU adds,
//            and is bit-identical while the CPU's own sum is exact"
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#pragma clang fp contract(off)

namespace vqx {

// The float square of x read back as an integer: one binary32 product, round
// to nearest even, then an exact conversion (the product is an integer below
// 2^32) [MOMENT, Decision].
__device__ __forceinline__ uint32_t float_square(float x)
{
    const float p = x * x;
    return static_cast<uint32_t>(p);
}

// Index of the three square sums: noise, sum of ref squares, sum of dist
// squares.
enum : int { kSqNoise = 0, kSqRef = 1, kSqDist = 2, kSquares = 3 };

// Square term `which` of one sample pair, in units of 1/scaler^2.  At 8 bits
// every square is below 2^16 and so exact in binary32: the integer square is
// the float square [PSNR, Context].
template <int kBytes>
__device__ __forceinline__ uint32_t square_term(int which, uint32_t r, uint32_t d)
{
    if constexpr (kBytes == 1) {
        const int32_t e = static_cast<int32_t>(r) - static_cast<int32_t>(d);
        const uint32_t x = which == kSqNoise ? static_cast<uint32_t>(e * e)
                          : which == kSqRef  ? r * r
                                             : d * d;
        return x;
    } else {
        const float fr = static_cast<float>(r), fd = static_cast<float>(d);
        return which == kSqNoise ? float_square(fr - fd)
             : which == kSqRef   ? float_square(fr)
                                 : float_square(fd);
    }
}

}  // namespace vqx
