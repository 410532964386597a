// gdn_bf16.h - the fp32 -> bf16 (hi, lo) split of an activation, shared by the
// projections' split pass and the single-launch decode's epilogue so the two write
// the same bits.
#pragma once

#include <hip/hip_runtime.h>

namespace gdn {

// fp32 -> bf16 bits, round to nearest even.  NaN stays a quiet NaN; a finite value
// that would round up to infinity is truncated instead (stays finite).
__device__ __forceinline__ unsigned bf16_rne(float x) {
    const unsigned u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    const unsigned r = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    const bool finite = (u & 0x7f800000u) != 0x7f800000u;
    return (finite && (r & 0x7f80u) == 0x7f80u) ? (u >> 16) : r;
}

// hi = bf16(x), lo = bf16(x - hi); x - hi is exact in fp32, and an infinite or NaN hi
// carries the whole value (lo = 0)
__device__ __forceinline__ void split_bf16(float x, unsigned& hi, unsigned& lo) {
    hi = bf16_rne(x);
    lo = (hi & 0x7f80u) == 0x7f80u ? 0u : bf16_rne(x - __uint_as_float(hi << 16));
}

}  // namespace gdn
