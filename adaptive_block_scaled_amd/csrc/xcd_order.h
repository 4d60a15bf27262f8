// Device helper shared by the one-wave dequantize kernels (HIP translation
// units only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace if4 {

// Workgroups are handed to the 8 XCDs in turn (workgroup b to XCD b mod 8),
// and two neighbouring one-wave workgroups of a dequantize share a 128-byte
// line of scale bytes (64 each): on two XCDs both L2s would fetch it.  Within
// each run of 16 workgroups this permutation gives the groups of workgroups
// 2k and 2k + 1 (in tensor order) to workgroups on the same XCD; the last
// nb % 16 keep their own index.  (Giving each XCD one contiguous eighth of
// the tensor also fetches each line once, but streams 8% slower.)
__device__ __forceinline__ int64_t xcd_paired_block(unsigned b, unsigned nb) {
    const unsigned full = nb & ~15u, j = b & 15u;
    return b < full ? (int64_t)(b - j + 2u * (j & 7u) + (j >> 3)) : (int64_t)b;
}

}  // namespace if4
