// decode_tile.hpp -- the LDS layout of one decode workgroup's page tile,
// shared by the sparse page kernels and the dense decode baseline.
#pragma once

#include "msa_common.hpp"

namespace msa {

constexpr int kDecThreads = 256;
// V sits in LDS as 128 rows (tokens) of 256 B, unpadded; the 16-byte chunk c
// of token t is stored at chunk c ^ 2(t mod 8).  A transpose read takes the
// same 32 B of 16 consecutive tokens, and the swizzle puts any 8 consecutive
// tokens' copies of those 32 B on 8 disjoint sets of 8 banks, so the reads are
// conflict-free; with no padding, four workgroups fit in a compute unit.
__device__ __forceinline__ int vs_off(int t, int d) {  // bf16 offset of (token t, dim d)
    return t * kHeadDim + ((((d >> 3) ^ ((t & 7) << 1))) << 3) + (d & 7);
}
constexpr int kPStride = kBlock + 8;     // bf16 per P row (heads x tokens)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct DecodeShared {
    uint16_t vs[kBlock * kHeadDim];
    uint16_t pl[kMaxGroup * kPStride];
    float red_max[4][kMaxGroup];
    float red_sum[4][kMaxGroup];
};

}  // namespace msa
