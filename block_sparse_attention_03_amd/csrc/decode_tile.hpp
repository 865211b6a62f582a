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

// K of a wavefront's 32 tokens (32w .. 32w+31 of a page) as eight
// contiguous 1 KB loads: load j covers tokens 32w + 4j .. +3, lane l takes
// token 32w + 4j + l/16, 16-byte chunk l % 16.  Whole lines per instruction,
// where loading in matrix-operand order would request quarter lines.
__device__ __forceinline__ void load_k_rows(const uint16_t* __restrict__ kp, int wave, int lane,
                                            u32x4 (&kraw)[8]) {
    const u32x4* kp4 = reinterpret_cast<const u32x4*>(kp) + 32 * wave * (kHeadDim / 8);
#pragma unroll
    for (int j = 0; j < 8; ++j) kraw[j] = ld16_stream(kp4 + kWave * j + lane);
}

// The loaded rows -> 16x16x32 A operands (rows 32w + 16j + n, dims 32i + 8kg,
// i.e. 16-byte chunk 4i + kg) through this wavefront's 8 KB quarter of the V
// tile: chunk c of local token t sits at chunk c ^ (t mod 8), so both the
// stores and the operand reads are free of bank conflicts.  The caller puts
// a barrier between this and the V tile's own stores.
__device__ __forceinline__ void k_rows_to_operands(const u32x4 (&kraw)[8], int wave, int lane,
                                                   uint16_t* vs, bf16x8 (&ka)[2][4]) {
    u32x4* kst = reinterpret_cast<u32x4*>(vs) + wave * 32 * (kHeadDim / 8);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int t = 4 * j + lane / 16;
        kst[t * 16 + ((lane % 16) ^ (t & 7))] = kraw[j];
    }
    const int n = lane % 16, kg = lane / 16;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = 16 * j + n;
            ka[j][i] = as_bf16x8(kst[t * 16 + ((4 * i + kg) ^ (t & 7))]);
        }
}

struct DecodeShared {
    uint16_t vs[kBlock * kHeadDim];
    uint16_t pl[kMaxGroup * kPStride];
    float red_max[4][kMaxGroup];
    float red_sum[4][kMaxGroup];
};

}  // namespace msa
