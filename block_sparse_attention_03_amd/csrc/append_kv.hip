// append_kv.hip -- the new tokens' K, V and index keys into the paged caches.
//
// What it computes (aivizor serving-report news item, paragraph on MSA with
// paged attention: the KV cache is paged, one page per 128-token block): the
// i-th new token of sequence s sits at position p = seq_lens[s] - n_s + i
// (its K/V/k_idx belong to the cache before scoring, decode or prefill), in
// page block_table[s][p / Bk], slot p % Bk.  Every KV group's K and V row and
// every index head's key row of the token are copied there.
//
// Mapping.  One 256-thread workgroup per new token; wavefront 0 finds the
// token's sequence in cu_q, then the workgroup copies the token's rows in
// 16-byte pieces: H_kv x 256 B of K, the same of V and H_idx x 128 B of
// index keys, each a contiguous run on both sides.  Pure data movement.
#include "select.hpp"

namespace msa {
namespace {

constexpr int kAppendThreads = 256;

__global__ __launch_bounds__(kAppendThreads)
void append_kv_kernel(const uint16_t* __restrict__ k_new,     // [T, Hkv, 128]
                      const uint16_t* __restrict__ v_new,     // [T, Hkv, 128]
                      const uint16_t* __restrict__ kidx_new,  // [T, Hidx, 64]
                      const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens,
                      const int32_t* __restrict__ cu_q, uint16_t* __restrict__ k_cache,
                      uint16_t* __restrict__ v_cache, uint16_t* __restrict__ kidx_cache, int B,
                      int Hkv, int Hidx, int maxblk) {
    __shared__ int where[2];  // page, slot
    const int t = blockIdx.x;
    if (threadIdx.x < kWave) {
        const SeqInfo si = lookup_seq(cu_q, seq_lens, B, t);
        const int p = si.L - si.nq + (t - si.q0);
        if (threadIdx.x == 0) {
            where[0] = block_table[(size_t)si.s * maxblk + p / kBlock];
            where[1] = p % kBlock;
        }
    }
    __syncthreads();
    const int page = where[0];
    const int slot = where[1];
    constexpr int kKvPieces = kHeadDim / 8;  // 16-byte pieces per K (or V) row
    constexpr int kIdxPieces = kIdxDim / 8;  // per index-key row
    const int n_kv = Hkv * kKvPieces;
    const int n_all = 2 * n_kv + Hidx * kIdxPieces;
    for (int c = threadIdx.x; c < n_all; c += kAppendThreads) {
        if (c < 2 * n_kv) {
            const bool is_v = c >= n_kv;
            const int cc = is_v ? c - n_kv : c;
            const int g = cc / kKvPieces, piece = cc % kKvPieces;
            const size_t src = ((size_t)t * Hkv + g) * kHeadDim + 8 * piece;
            const size_t dst = (((size_t)page * Hkv + g) * kBlock + slot) * kHeadDim + 8 * piece;
            if (is_v)
                *reinterpret_cast<u32x4*>(v_cache + dst) = ld16(v_new + src);
            else
                *reinterpret_cast<u32x4*>(k_cache + dst) = ld16(k_new + src);
        } else {
            const int cc = c - 2 * n_kv;
            const int ih = cc / kIdxPieces, piece = cc % kIdxPieces;
            const size_t src = ((size_t)t * Hidx + ih) * kIdxDim + 8 * piece;
            const size_t dst = (((size_t)page * Hidx + ih) * kBlock + slot) * kIdxDim + 8 * piece;
            *reinterpret_cast<u32x4*>(kidx_cache + dst) = ld16(kidx_new + src);
        }
    }
}

}  // namespace
}  // namespace msa

hipError_t msa_launch_append_kv(const MsaShape& s, int total_q, const uint16_t* k_new,
                                const uint16_t* v_new, const uint16_t* kidx_new,
                                const int32_t* block_table, const int32_t* seq_lens,
                                const int32_t* cu_q, uint16_t* k_cache, uint16_t* v_cache,
                                uint16_t* kidx_cache, hipStream_t st) {
    using namespace msa;
    if (total_q == 0) return hipSuccess;
    hipLaunchKernelGGL(append_kv_kernel, dim3(total_q), dim3(kAppendThreads), 0, st, k_new, v_new,
                       kidx_new, block_table, seq_lens, cu_q, k_cache, v_cache, kidx_cache, s.B,
                       s.Hkv, s.Hidx, s.maxblk);
    return hipGetLastError();
}
