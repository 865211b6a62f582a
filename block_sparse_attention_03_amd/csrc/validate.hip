// validate.hip -- device-side check of the content preconditions that the
// host cannot see (sequence lengths, query ranges, block-table entries), for
// callers that want them verified before the hot-path calls.  Not on the hot
// path: one pass over seq_lens, cu_q and the used part of block_table.
#include "../../include/msa.h"
#include "msa_common.hpp"

namespace msa {
namespace {

__global__ void validate_clear_kernel(int32_t* __restrict__ status) { *status = 0; }

// One wavefront per sequence: its length, its query range and the block-table
// entries of its ceil(L / Bk) blocks.  Violations are OR-ed into *status.
__global__ __launch_bounds__(256)
void validate_kernel(const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens,
                     const int32_t* __restrict__ cu_q, int32_t* __restrict__ status, int B,
                     int maxblk, int num_pages, int total_q) {
    const int s = blockIdx.x * 4 + threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    if (s >= B) return;
    int bad = 0;
    const int L = seq_lens[s];
    if (L < 1) bad |= MSA_FAULT_SEQ_LEN;
    if ((int64_t)L > (int64_t)maxblk * kBlock) bad |= MSA_FAULT_SEQ_LEN;
    if (cu_q) {
        const int q0 = cu_q[s], q1 = cu_q[s + 1];
        if (q0 < 0 || q1 < q0 || q1 > total_q || q1 - q0 > L) bad |= MSA_FAULT_CU_Q;
        if (s == 0 && q0 != 0) bad |= MSA_FAULT_CU_Q;
        if (s == B - 1 && q1 != total_q) bad |= MSA_FAULT_CU_Q;
    }
    const int nblk = (L >= 1) ? min(maxblk, ceil_div(L, kBlock)) : 0;
    for (int b = lane; b < nblk; b += kWave) {
        const int pg = block_table[(size_t)s * maxblk + b];
        if (pg < 0 || pg >= num_pages) bad |= MSA_FAULT_BLOCK_TABLE;
    }
    // one atomic per wavefront with any violation
    for (int off = 1; off < kWave; off <<= 1) bad |= __shfl_xor(bad, off, kWave);
    if (lane == 0 && bad) atomicOr(status, bad);
}

}  // namespace
}  // namespace msa

hipError_t msa_launch_validate(const MsaShape& s, int total_q, const int32_t* block_table,
                               const int32_t* seq_lens, const int32_t* cu_q, int32_t* status,
                               hipStream_t st) {
    using namespace msa;
    hipLaunchKernelGGL(validate_clear_kernel, dim3(1), dim3(1), 0, st, status);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || s.B == 0) return e;
    hipLaunchKernelGGL(validate_kernel, dim3(ceil_div(s.B, 4)), dim3(256), 0, st, block_table,
                       seq_lens, cu_q, status, s.B, s.maxblk, s.num_pages, total_q);
    return hipGetLastError();
}
