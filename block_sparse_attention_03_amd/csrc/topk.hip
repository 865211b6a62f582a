// topk.hip -- MSA top-k block selection and the decode page table.
//
// Selection (youmind page, bullet "Costo predecible a cualquier longitud":
// k = 16 blocks per query and GQA group): candidates are blocks 0..b_loc of a
// (query, group) row; the own block b_loc is always kept; the rest rank by
// score, equal scores to the lower block index.  Output: the kept blocks in
// ascending order, then -1.
//
// The selection itself (ordered keys, lane-maximum prefilter, ballot-counted
// bitwise threshold search, lower-index tie fill) lives in select.hpp.
//
// Page table (aivizor news item, paragraph on MSA with paged attention): the
// KV-group dimension is flattened into the batch and each row's pages are the
// physical pages of its selected blocks.
#include "select.hpp"

namespace msa {
namespace {

// W wavefronts per row; when W == 1, each of the 4 wavefronts of a workgroup
// takes its own row.  The 8-per-lane form is held to 64 VGPRs, eight
// wavefronts per SIMD (65,536 rows of 512: ~37.5 -> ~36 us, bit-equal).
template <int NPT, int W>
__global__ __launch_bounds__((W == 1 ? 4 : W) * kWave) __attribute__((amdgpu_waves_per_eu(NPT == 8 && W == 1 ? 8 : 1)))
void topk_kernel(const float* __restrict__ scores, const int32_t* __restrict__ seq_lens,
                 const int32_t* __restrict__ cu_q, int32_t* __restrict__ sel, int B, int Hkv,
                 int maxblk, int total_rows) {
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int w = (W == 1) ? 0 : wave;  // wave index within the row
    const int row = (W == 1) ? blockIdx.x * 4 + wave : blockIdx.x;
    // W == 1: one selection scratch per wavefront (each has its own row)
    __shared__ SelectShared<W> sh[W == 1 ? 4 : 1];
    if (row >= total_rows) return;  // W == 1 only: whole wavefront leaves together

    const int t = row / Hkv;
    // score loads do not wait for the sequence lookup; slots past the own
    // block are discarded
    float raw[NPT];
    int page[NPT];
    load_candidates<NPT, W, false>(scores + (size_t)row * maxblk, nullptr, maxblk, w, lane, raw,
                                   page);
    // cu_q == nullptr: decode, query token t is sequence t's only query
    const int p = cu_q ? [&] {
        const SeqInfo si = lookup_seq(cu_q, seq_lens, B, t);
        return si.L - si.nq + (t - si.q0);
    }() : seq_lens[t] - 1;
    int32_t* out = sel + (size_t)row * kTopK;
    select_row<NPT, W>(raw, page, p / kBlock, w, lane, &sh[W == 1 ? wave : 0],
                       [&](int pos, uint32_t, int b, int) { out[pos] = b; });
}

__global__ void page_table_kernel(const int32_t* __restrict__ sel,
                                  const int32_t* __restrict__ block_table,
                                  const int32_t* __restrict__ seq_lens,
                                  int32_t* __restrict__ page_table, int32_t* __restrict__ row_lens,
                                  int Hkv, int maxblk, int rows) {
    const int idx = blockIdx.x * blockDim.x + threadIdx.x;
    const int r = idx / kTopK;
    const int i = idx % kTopK;
    if (r >= rows) return;
    const int s = r / Hkv;
    const int b = sel[(size_t)r * kTopK + i];
    page_table[(size_t)r * kTopK + i] = (b >= 0) ? block_table[(size_t)s * maxblk + b] : -1;
    if (i == 0) {
        int n_sel = 0;
        for (int j = 0; j < kTopK; ++j) n_sel += (sel[(size_t)r * kTopK + j] >= 0);
        const int p = seq_lens[s] - 1;
        const int b_loc = p / kBlock;
        row_lens[r] = (n_sel - 1) * kBlock + (p - kBlock * b_loc + 1);
    }
}

template <int NPT, int W>
hipError_t launch_topk(int rows, const float* scores, const int32_t* seq_lens,
                       const int32_t* cu_q, int32_t* sel, int B, int Hkv, int maxblk,
                       hipStream_t st) {
    if constexpr (W == 1) {
        hipLaunchKernelGGL((topk_kernel<NPT, 1>), dim3(ceil_div(rows, 4)), dim3(4 * kWave), 0,
                           st, scores, seq_lens, cu_q, sel, B, Hkv, maxblk, rows);
    } else {
        hipLaunchKernelGGL((topk_kernel<NPT, W>), dim3(rows), dim3(W * kWave), 0, st, scores,
                           seq_lens, cu_q, sel, B, Hkv, maxblk, rows);
    }
    return hipGetLastError();
}

}  // namespace
}  // namespace msa

hipError_t msa_launch_topk(const MsaShape& s, int total_q, const float* scores,
                           const int32_t* seq_lens, const int32_t* cu_q, int32_t* sel,
                           hipStream_t st) {
    using namespace msa;
    const int rows = total_q * s.Hkv;
    if (rows == 0) return hipSuccess;
    const int m = s.maxblk;
    if (m <= 8 * kWave) return launch_topk<8, 1>(rows, scores, seq_lens, cu_q, sel, s.B, s.Hkv, m, st);
    if (m <= 16 * kWave) return launch_topk<16, 1>(rows, scores, seq_lens, cu_q, sel, s.B, s.Hkv, m, st);
    if (m <= 8 * kWave * 4) return launch_topk<8, 4>(rows, scores, seq_lens, cu_q, sel, s.B, s.Hkv, m, st);
    if (m <= 8 * kWave * 8) return launch_topk<8, 8>(rows, scores, seq_lens, cu_q, sel, s.B, s.Hkv, m, st);
    if (m <= 8 * kWave * 16) return launch_topk<8, 16>(rows, scores, seq_lens, cu_q, sel, s.B, s.Hkv, m, st);
    return launch_topk<16, 16>(rows, scores, seq_lens, cu_q, sel, s.B, s.Hkv, m, st);
}

hipError_t msa_launch_page_table(const MsaShape& s, const int32_t* sel,
                                 const int32_t* block_table, const int32_t* seq_lens,
                                 int32_t* page_table, int32_t* row_lens, hipStream_t st) {
    using namespace msa;
    const int rows = s.B * s.Hkv;
    const int n = rows * kTopK;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(page_table_kernel, dim3(ceil_div(n, 256)), dim3(256), 0, st, sel,
                       block_table, seq_lens, page_table, row_lens, s.Hkv, s.maxblk, rows);
    return hipGetLastError();
}
