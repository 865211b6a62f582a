// topk.hip -- MSA top-k block selection and the decode page table.
//
// Selection (youmind page, bullet "Costo predecible a cualquier longitud":
// k = 16 blocks per query and GQA group): candidates are blocks 0..b_loc of a
// (query, group) row; the own block b_loc is always kept; the rest rank by
// score, equal scores to the lower block index.  Output: the kept blocks in
// ascending order, then -1.
//
// Method.  Each candidate becomes a 32-bit key whose unsigned order is the
// float order of its score (-0.0 folded into +0.0); the own block gets the
// largest key.  The kk-th largest key (kk = min(k, b_loc+1)) is found by a
// 32-step bitwise search whose counts come from wavefront ballots and
// popcounts, so no sorting network, LDS histogram or atomics on keys is
// needed.  Keys above the threshold are kept; among keys equal to it, the
// lowest block indices fill the remaining slots.  Candidates are dealt to
// lanes interleaved (block = slot*threads + thread), so loads are coalesced and
// ascending block order is (slot, wave, lane) order: output positions come
// from ballot prefix counts.  A row of up to 1024 candidates is one wavefront;
// longer rows use up to 16 wavefronts that add their counts through LDS.
//
// Page table (aivizor news item, paragraph on MSA with paged attention): the
// KV-group dimension is flattened into the batch and each row's pages are the
// physical pages of its selected blocks.
#include "msa_common.hpp"

namespace msa {
namespace {

__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (f == 0.0f) u = 0u;  // -0.0 and +0.0 compare equal
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

struct SeqInfo {
    int q0, nq, L;  // first query token, query count and cache length of the sequence
};

// Sequence of the wave-uniform query token t.  Lanes read cu_q / seq_lens of
// 64 sequences at once and a ballot counts the sequences that end at or before
// t, so a batch of up to 64 sequences costs one round of loads.  t < cu_q[B].
__device__ __forceinline__ SeqInfo lookup_seq(const int32_t* __restrict__ cu_q,
                                              const int32_t* __restrict__ seq_lens, int B, int t) {
    const int lane = __lane_id();
    for (int base = 0;; base += kWave) {
        const int i = base + lane;
        const bool ok = i < B;
        const int c0 = ok ? cu_q[i] : 0;
        const int c1 = ok ? cu_q[i + 1] : 0x7FFFFFFF;
        const int L = ok ? seq_lens[i] : 0;
        const int cnt = __popcll(__ballot(c1 <= t));
        if (cnt < kWave || base + kWave >= B) {
            SeqInfo r;
            r.q0 = __shfl(c0, cnt, kWave);
            r.nq = __shfl(c1, cnt, kWave) - r.q0;
            r.L = __shfl(L, cnt, kWave);
            return r;
        }
    }
}

// W wavefronts per row; when W == 1, each of the 4 wavefronts of a workgroup
// takes its own row.
template <int NPT, int W>
__global__ __launch_bounds__((W == 1 ? 4 : W) * kWave)
void topk_kernel(const float* __restrict__ scores, const int32_t* __restrict__ seq_lens,
                 const int32_t* __restrict__ cu_q, int32_t* __restrict__ sel, int B, int Hkv,
                 int maxblk, int total_rows) {
    constexpr int kThreads = W * kWave;
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int w = (W == 1) ? 0 : wave;  // wave index within the row
    const int row = (W == 1) ? blockIdx.x * 4 + wave : blockIdx.x;

    __shared__ int cnt_bits[W == 1 ? 1 : 34];
    __shared__ int cnt_eq[W == 1 ? 1 : NPT][W];
    __shared__ int cnt_sel[W == 1 ? 1 : NPT][W];
    if constexpr (W > 1) {
        if (threadIdx.x < 34) cnt_bits[threadIdx.x] = 0;
        __syncthreads();
    }
    if (row >= total_rows) return;  // W == 1 only: whole wavefront leaves together

    const int t = row / Hkv;
    const float* sc = scores + (size_t)row * maxblk;
    // score loads do not wait for the sequence lookup: every slot below maxblk
    // is in the row; slots past the own block are discarded below
    float raw[NPT];
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
        const int c = i * kThreads + w * kWave + lane;
        raw[i] = (c < maxblk) ? sc[c] : 0.f;
    }
    const SeqInfo si = lookup_seq(cu_q, seq_lens, B, t);
    const int p = si.L - si.nq + (t - si.q0);
    const int b_loc = p / kBlock;
    const int ncand = b_loc + 1;
    const int kk = ncand < kTopK ? ncand : kTopK;
    int32_t* out = sel + (size_t)row * kTopK;

    if (ncand <= kTopK) {  // every eligible block is kept
        if (w == 0 && lane < kTopK) out[lane] = (lane < ncand) ? lane : -1;
        return;
    }

    uint32_t key[NPT];
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
        const int c = i * kThreads + w * kWave + lane;
        uint32_t k = 0u;
        if (c < b_loc) k = order_key(raw[i]);
        else if (c == b_loc) k = 0xFFFFFFFFu;
        key[i] = k;
    }

    // kk-th largest key: the largest T with #{key >= T} >= kk.
    uint32_t T = 0u;
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = T | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int i = 0; i < NPT; ++i) cnt += __popcll(__ballot(key[i] >= cand));
        if constexpr (W > 1) {
            if (lane == 0) atomicAdd(&cnt_bits[bit], cnt);
            __syncthreads();
            cnt = cnt_bits[bit];
        }
        if (cnt >= kk) T = cand;
    }

    uint64_t gt[NPT], eq[NPT];
    int n_gt = 0;
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
        gt[i] = __ballot(key[i] > T);
        eq[i] = __ballot(key[i] == T);
        n_gt += __popcll(gt[i]);
    }
    if constexpr (W > 1) {
        if (lane == 0) {
            atomicAdd(&cnt_bits[32], n_gt);
#pragma unroll
            for (int i = 0; i < NPT; ++i) cnt_eq[i][w] = __popcll(eq[i]);
        }
        __syncthreads();
        n_gt = cnt_bits[32];
    }
    const int need = kk - n_gt;  // equal keys still to take, lowest blocks first

    // rank of each equal key in ascending block order -> selection mask
    uint64_t sm[NPT];
    int eq_before = 0;
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
        int base = eq_before;
        int slot_total = __popcll(eq[i]);
        if constexpr (W > 1) {
            slot_total = 0;
            for (int v = 0; v < W; ++v) {
                const int c = cnt_eq[i][v];
                if (v < w) base += c;
                slot_total += c;
            }
        }
        const bool is_eq = (eq[i] >> lane) & 1ull;
        const bool take_eq = is_eq && (base + mbcnt(eq[i]) < need);
        const bool take = ((gt[i] >> lane) & 1ull) || take_eq;
        sm[i] = __ballot(take);
        eq_before += slot_total;
    }
    if constexpr (W > 1) {
        if (lane == 0) {
#pragma unroll
            for (int i = 0; i < NPT; ++i) cnt_sel[i][w] = __popcll(sm[i]);
        }
        __syncthreads();
    }
    int sel_before = 0;
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
        int base = sel_before;
        int slot_total = __popcll(sm[i]);
        if constexpr (W > 1) {
            slot_total = 0;
            for (int v = 0; v < W; ++v) {
                const int c = cnt_sel[i][v];
                if (v < w) base += c;
                slot_total += c;
            }
        }
        if ((sm[i] >> lane) & 1ull) out[base + mbcnt(sm[i])] = i * kThreads + w * kWave + lane;
        sel_before += slot_total;
    }
    if (w == 0 && lane >= kk && lane < kTopK) out[lane] = -1;
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
    if (m <= 16 * kWave * 4) return launch_topk<16, 4>(rows, scores, seq_lens, cu_q, sel, s.B, s.Hkv, m, st);
    if (m <= 16 * kWave * 8) return launch_topk<16, 8>(rows, scores, seq_lens, cu_q, sel, s.B, s.Hkv, m, st);
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
