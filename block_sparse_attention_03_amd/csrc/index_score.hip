// index_score.hip -- MSA index-branch block scores on CDNA4 matrix cores.
//
// What it computes (aivizor serving-report news item, paragraph on the two
// MSA stages; youmind page, MSA figure caption): for every query token t and
// KV group g, and every KV block b of the query's sequence,
//   score[t,g,b] = max over tokens j of block b with j <= p(t) of
//                  sum_i q_idx[t,g,i] * k_idx[j,i]          (fp32 accumulate)
// and -inf for blocks after the query's own block p/Bk.
//
// Mapping.  One wavefront owns one (sequence, index head, block): it holds
// the block's 128 x 64 index keys in registers as matrix-core A operands
// (tokens = rows) and sweeps the sequence's (query, group) rows 16 at a time
// as B operands, so the block is read from HBM once whatever the number of
// queries.  Each 16x16x32 bf16 product yields 4 token scores per lane for one
// row; the block maximum is a register max followed by two cross-lane steps.
// In decode (one query per sequence) the kernel is a single pass over the
// index-key cache: it is HBM-bound, and the matrix core keeps the ALU work
// far below the load time.
#include "msa_common.hpp"

namespace msa {
namespace {

constexpr int kScoreWaves = 4;  // blocks per workgroup (one per wavefront)

__global__ __launch_bounds__(kScoreWaves * kWave)
void index_score_kernel(const uint16_t* __restrict__ q_idx,   // [T, Hkv, 64]
                        const uint16_t* __restrict__ kidx,    // [P, Hidx, 128, 64]
                        const int32_t* __restrict__ block_table,
                        const int32_t* __restrict__ seq_lens,
                        const int32_t* __restrict__ cu_q,
                        float* __restrict__ scores,           // [T, Hkv, maxblk]
                        int Hkv, int Hidx, int maxblk) {
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int b = blockIdx.x * kScoreWaves + wave;
    const int s = blockIdx.y / Hidx;
    const int ih = blockIdx.y % Hidx;
    if (b >= maxblk) return;

    const int L = seq_lens[s];
    const int q0 = cu_q[s];
    const int nq = cu_q[s + 1] - q0;
    if (nq <= 0) return;
    const int R = (Hidx == 1) ? Hkv : 1;  // rows per query served by this index head
    const int nrows = nq * R;
    const int first_pos = L - nq;          // position of the sequence's first query

    // Rows whose own block is before b see nothing of block b: -inf.  If that
    // holds for every row, skip the loads.
    const int last_pos = L - 1;
    const bool any_visible = (b * kBlock <= last_pos);
    const int m_in = lane % 16;  // row of A / column of B and of the result
    const int kg = lane / 16;    // lane group: reduction-index slice / result row quad

    if (!any_visible) {
        for (int r0 = 0; r0 < nrows; r0 += kWave) {
            const int rho = r0 + lane;
            if (rho < nrows) {
                const int t = q0 + rho / R;
                const int g = (Hidx == 1) ? (rho % R) : ih;
                scores[((size_t)t * Hkv + g) * maxblk + b] = -__builtin_inff();
            }
        }
        return;
    }

    // A operands: the block's index keys.  Tile mt covers tokens 16*mt..16*mt+15;
    // k-step i of lane group kg takes dims 32*i + 8*kg .. +7 of the token row.
    const int page = block_table[(size_t)s * maxblk + b];
    const uint16_t* kb = kidx + ((size_t)page * Hidx + ih) * kBlock * kIdxDim;
    bf16x8 a[8][2];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
        const uint16_t* row = kb + (mt * 16 + m_in) * kIdxDim;
#pragma unroll
        for (int i = 0; i < 2; ++i) a[mt][i] = as_bf16x8(ld16(row + 32 * i + 8 * kg));
    }

    const int tok0 = b * kBlock;
    for (int r0 = 0; r0 < nrows; r0 += 16) {
        const int rho = r0 + m_in;
        const bool row_ok = rho < nrows;
        const int qi = row_ok ? rho / R : 0;
        const int t = q0 + qi;
        const int g = (Hidx == 1) ? (row_ok ? rho % R : 0) : ih;
        const int p = first_pos + qi;
        bf16x8 bq[2];
        const uint16_t* qrow = q_idx + ((size_t)t * Hkv + g) * kIdxDim;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            u32x4 v = row_ok ? ld16(qrow + 32 * i + 8 * kg) : u32x4{0u, 0u, 0u, 0u};
            bq[i] = as_bf16x8(v);
        }
        float best = -__builtin_inff();
        // tokens of this lane: tok0 + 16*mt + 4*kg + r; visible iff <= p
        const int lim = p - tok0 - 4 * kg;  // visible iff 16*mt + r <= lim
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = mfma16(a[mt][0], bq[0], acc);
            acc = mfma16(a[mt][1], bq[1], acc);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float v = (16 * mt + r <= lim) ? acc[r] : -__builtin_inff();
                best = fmaxf(best, v);
            }
        }
        best = wave_max_xor(best, 16);
        best = wave_max_xor(best, 32);
        if (kg == 0 && row_ok) scores[((size_t)t * Hkv + g) * maxblk + b] = best;
    }
}

}  // namespace
}  // namespace msa

hipError_t msa_launch_index_score(const MsaShape& s, int total_q, const uint16_t* q_idx,
                                  const uint16_t* kidx, const int32_t* block_table,
                                  const int32_t* seq_lens, const int32_t* cu_q, float* scores,
                                  hipStream_t st) {
    using namespace msa;
    if (total_q == 0) return hipSuccess;
    dim3 grid(ceil_div(s.maxblk, kScoreWaves), s.B * s.Hidx);
    hipLaunchKernelGGL(index_score_kernel, grid, dim3(kScoreWaves * kWave), 0, st, q_idx, kidx,
                       block_table, seq_lens, cu_q, scores, s.Hkv, s.Hidx, s.maxblk);
    return hipGetLastError();
}
