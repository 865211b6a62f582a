// select.hpp -- top-k block selection of one (query, group) row, shared by
// the standalone selection kernel and the fused decode step.
//
// Rule (youmind page, bullet "Costo predecible a cualquier longitud": k = 16
// blocks per query and GQA group): candidates are blocks 0..b_loc; the own
// block b_loc is always kept; the rest rank by score, equal scores to the
// lower block index; the kept blocks are written in ascending order, then -1.
//
// Method.  Each candidate becomes a 32-bit key whose unsigned order is the
// float order of its score (-0.0 folded into +0.0); the own block gets the
// largest key.  The kk-th largest key (kk = min(k, b_loc+1)) is found by a
// 32-step bitwise search whose counts are wavefront ballot popcounts.  Keys
// above it are kept; among keys equal to it the lowest blocks fill the rest.
// Candidates are dealt to lanes interleaved (block = slot*64 + lane), so the
// score loads are coalesced and ascending block order is (slot, lane) order: output positions are ballot prefix counts.  Long rows are
// split over W wavefronts, each selecting its range's top-k, and one
// wavefront then selects from the survivors.
#pragma once

#include "msa_common.hpp"

namespace msa {

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

// Wave-level selection.  Candidates sit at positions i*64 + lane (i < NPT) in
// ascending block order; idx[i] < 0 marks an empty position.  Keeps
// min(k, #candidates) of them -- the own block b_loc first, then higher score,
// then lower block -- and writes their block indices in ascending order to
// out[0..] (and their scores to out_score if given), then -1 up to k.
template <int NPT>
__device__ void select_wave(const int (&idx)[NPT], const float (&raw)[NPT], int b_loc, int lane,
                            int32_t* out, float* out_score) {
    uint32_t key[NPT];
    int n = 0;
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
        key[i] = idx[i] < 0 ? 0u : (idx[i] == b_loc ? 0xFFFFFFFFu : order_key(raw[i]));
        n += __popcll(__ballot(idx[i] >= 0));
    }
    const int kk = n < kTopK ? n : kTopK;
    uint32_t T = 1u;  // every candidate's key is >= 1 (order_key(-inf) = 0x007FFFFF)
    if (n > kTopK) {
        // kk-th largest key: the largest T with #{key >= T} >= kk.
        T = 0u;
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t cand = T | (1u << bit);
            int cnt = 0;
#pragma unroll
            for (int i = 0; i < NPT; ++i) cnt += __popcll(__ballot(key[i] >= cand));
            if (cnt >= kk) T = cand;
        }
    }
    int n_gt = 0;
    uint64_t gt[NPT], eq[NPT];
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
        gt[i] = __ballot(key[i] > T);
        eq[i] = __ballot(key[i] == T);
        n_gt += __popcll(gt[i]);
    }
    const int need = kk - n_gt;  // keys equal to T still to take, lowest blocks first
    int eq_before = 0, sel_before = 0;
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
        const bool is_eq = (eq[i] >> lane) & 1ull;
        const bool take = ((gt[i] >> lane) & 1ull) || (is_eq && eq_before + mbcnt(eq[i]) < need);
        const uint64_t sm = __ballot(take);
        if (take) {
            const int pos = sel_before + mbcnt(sm);
            out[pos] = idx[i];
            if (out_score) out_score[pos] = raw[i];
        }
        eq_before += __popcll(eq[i]);
        sel_before += __popcll(sm);
    }
    if (lane >= kk && lane < kTopK) {
        out[lane] = -1;
        if (out_score) out_score[lane] = 0.f;
    }
}

// Scratch of the W-wavefront selection: each wavefront's local winners.
template <int W>
struct SelectScratch {
    int32_t idx[W][kTopK];
    float score[W][kTopK];
};

// Loads this thread's candidate scores.  W == 1: block i*64 + lane.  W > 1:
// wavefront w owns the contiguous range [w*NPT*64, (w+1)*NPT*64), block
// w*NPT*64 + i*64 + lane.  Slots past maxblk read nothing.
template <int NPT, int W>
__device__ __forceinline__ void load_candidates(const float* __restrict__ sc, int maxblk, int w,
                                                int lane, float (&raw)[NPT]) {
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
        const int c = w * NPT * kWave + i * kWave + lane;
        raw[i] = (c < maxblk) ? sc[c] : 0.f;
    }
}

// Selects the row's blocks (eligible: 0..b_loc) and writes kTopK entries to
// out (global or LDS).  W == 1 is wave-local.  With W > 1 every thread of the
// W-wavefront workgroup must call it: each wavefront selects its own range's
// top-k with no barrier, and wavefront 0 selects the final k among the
// W*k survivors -- which already sit in ascending block order, so the same
// rule (and tie-break) applies.  The global top-k is contained in the union
// of the ranges' top-k under that total order.
template <int NPT, int W>
__device__ void select_row(const float (&raw)[NPT], int b_loc, int w, int lane,
                           SelectScratch<W>* sh, int32_t* out) {
    int idx[NPT];
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
        const int c = w * NPT * kWave + i * kWave + lane;
        idx[i] = c <= b_loc ? c : -1;
    }
    if constexpr (W == 1) {
        select_wave<NPT>(idx, raw, b_loc, lane, out, nullptr);
    } else {
        select_wave<NPT>(idx, raw, b_loc, lane, sh->idx[w], sh->score[w]);
        __syncthreads();
        if (w == 0) {
            constexpr int N2 = (W * kTopK + kWave - 1) / kWave;
            int idx2[N2];
            float raw2[N2];
#pragma unroll
            for (int i = 0; i < N2; ++i) {
                const int pos = i * kWave + lane;
                const bool ok = pos < W * kTopK;
                idx2[i] = ok ? sh->idx[pos / kTopK][pos % kTopK] : -1;
                raw2[i] = ok ? sh->score[pos / kTopK][pos % kTopK] : 0.f;
            }
            select_wave<N2>(idx2, raw2, b_loc, lane, out, nullptr);
        }
    }
}

}  // namespace msa
