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
// largest key and an empty slot the key 0.  Candidates are dealt to lanes
// interleaved (block = base + slot*64 + lane), so score loads are coalesced and
// ascending block order is (slot, lane) order.
//
// The kk-th largest key (kk = min(k, #candidates)) comes from a bitwise
// search whose counts are wavefront ballot popcounts.  On this hardware one
// step costs a vector compare per register, each followed by a scalar
// popcount of its lane mask, so the search is run on as few registers as
// possible:
//   1. each lane takes the largest of its keys; the kk-th largest of these 64
//      lane maxima, T0, is at most the kk-th largest key (kk distinct lanes
//      hold a key >= T0), so every key of the selection is >= T0;
//   2. the keys >= T0 (usually a few more than kk) are compacted, in
//      ascending block order, one per lane through LDS;
//   3. each survivor counts the survivors ahead of it (larger key, or equal
//      key and lower block) from broadcast LDS reads of 64-bit (key, order)
//      values -- vector work only -- and the kk survivors with fewer than kk
//      ahead are kept.
// When more than 64 keys are >= T0 (heavy ties) the search runs on all keys;
// keys above its threshold are kept and among keys equal to it the lowest
// blocks fill the rest.  A search stops early once exactly kk keys are >= the
// candidate threshold: those keys are then the selection.
//
// Long rows are split over W wavefronts, each selecting its range's top-k;
// wavefront 0 then selects from the W*k survivors, which already sit in
// ascending block order, so the same rule and tie-break apply.
#pragma once

#include "msa_common.hpp"

namespace msa {

__device__ __forceinline__ uint32_t order_key(float f) {
    // f + 0 turns -0.0 into +0.0 (they compare equal); negative values have
    // all bits flipped, the others only the sign bit
    const uint32_t u = __float_as_uint(f + 0.0f);
    return u ^ (static_cast<uint32_t>(static_cast<int32_t>(u) >> 31) | 0x80000000u);
}

struct SeqInfo {
    int q0, nq, L;  // first query token, query count and cache length of the sequence
    int s;          // the sequence
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
            r.s = base + cnt;
            return r;
        }
    }
}

// A candidate in LDS: ordered key, block index and physical page.
struct alignas(16) Cand {
    uint32_t key;
    int32_t idx;
    int32_t page;
    int32_t pad;
};

// Largest T with #{key >= T} >= kk, or an earlier T with #{key >= T} == kk.
// Either way the keys > T, then the lowest-block keys == T up to kk in all,
// are the kk largest keys with ties to the lower block.  Needs
// 1 <= kk <= #{key >= 1}.
template <int NPT>
__device__ __forceinline__ uint32_t kth_key(const uint32_t (&key)[NPT], int kk) {
    uint32_t T = 0u;
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = T | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int i = 0; i < NPT; ++i) cnt += __popcll(__ballot(key[i] >= cand));
        if (cnt >= kk) {
            T = cand;
            if (cnt == kk) break;
        }
    }
    return T;
}

// Writes the kept candidates (threshold T, see kth_key) in ascending block
// order through out(pos, key, idx_of(i), page_of(i)), then out(pos, 0, -1, -1)
// for the positions kk .. k-1.  idx_of / page_of give the block and page of
// this lane's slot i.
template <int NPT, class Idx, class Page, class Out>
__device__ __forceinline__ void emit(const uint32_t (&key)[NPT], Idx&& idx_of, Page&& page_of,
                                     uint32_t T, int kk, int lane, Out&& out) {
    int n_gt = 0;
#pragma unroll
    for (int i = 0; i < NPT; ++i) n_gt += __popcll(__ballot(key[i] > T));
    const int need = kk - n_gt;  // keys equal to T still to take, lowest blocks first
    int eq_before = 0, sel_before = 0;
#pragma unroll
    for (int i = 0; i < NPT; ++i) {  // masks are formed where used: no per-slot arrays
        const uint64_t eq = __ballot(key[i] == T);
        const bool take = key[i] > T || (key[i] == T && eq_before + mbcnt(eq) < need);
        const uint64_t sm = __ballot(take);
        if (take) out(sel_before + mbcnt(sm), key[i], idx_of(i), page_of(i));
        eq_before += __popcll(eq);
        sel_before += __popcll(sm);
    }
    if (lane >= kk && lane < kTopK) out(lane, 0u, -1, -1);
}

// One wavefront's LDS scratch: compacted survivors and their rank keys.
struct alignas(16) WaveScratch {
    Cand surv[kWave];
    uint64_t rkey[kWave];
};

__device__ __forceinline__ void wave_sync_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One candidate per lane (key 0 = empty), lanes in ascending block order, no
// candidate at or past lane `span`: a lane's rank is the number of lanes ahead
// of it (larger key, or equal key and lower lane), and the kk lanes of rank
// < kk are kept.  Needs kk <= #candidates.
template <class Out>
__device__ __forceinline__ void select_ranked(uint32_t key, int idx, int page, int span, int kk,
                                              int lane, uint64_t* rkey, Out&& out) {
    // rank key (key, 63 - lane): distinct, and larger means ahead
    const uint64_t ci = (static_cast<uint64_t>(key) << 32) | static_cast<uint32_t>(kWave - 1 - lane);
    rkey[lane] = ci;
    wave_sync_lds();
    int rank = 0;
    for (int j0 = 0; j0 < span; j0 += 16) {  // 16 rank keys per pass, read first
        u64x2 cj[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) cj[u] = *reinterpret_cast<const u64x2*>(rkey + j0 + 2 * u);
#pragma unroll
        for (int u = 0; u < 8; ++u) rank += (cj[u][0] > ci ? 1 : 0) + (cj[u][1] > ci ? 1 : 0);
    }
    const bool take = key != 0u && rank < kk;
    const uint64_t sm = __ballot(take);
    if (take) out(mbcnt(sm), key, idx, page);
    if (lane >= kk && lane < kTopK) out(lane, 0u, -1, -1);
}

// Wave-level selection over keys at positions slot*64 + lane (key 0 = empty)
// of which n are candidates; ws is this wavefront's own LDS scratch.  Every
// lane of the wavefront calls it.
template <int NPT, class Idx, class Page, class Out>
__device__ void select_wave(const uint32_t (&key)[NPT], Idx&& idx_of, Page&& page_of, int n,
                            int lane, WaveScratch* ws, Out&& out) {
    const int kk = n < kTopK ? n : kTopK;
    if (n <= kTopK) {  // every candidate is kept
        emit<NPT>(key, idx_of, page_of, 1u, kk, lane, out);
        return;
    }
    if constexpr (NPT == 1) {
        select_ranked(key[0], idx_of(0), page_of(0), kWave, kk, lane, ws->rkey, out);
    } else {
        // 1. threshold from the lane maxima (n > k candidates fill > k lanes)
        uint32_t lm[1] = {key[0]};
#pragma unroll
        for (int i = 1; i < NPT; ++i) lm[0] = max(lm[0], key[i]);
        const uint32_t T0 = kth_key<1>(lm, kk);
        // 2. compact the keys >= T0 in (slot, lane) order; past 64 of them the
        // scratch is not used
        int tot = 0;
#pragma unroll
        for (int i = 0; i < NPT; ++i) {
            const uint64_t sm = __ballot(key[i] >= T0);
            const int pos = tot + mbcnt(sm);
            if (key[i] >= T0 && pos < kWave) {
                Cand c;
                c.key = key[i];
                c.idx = idx_of(i);
                c.page = page_of(i);
                c.pad = 0;
                ws->surv[pos] = c;
            }
            tot += __popcll(sm);
        }
        if (tot <= kWave) {
            wave_sync_lds();
            Cand c;
            c.key = 0u;
            c.idx = -1;
            c.page = -1;
            if (lane < tot) c = ws->surv[lane];
            // 3. rank the survivors
            select_ranked(c.key, c.idx, c.page, tot, kk, lane, ws->rkey, out);
            return;
        }
        emit<NPT>(key, idx_of, page_of, kth_key<NPT>(key, kk), kk, lane, out);
    }
}

// LDS of a W-wavefront row selection: per-wavefront compaction scratch and
// each wavefront's local winners.
template <int W>
struct SelectShared {
    WaveScratch ws[W];
    Cand win[W > 1 ? W : 1][kTopK];
};

// Candidates of wavefront w: W == 1 owns blocks slot*64 + lane; W > 1 owns the
// contiguous range [w*NPT*64, (w+1)*NPT*64).  Slots at or past maxblk re-read
// the last block (they are past b_loc, so their values are never used): the
// loads carry no condition and are all in flight together.  With PAGES the
// block-table entry of each candidate is loaded beside its score (bt_row = the
// sequence's block-table row).
template <int NPT, int W, bool PAGES>
__device__ __forceinline__ void load_candidates(const float* __restrict__ sc,
                                                const int32_t* __restrict__ bt_row, int maxblk,
                                                int w, int lane, float (&raw)[NPT],
                                                int (&page)[NPT]) {
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
        const int c = min(w * NPT * kWave + i * kWave + lane, maxblk - 1);
        raw[i] = sc[c];
        page[i] = PAGES ? bt_row[c] : -1;
    }
}

// Number of candidates (blocks 0..b_loc) in wavefront w's range.
template <int NPT>
__device__ __forceinline__ int wave_candidates(int b_loc, int w) {
    const int n = b_loc + 1 - w * NPT * kWave;
    return n < 0 ? 0 : (n > NPT * kWave ? NPT * kWave : n);
}

// Selects the row's blocks (eligible: 0..b_loc) from the scores loaded by
// load_candidates and reports them through out(pos, key, block, page).  With
// W > 1 every thread of the W-wavefront workgroup must call it (one barrier
// inside) and out is called by wavefront 0 only.
template <int NPT, int W, class Out>
__device__ void select_row(const float (&raw)[NPT], const int (&page)[NPT], int b_loc, int w,
                           int lane, SelectShared<W>* sh, Out&& out) {
    // b_loc and w are the same on every lane of the wavefront; saying so keeps
    // the counts, kk and the thresholds in scalar registers, so the searches
    // below run as scalar loops instead of exec-masked vector code
    b_loc = __builtin_amdgcn_readfirstlane(b_loc);
    w = __builtin_amdgcn_readfirstlane(w);
    const int base = w * NPT * kWave;
    uint32_t key[NPT];
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
        const int c = base + i * kWave + lane;
        key[i] = c > b_loc ? 0u : (c == b_loc ? 0xFFFFFFFFu : order_key(raw[i]));
    }
    const int n = wave_candidates<NPT>(b_loc, w);
    auto idx_of = [&](int i) { return base + i * kWave + lane; };
    auto page_of = [&](int i) { return page[i]; };
    if constexpr (W == 1) {
        select_wave<NPT>(key, idx_of, page_of, n, lane, &sh->ws[0], out);
    } else {
        select_wave<NPT>(key, idx_of, page_of, n, lane, &sh->ws[w],
                         [&](int pos, uint32_t k, int b, int pg) {
                             Cand c;
                             c.key = k;
                             c.idx = b;
                             c.page = pg;
                             c.pad = 0;
                             sh->win[w][pos] = c;
                         });
        __syncthreads();
        if (w == 0) {
            constexpr int N2 = (W * kTopK + kWave - 1) / kWave;
            uint32_t key2[N2];
            int idx2[N2], page2[N2];
#pragma unroll
            for (int i = 0; i < N2; ++i) {
                const int pos = i * kWave + lane;
                Cand c;
                c.key = 0u;
                c.idx = -1;
                c.page = -1;
                if (pos < W * kTopK) c = sh->win[pos / kTopK][pos % kTopK];
                key2[i] = c.key;
                idx2[i] = c.idx;
                page2[i] = c.page;
            }
            int n2 = 0;
#pragma unroll
            for (int v = 0; v < W; ++v) {
                const int nv = wave_candidates<NPT>(b_loc, v);
                n2 += nv < kTopK ? nv : kTopK;
            }
            select_wave<N2>(key2, [&](int i) { return idx2[i]; }, [&](int i) { return page2[i]; },
                            n2, lane, &sh->ws[0], out);
        }
    }
}

}  // namespace msa
