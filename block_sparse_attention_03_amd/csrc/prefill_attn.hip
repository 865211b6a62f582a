// prefill_attn.hip -- MSA sparse prefill attention, KV-block-major.
//
// What it computes (aivizor serving-report news item, KV-Block-Major
// paragraph; mechatronicstore "MoE de 428B" page, section on what makes M3
// different): the outer loop runs over KV blocks, each read from HBM once and
// contiguously; the inner loop runs over the queries that selected the block,
// producing partial outputs; a final Log-Sum-Exp reduction recomposes each
// query's result.  The result equals softmax attention over the union of the
// query's selected blocks, cut at its position.
//
// Steps (all on the caller's stream):
//   1. inverse map: histogram of (sequence, group, block) buckets over the
//      selection, exclusive scan (which also lists the nonempty buckets),
//      placement of (query, slot) entries;
//   2. block-major attention: one workgroup per nonempty bucket stages the block's K
//      and V (direct-to-LDS loads, 16-byte chunks swizzled by token) in LDS
//      once, two workgroups to a compute unit, then its wavefronts sweep
//      the bucket's (query, head) rows 32 at a time with 32x32x16 bf16 matrix
//      cores: S^T = K Q^T, row softmax in registers, P rounded to bf16 and
//      fed straight from the S^T accumulators as the B operand of
//      O^T = V^T P^T, whose V^T operand comes from LDS transpose reads.  The
//      next row tile's query gathers are issued before the current tile's
//      softmax, hiding their latency.  Each (query, head, slot) gets a normalised bf16 partial
//      output and an fp32 log-sum-exp, stored in bucket order (a tile's 32 rows
//      are consecutive: contiguous streaming stores, where rows placed by query
//      would scatter 256-byte pieces), and the inverse map records where each
//      selection's partials went;
//      Buckets of at most 32 (query, head) rows -- a few queries per sequence,
//      as in multi-query decode -- go to a lighter kernel instead: 256
//      threads, each wavefront's 32 tokens of K held as 16x16x32 A operands,
//      V in a swizzled unpadded LDS tile, the rows 16 at a time, so that four
//      workgroups share a compute unit and the page loads overlap;
//   3. merge: per (query, head), the partials of its selected slots, found
//      through the map's record, combine in slot order (deterministic; no
//      float atomics).
#include <algorithm>

#include "decode_tile.hpp"
#include "msa_common.hpp"
#include "select.hpp"

namespace msa {
namespace {

// Buckets of at most this many (query, head) rows take the small-bucket kernel.
constexpr int kSmallRows = 32;

// Inverse-map tiles: the selections of one KV group over kTileTokens
// consecutive query tokens of one sequence.
constexpr int kTileTokens = 256;  // 264 tiles on the 8k chunk with 8 groups: fill 10.7 us, against
                                  // 14.3 with 512-token tiles (136 workgroups on 256 CUs)
constexpr int kMapThreads = 256;
constexpr int kMapBatch = 16;  // selections each map thread loads at once

// Upper bound on the number of tiles (sum over sequences of ceil(nq / tile)
// is at most total_q / tile + B), times the KV groups.
__host__ __device__ inline int max_tiles(int total_q, int B, int Hkv) {
    return Hkv * (ceil_div(total_q, kTileTokens) + B);
}

struct PrefillWs {
    int32_t* counts;     // [NB] entries per (sequence, group, block) bucket
    int32_t* offsets;    // [NB + 1] exclusive scan of counts
    int32_t* buckets;    // [NB + 1]: [0] = buckets of more than kSmallRows rows, then their ids
    int32_t* small;      // [NB + 1]: [0] = nonempty buckets of at most kSmallRows rows, then ids
    int32_t* tile_base;  // [max_tiles, maxblk] a tile's first position within a bucket
    int32_t* entries;    // [total_q * Hkv * k]: query << 4 | slot, grouped by bucket
    int32_t* pos_of;     // [total_q, Hkv, k]: position in entries of selection (t, g, slot), -1 if none
    uint16_t* part_o;    // [total_q * Hq * k, 128] bf16 partial outputs: row e G + n = head n of
                         // the group for the entry at position e (inverse-map form), row
                         // (t Hq + h) k + slot (multi-query form)
    float* part_lse;     // [total_q * Hq * k]: their log-sum-exps, the same rows
    uint16_t* trash_o;   // [128] bf16: where padding rows' partial stores go
    float* trash_lse;    // [64]
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) / 256 * 256; }

__host__ __device__ inline PrefillWs prefill_ws(void* base, int B, int Hkv, int maxblk,
                                                int total_q, int Hq) {
    const size_t NB = (size_t)B * Hkv * maxblk;
    char* p = static_cast<char*>(base);
    PrefillWs w;
    w.counts = reinterpret_cast<int32_t*>(p);
    p += align256(NB * 4);
    w.offsets = reinterpret_cast<int32_t*>(p);
    p += align256((NB + 1) * 4);
    w.buckets = reinterpret_cast<int32_t*>(p);
    p += align256((NB + 1) * 4);
    w.small = reinterpret_cast<int32_t*>(p);
    p += align256((NB + 1) * 4);
    w.tile_base = reinterpret_cast<int32_t*>(p);
    p += align256((size_t)max_tiles(total_q, B, Hkv) * maxblk * 4);
    w.entries = reinterpret_cast<int32_t*>(p);
    p += align256((size_t)total_q * Hkv * kTopK * 4);
    w.pos_of = reinterpret_cast<int32_t*>(p);
    p += align256((size_t)total_q * Hkv * kTopK * 4);
    w.part_o = reinterpret_cast<uint16_t*>(p);
    p += align256((size_t)total_q * Hq * kTopK * kHeadDim * 2);
    w.part_lse = reinterpret_cast<float*>(p);
    p += align256((size_t)total_q * Hq * kTopK * 4);
    w.trash_o = reinterpret_cast<uint16_t*>(p);
    p += align256(kHeadDim * 2);
    w.trash_lse = reinterpret_cast<float*>(p);
    return w;
}

__host__ __device__ inline size_t prefill_ws_size(int B, int Hkv, int maxblk, int total_q, int Hq) {
    PrefillWs w = prefill_ws(nullptr, B, Hkv, maxblk, total_q, Hq);
    return reinterpret_cast<size_t>(w.trash_lse) + align256(kWave * 4);
}

__global__ void zero_kernel(int32_t* a, int na) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < na; i += gridDim.x * blockDim.x) a[i] = 0;
}

struct MapTile {
    int s, g, t0, t1;  // sequence, KV group, query tokens [t0, t1); s < 0: no such tile
};

// Tile `tile` = (group tile % Hkv, k-th (sequence, token chunk) pair in
// sequence order, k = tile / Hkv).  Wavefront 0 finds the pair -- lanes count
// the chunks of 64 sequences at a time and a prefix over lanes locates k -- and
// publishes it through sh; every thread must call it (one barrier).
__device__ MapTile find_map_tile(const int32_t* __restrict__ cu_q, int B, int Hkv, int tile,
                                 int* sh) {
    if (threadIdx.x < kWave) {
        const int lane = threadIdx.x;
        int k = tile / Hkv;
        int found = -1, chunk = 0;
        for (int base = 0; base < B && found < 0; base += kWave) {
            const int i = base + lane;
            const int nq = i < B ? cu_q[i + 1] - cu_q[i] : 0;
            const int n = ceil_div(nq, kTileTokens);
            int incl = n;  // inclusive prefix of chunk counts over lanes
#pragma unroll
            for (int d = 1; d < kWave; d <<= 1) {
                const int v = __shfl_up(incl, d, kWave);
                if (lane >= d) incl += v;
            }
            const uint64_t hit = __ballot(incl > k);
            if (hit) {
                const int l = __ffsll((unsigned long long)hit) - 1;
                found = base + l;
                chunk = k - (__shfl(incl, l, kWave) - __shfl(n, l, kWave));
            } else {
                k -= __shfl(incl, kWave - 1, kWave);
            }
        }
        if (lane == 0) {
            sh[0] = found;
            sh[1] = chunk;
        }
    }
    __syncthreads();
    MapTile m;
    m.s = sh[0];
    m.g = tile % Hkv;
    m.t0 = m.t1 = 0;
    if (m.s >= 0) {
        m.t0 = cu_q[m.s] + sh[1] * kTileTokens;
        m.t1 = min(cu_q[m.s + 1], m.t0 + kTileTokens);
    }
    return m;
}

// Pass 1: a tile counts its selections per block in LDS, then adds each
// nonzero count to the bucket's global count with one atomic; the value that
// atomic returns is the tile's first position within the bucket.  Block
// indices outside [0, maxblk) are not selections.
__global__ __launch_bounds__(kMapThreads)
void bucket_count_kernel(const int32_t* __restrict__ sel, const int32_t* __restrict__ cu_q,
                         int32_t* __restrict__ counts, int32_t* __restrict__ tile_base, int B,
                         int Hkv, int maxblk) {
    extern __shared__ int32_t hist[];  // [maxblk]
    __shared__ int sh[2];
    for (int b = threadIdx.x; b < maxblk; b += kMapThreads) hist[b] = 0;
    const MapTile m = find_map_tile(cu_q, B, Hkv, blockIdx.x, sh);  // contains a barrier
    if (m.s < 0) return;  // uniform
    const int n = (m.t1 - m.t0) * kTopK;
    // kMapBatch selections per thread loaded together, then counted
    for (int e0 = threadIdx.x; e0 < n; e0 += kMapThreads * kMapBatch) {
        int bv[kMapBatch];
#pragma unroll
        for (int u = 0; u < kMapBatch; ++u) {
            const int e = e0 + kMapThreads * u;
            bv[u] = e < n ? sel[((size_t)(m.t0 + e / kTopK) * Hkv + m.g) * kTopK + e % kTopK] : -1;
        }
#pragma unroll
        for (int u = 0; u < kMapBatch; ++u)
            if (bv[u] >= 0 && bv[u] < maxblk) atomicAdd(&hist[bv[u]], 1);
    }
    __syncthreads();
    const size_t bucket0 = ((size_t)m.s * Hkv + m.g) * maxblk;
    for (int b = threadIdx.x; b < maxblk; b += kMapThreads) {
        const int c = hist[b];
        if (c > 0) tile_base[(size_t)blockIdx.x * maxblk + b] = atomicAdd(&counts[bucket0 + b], c);
    }
}

// Inclusive prefix sum of v over the lanes of the wavefront.
__device__ __forceinline__ int wave_inclusive_sum(int v) {
    const int lane = __lane_id();
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int u = __shfl_up(v, off, kWave);
        if (lane >= off) v += u;
    }
    return v;
}

// Exclusive scan of counts[0..n) into offsets[0..n], one workgroup; it also
// lists the nonempty buckets in order, those of more than small_cnt entries in
// buckets and the others in small ([0] = how many, then their ids), so each
// attention kernel launches only as many workgroups as there can be buckets
// and none walks an empty one.  The counts go through in tiles of 8192: each
// thread takes 8 consecutive buckets (two 16-byte loads), wavefront prefix
// sums by lane shuffles, one LDS exchange of the 16 wavefront totals, and a
// running carry from tile to tile.
__global__ __launch_bounds__(1024)
void scan_kernel(const int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                 int32_t* __restrict__ buckets, int32_t* __restrict__ small, int n,
                 int small_cnt) {
    constexpr int kPer = 8;
    constexpr int kScanWaves = 1024 / kWave;
    __shared__ int wsum[3][kScanWaves];
    __shared__ int carry[3];
    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = tid / kWave;
    if (tid < 3) carry[tid] = 0;
    for (int t0 = 0; t0 < n; t0 += 1024 * kPer) {
        const int a = t0 + tid * kPer;
        int c[kPer];
        if (a + kPer <= n) {  // counts is 256-byte aligned and a is a multiple of 8
            const u32x4 v0 = *reinterpret_cast<const u32x4*>(counts + a);
            const u32x4 v1 = *reinterpret_cast<const u32x4*>(counts + a + 4);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                c[u] = (int)v0[u];
                c[4 + u] = (int)v1[u];
            }
        } else {
#pragma unroll
            for (int u = 0; u < kPer; ++u) c[u] = (a + u < n) ? counts[a + u] : 0;
        }
        int sum = 0, nl = 0, ns = 0;
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            sum += c[u];
            nl += c[u] > small_cnt;
            ns += c[u] > 0 && c[u] <= small_cnt;
        }
        const int isum = wave_inclusive_sum(sum);
        const int inl = wave_inclusive_sum(nl);
        const int ins = wave_inclusive_sum(ns);
        if (lane == kWave - 1) {
            wsum[0][wave] = isum;
            wsum[1][wave] = inl;
            wsum[2][wave] = ins;
        }
        __syncthreads();  // wavefront totals and the carry are visible
        int run = carry[0] + isum - sum;  // exclusive prefixes of this thread's buckets
        int runl = carry[1] + inl - nl;
        int runs = carry[2] + ins - ns;
        for (int k = 0; k < wave; ++k) {
            run += wsum[0][k];
            runl += wsum[1][k];
            runs += wsum[2][k];
        }
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            if (a + u < n) {
                offsets[a + u] = run;
                run += c[u];
                if (c[u] > small_cnt)
                    buckets[1 + runl++] = a + u;
                else if (c[u] > 0)
                    small[1 + runs++] = a + u;
            }
        }
        __syncthreads();  // every thread has read wsum and carry
        if (tid == 1023) {  // the last thread ends at the running totals
            carry[0] = run;
            carry[1] = runl;
            carry[2] = runs;
        }
    }
    __syncthreads();
    if (tid == 0) {
        offsets[n] = carry[0];
        buckets[0] = carry[1];
        small[0] = carry[2];
    }
}

// Small inverse map: the whole map (count, scan, bucket lists, placement)
// in one 1024-thread workgroup with the bucket counts in LDS, for a few
// queries per sequence (multi-query decode), where the four-kernel form is
// dominated by launch latency.  Counts, then offsets, are 16-bit halves of
// LDS words (at most kSmallMapSel selections); ranks within a bucket come
// from the LDS atomics.  Only the nonempty buckets' counts and offsets are
// written to the workspace: they are the only ones the attention kernels
// read.  A single workgroup pays every memory latency in full, so each
// thread loads its selections once, all together, and scans a run of
// buckets that is a whole number of 16-byte LDS chunks (no word shared with
// another thread, so the offsets go back with plain stores).
constexpr int kSmallMapBuckets = 49152;
constexpr int kSmallMapSel = 16384;
constexpr int kSmallMapThreads = 1024;
constexpr int kSmallSelPer = kSmallMapSel / kSmallMapThreads;              // selections per thread
constexpr int kSmallChunks = kSmallMapBuckets / kSmallMapThreads / 8;      // 16-byte chunks per thread

__global__ __launch_bounds__(kSmallMapThreads)
void inverse_map_small_kernel(const int32_t* __restrict__ sel, const int32_t* __restrict__ cu_q,
                              PrefillWs w, int total_q, int B, int Hkv, int maxblk,
                              int small_cnt) {
    __shared__ __attribute__((aligned(16))) uint32_t cnt2[kSmallMapBuckets / 2];  // two 16-bit counts (later offsets) per word
    __shared__ uint16_t rank[kSmallMapSel];
    __shared__ int seq_of[kSmallMapSel / kTopK];      // query token -> sequence
    __shared__ int wsum[3][kSmallMapThreads / kWave];
    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = tid / kWave;
    const int NB = B * Hkv * maxblk;
    const int n_sel = total_q * Hkv * kTopK;
    if (n_sel <= 0) return;  // uniform

    // this thread's selections e = tid + 1024 k, loaded together (clamped
    // indices keep every load in bounds; the copies past n_sel are unused)
    int selv[kSmallSelPer];
#pragma unroll
    for (int k = 0; k < kSmallSelPer; ++k)
        selv[k] = sel[min(tid + kSmallMapThreads * k, n_sel - 1)];
    // buckets [a, a + per) of this thread: per is a multiple of 8
    const int per = (ceil_div(NB, kSmallMapThreads) + 7) & ~7;  // <= 48
    const int a = tid * per;
    u32x4* cnt4 = reinterpret_cast<u32x4*>(cnt2);
#pragma unroll
    for (int c = 0; c < kSmallChunks; ++c)
        if (8 * c < per) cnt4[a / 8 + c] = u32x4{0u, 0u, 0u, 0u};
    for (int sq = tid; sq < B; sq += kSmallMapThreads)
        for (int t = cu_q[sq]; t < cu_q[sq + 1]; ++t) seq_of[t] = sq;
    __syncthreads();

    // count: each selection's rank in its bucket
    auto bucket_of = [&](int e, int b) {
        const int t = e / (Hkv * kTopK);
        const int g = (e / kTopK) % Hkv;
        return (seq_of[t] * Hkv + g) * maxblk + b;
    };
#pragma unroll
    for (int k = 0; k < kSmallSelPer; ++k) {
        const int e = tid + kSmallMapThreads * k;
        const int b = selv[k];
        if (e < n_sel && b >= 0 && b < maxblk) {
            const int bk = bucket_of(e, b);
            const int sh = 16 * (bk & 1);
            const uint32_t old = atomicAdd(&cnt2[bk >> 1], 1u << sh);
            rank[e] = (uint16_t)((old >> sh) & 0xFFFFu);
        }
    }
    __syncthreads();

    // scan: this thread's counts in registers (16-byte LDS reads), totals,
    // wavefront prefix sums, then the 16 wavefront totals through LDS
    uint32_t cw[4 * kSmallChunks];
#pragma unroll
    for (int c = 0; c < kSmallChunks; ++c) {
        const u32x4 v = (8 * c < per) ? cnt4[a / 8 + c] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int x = 0; x < 4; ++x) cw[4 * c + x] = v[x];
    }
    auto cnt_of = [&](int j) { return (int)((cw[j >> 1] >> (16 * (j & 1))) & 0xFFFFu); };
    int sum = 0, nl = 0, ns = 0;
#pragma unroll
    for (int j = 0; j < 8 * kSmallChunks; ++j) {
        const int c = cnt_of(j);  // zero past per and past NB
        sum += c;
        nl += c > small_cnt;
        ns += c > 0 && c <= small_cnt;
    }
    int isum = sum, inl = nl, ins = ns;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int u0 = __shfl_up(isum, off, kWave), u1 = __shfl_up(inl, off, kWave),
                  u2 = __shfl_up(ins, off, kWave);
        if (lane >= off) {
            isum += u0;
            inl += u1;
            ins += u2;
        }
    }
    if (lane == kWave - 1) {
        wsum[0][wave] = isum;
        wsum[1][wave] = inl;
        wsum[2][wave] = ins;
    }
    __syncthreads();
    int run = isum - sum, runl = inl - nl, runs = ins - ns;
    for (int k = 0; k < wave; ++k) {
        run += wsum[0][k];
        runl += wsum[1][k];
        runs += wsum[2][k];
    }
    // nonempty buckets -> workspace; counts -> exclusive offsets, word by
    // word in the same registers, then back to LDS
    auto emit = [&](int i, int c) {
        if (c > 0) {
            w.counts[i] = c;
            w.offsets[i] = run;
            if (c > small_cnt)
                w.buckets[1 + runl++] = i;
            else
                w.small[1 + runs++] = i;
        }
        const int o = run;
        run += c;
        return (uint32_t)o;
    };
#pragma unroll 2
    for (int x = 0; x < 4 * kSmallChunks; ++x) {
        const uint32_t o0 = emit(a + 2 * x, (int)(cw[x] & 0xFFFFu));
        const uint32_t o1 = emit(a + 2 * x + 1, (int)(cw[x] >> 16));
        cw[x] = o0 | (o1 << 16);
    }
#pragma unroll
    for (int c = 0; c < kSmallChunks; ++c)
        if (8 * c < per) cnt4[a / 8 + c] = u32x4{cw[4 * c], cw[4 * c + 1], cw[4 * c + 2], cw[4 * c + 3]};
    if (tid == kSmallMapThreads - 1) {
        w.buckets[0] = runl;
        w.small[0] = runs;
    }
    __syncthreads();

    // place: entries[offset + rank] = query << 4 | slot, and the position
    // (or -1) in pos_of
    auto off_at = [&](int i) { return (int)((cnt2[i >> 1] >> (16 * (i & 1))) & 0xFFFFu); };
#pragma unroll
    for (int k = 0; k < kSmallSelPer; ++k) {
        const int e = tid + kSmallMapThreads * k;
        const int b = selv[k];
        if (e < n_sel) {
            int pos = -1;
            if (b >= 0 && b < maxblk) {
                pos = off_at(bucket_of(e, b)) + rank[e];
                w.entries[pos] = ((e / (Hkv * kTopK)) << 4) | (e % kTopK);
            }
            w.pos_of[e] = pos;
        }
    }
}

// Pass 3: the tile places each selection at offsets[bucket] + its tile's base
// in the bucket + its rank among the tile's selections of that block (LDS
// counters; entries within a bucket are in no particular order), and records
// that position, or -1 for a slot that selects nothing, in pos_of.
__global__ __launch_bounds__(kMapThreads)
void bucket_fill_kernel(const int32_t* __restrict__ sel, const int32_t* __restrict__ cu_q,
                        const int32_t* __restrict__ offsets, const int32_t* __restrict__ tile_base,
                        int32_t* __restrict__ entries, int32_t* __restrict__ pos_of, int B, int Hkv,
                        int maxblk) {
    extern __shared__ int32_t cur[];  // [maxblk]
    __shared__ int sh[2];
    for (int b = threadIdx.x; b < maxblk; b += kMapThreads) cur[b] = 0;
    const MapTile m = find_map_tile(cu_q, B, Hkv, blockIdx.x, sh);  // contains a barrier
    if (m.s < 0) return;  // uniform
    const int n = (m.t1 - m.t0) * kTopK;
    const size_t bucket0 = ((size_t)m.s * Hkv + m.g) * maxblk;
    // kMapBatch selections per thread: their blocks, then their buckets'
    // bases, each round of loads issued together
    for (int e0 = threadIdx.x; e0 < n; e0 += kMapThreads * kMapBatch) {
        int bv[kMapBatch], base[kMapBatch];
#pragma unroll
        for (int u = 0; u < kMapBatch; ++u) {
            const int e = e0 + kMapThreads * u;
            const int b = e < n ? sel[((size_t)(m.t0 + e / kTopK) * Hkv + m.g) * kTopK + e % kTopK] : -1;
            bv[u] = (b >= 0 && b < maxblk) ? b : -1;
        }
#pragma unroll
        for (int u = 0; u < kMapBatch; ++u)
            base[u] = bv[u] >= 0 ? offsets[bucket0 + bv[u]] + tile_base[(size_t)blockIdx.x * maxblk + bv[u]] : 0;
#pragma unroll
        for (int u = 0; u < kMapBatch; ++u) {
            const int e = e0 + kMapThreads * u;
            if (e < n) {
                const int t = m.t0 + e / kTopK;
                int pos = -1;
                if (bv[u] >= 0) {
                    pos = base[u] + atomicAdd(&cur[bv[u]], 1);
                    entries[pos] = (t << 4) | (e % kTopK);
                }
                pos_of[((size_t)t * Hkv + m.g) * kTopK + e % kTopK] = pos;
            }
        }
    }
}

// Block-major attention: 256-thread workgroups that fit two to a compute
// unit (K and V unpadded in LDS with swizzled 16-byte chunks, 64 KB, plus a
// 16 KB output staging tile), so that one workgroup's block staging and last
// tiles overlap the other's products.
constexpr int kPfThreads = 256;
__device__ __forceinline__ int bk_off(int t, int d) {  // bf16 offset of K (token t, dim d)
    return t * kHeadDim + ((((d >> 3) ^ (t & 15))) << 3) + (d & 7);
}

__global__ __launch_bounds__(kPfThreads, 2)
void block_major_kernel(const uint16_t* __restrict__ q,        // [T, Hq, 128]
                        const uint16_t* __restrict__ k_cache,  // [P, Hkv, 128, 128]
                        const uint16_t* __restrict__ v_cache,
                        const int32_t* __restrict__ block_table,
                        const int32_t* __restrict__ seq_lens,
                        const int32_t* __restrict__ cu_q, PrefillWs w, int Hq, int Hkv,
                        int maxblk, float scale_log2) {
    // K and V unpadded (32 KB each), 16-byte chunks swizzled by token (K:
    // bk_off, V: vs_off); per wavefront a 32-row x 64-dim output staging tile
    __shared__ __attribute__((aligned(16))) uint16_t ks[kBlock * kHeadDim];
    __shared__ __attribute__((aligned(16))) uint16_t vs[kBlock * kHeadDim];
    __shared__ __attribute__((aligned(16))) uint16_t stg[(kPfThreads / kWave) * 32 * 64];

    // Workgroups reach the 8 XCDs round-robin by index: XCD x takes list
    // entries x per .. x per + per - 1, a contiguous run of the (sequence,
    // group, block)-ordered list, so each XCD's L2 serves the query rows of
    // about one eighth of the (sequence, group)s instead of all of them
    // (8k chunk: attention call 0.948 -> 0.934 ms; with streaming query
    // loads, which skip the caches, it takes 1.68 ms).  The grid is a
    // multiple of 8 that covers every entry.
    const int nbk = w.buckets[0];
    const int per = (nbk + 7) / 8;
    const int jj = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
    if (jj >= nbk) return;  // uniform
    const int bk = w.buckets[1 + jj];
    const int cnt = w.counts[bk];
    const int base = w.offsets[bk];
    const int b = bk % maxblk;
    const int g = (bk / maxblk) % Hkv;
    const int s = bk / (maxblk * Hkv);
    const int G = Hq / Hkv;
    const int L = seq_lens[s];
    const int nq = cu_q[s + 1] - cu_q[s];
    const int pos0 = L - nq - cu_q[s];  // p = pos0 + t
    const int nv = min(kBlock, L - b * kBlock);
    const int page = block_table[(size_t)s * maxblk + b];
    const size_t page_off = ((size_t)page * Hkv + g) * kBlock * kHeadDim;
    const uint16_t* kp = k_cache + page_off;
    const uint16_t* vp = v_cache + page_off;
    const int tid = threadIdx.x;

    // Stage the block once with direct-to-LDS loads: wavefront w's eight
    // loads of each fill 16-byte chunks 512w .. 512w + 511 (tokens 32w ..
    // 32w + 31); lane l of load j fills chunk position l % 16 of token
    // (512w + 64j + l) / 16 and so reads that token's global chunk
    // (l % 16) ^ swizzle.  The page is allocated in full; V rows past the
    // sequence end are zeroed after the loads (P is 0 there, and 0 x a
    // non-finite value must not reach the sum), K rows there are cut by the
    // causal mask.
    {
        const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
        const int ln = tid % kWave;
#pragma unroll
        for (int jl = 0; jl < 8; ++jl) {
            const int chunk0 = (wv * 8 + jl) * kWave;
            const int tok = (chunk0 + ln) / 16, pos = ln % 16;
            __builtin_amdgcn_global_load_lds(kp + tok * kHeadDim + 8 * (pos ^ (tok & 15)),
                                             (__attribute__((address_space(3))) void*)(ks + chunk0 * 8),
                                             16, 0, 0);
            __builtin_amdgcn_global_load_lds(vp + tok * kHeadDim + 8 * (pos ^ ((tok & 7) << 1)),
                                             (__attribute__((address_space(3))) void*)(vs + chunk0 * 8),
                                             16, 0, 0);
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt 0: this wavefront's chunks are in LDS
        __syncthreads();
        if (nv < kBlock) {  // uniform: the sequence's partial last block
            for (int c = tid; c < (kBlock - nv) * (kHeadDim / 8); c += kPfThreads)
                *reinterpret_cast<u32x4*>(vs + (nv + c / 16) * kHeadDim + 8 * (c % 16)) =
                    u32x4{0u, 0u, 0u, 0u};
            __syncthreads();
        }
    }
    // wave-uniform to the compiler too, so the tile loop's exits are scalar
    // branches and its load waits stay exact across iterations
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int lane = tid % kWave;
    const int n = lane % 32;   // result column = row of this lane
    const int h = lane / 32;   // lane half
    const int nrows = cnt * G;
    const int tok0 = b * kBlock;
    constexpr int kWaves = kPfThreads / kWave;

    // Row n of a tile: its (query << 4 | slot) entry -- fetched two tiles
    // ahead -- and from it the query and head.  Rows past the bucket repeat
    // its last row (real data; results discarded).
    auto entry_of = [&](int tile) { return w.entries[base + min(tile * 32 + n, nrows - 1) / G]; };
    auto row_info = [&](int tile, int entry, int* t_out, int* head_out) {
        const int rho0 = tile * 32 + n;
        const int rho = rho0 < nrows ? rho0 : nrows - 1;
        *t_out = entry >> 4;
        *head_out = g * G + rho % G;
        return rho0 < nrows;
    };
    // Direct gather of a tile's query rows into B operands: lane (n, h) loads
    // dims 64h + 8i .. +7 of its row n for k-step i.
    auto gather_q = [&](int t_n, int head_n, u32x4* raw) {
        const uint16_t* qrow = q + ((size_t)t_n * Hq + head_n) * kHeadDim + 64 * h;
#pragma unroll
        for (int i = 0; i < 8; ++i) raw[i] = ld16(qrow + 8 * i);
    };

    // Every iteration issues the same memory operations -- the next tile's
    // query rows and the entries two tiles ahead, clamped to the bucket's
    // last row past its end, and partial stores that padding rows send to a
    // trash row -- so that each wait covers exactly the loads it needs and
    // never the previous tile's stores.
    int tile = wave;
    if (tile * 32 >= nrows) return;  // wavefront-uniform; no workgroup barrier follows
    // Query rows are gathered two tiles ahead into two register buffers used
    // in turn, so that while a tile computes the gathers of this wavefront's
    // next two tiles are in flight (the kernel's rate is set by the bytes it
    // keeps in flight).
    int tA = 0, hA = 0, tB = 0, hB = 0;
    bool okA = row_info(tile, entry_of(tile), &tA, &hA);
    bool okB = row_info(tile + kWaves, entry_of(tile + kWaves), &tB, &hB);
    int entry_next = entry_of(tile + 2 * kWaves);
    u32x4 qA[8], qB[8];
    gather_q(tA, hA, qA);
    gather_q(tB, hB, qB);
    // wait for the first two tiles' loads here, so that at the loop head
    // neither path has its query rows in flight and no wait there reaches the
    // previous tile's stores (s_waitcnt immediate: vmcnt 0, other counters
    // unconstrained)
    __builtin_amdgcn_s_waitcnt(0x0F70);

    auto step = [&](u32x4 (&qraw)[8], int& t, int& head, bool& row_ok) {
        // B operands (k-step i of lane half h: dims 64h + 8i .. +7)
        bf16x8 qb[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) qb[i] = as_bf16x8(qraw[i]);
        const int cur_t = t;
        const bool cur_ok = row_ok;
        // The rows two tiles ahead go into this buffer once this tile's
        // S^T products have read it (so the old and new rows never share
        // the registers' lifetime).  The entry of the tile after those is
        // loaded first: the next step needs it before its own gather, and
        // waits count loads in issue order.
        const int ahead = tile + 2 * kWaves;
        const int entry_after = entry_of(ahead + kWaves);

        // S^T = K Q^T: tile mt = tokens 32mt..32mt+31; value v of the lane is
        // token 32mt + 8(v/4) + 4h + v%4 of row n.  Operands of token tile
        // mt+1 are read while tile mt multiplies.
        f32x16 sacc[4];
        u32x4 ka[2][8];
#pragma unroll
        for (int i = 0; i < 8; ++i) ka[0][i] = *reinterpret_cast<const u32x4*>(ks + bk_off(n, 64 * h + 8 * i));
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            if (mt < 3) {
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    ka[(mt + 1) & 1][i] =
                        *reinterpret_cast<const u32x4*>(ks + bk_off(32 * (mt + 1) + n, 64 * h + 8 * i));
            }
            sacc[mt] = mfma32(as_bf16x8(ka[mt & 1][0]), qb[0], f32x16{});
#pragma unroll
            for (int i = 1; i < 8; ++i) sacc[mt] = mfma32(as_bf16x8(ka[mt & 1][i]), qb[i], sacc[mt]);
            // keep the scheduler from hoisting further tiles' operand reads
            __builtin_amdgcn_sched_barrier(0);
        }
        row_ok = row_info(ahead, entry_next, &t, &head);
        gather_q(t, head, qraw);
        entry_next = entry_after;

        // causal cut inside the query's own block
        const int lim = pos0 + cur_t - tok0;  // token index (within block) must be <= lim
        if (__ballot(lim < kBlock - 1)) {  // only tiles holding a row of this block's own queries
            // the lane's token is 32mt + 8(v/4) + 4h + v%4: compare the
            // constant part against lim - 4h (no per-lane index registers)
            const int limh = lim - 4 * h;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    if (32 * mt + 8 * (v / 4) + (v % 4) > limh) sacc[mt][v] = -__builtin_inff();
        }
        float mx = -__builtin_inff();
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[mt][v]);
        mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
        const float mscaled = mx * scale_log2;

        // P first (the S^T registers die as P is built), then O^T = V^T P^T.
        // k-step i covers tokens 16i..16i+15: the B operand is accumulator
        // values 8(i%2)..8(i%2)+7 of S^T tile i/2 (tokens 16i + 4h + 0..3 and
        // 16i + 8 + 4h + 0..3) rounded to bf16; the row sum uses the rounded
        // weights the product uses.
        bf16x8 pb[8];
        float sum = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            u32x4 pw;
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                const float p0 = __builtin_amdgcn_exp2f(sacc[i / 2][8 * (i % 2) + 2 * e2] * scale_log2 - mscaled);
                const float p1 = __builtin_amdgcn_exp2f(sacc[i / 2][8 * (i % 2) + 2 * e2 + 1] * scale_log2 - mscaled);
                pw[e2] = pack2_bf16(p0, p1);
                sum += bf16_lo(pw[e2]) + bf16_hi(pw[e2]);
            }
            pb[i] = as_bf16x8(pw);
        }
        // A operand: the same tokens of dims 32mt + n, from transpose reads of
        // row-major V (lanes 16*(lane/16) .. +15 read dims 32mt +
        // 16*((lane/16)%2) .. +15); dim tile mt+1 is read while mt multiplies.
        f32x16 oacc[4];
        const int j = lane % 16;
        const int vt = 4 * h + j / 4;
        const int vd = 16 * ((lane / 16) % 2) + 4 * (j % 4);
        u32x2 va[2][16];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            va[0][2 * i] = lds_read_tr16(vs + vs_off(16 * i + vt, vd));
            va[0][2 * i + 1] = lds_read_tr16(vs + vs_off(16 * i + 8 + vt, vd));
        }
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            if (mt < 3) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    va[(mt + 1) & 1][2 * i] = lds_read_tr16(vs + vs_off(16 * i + vt, 32 * (mt + 1) + vd));
                    va[(mt + 1) & 1][2 * i + 1] = lds_read_tr16(vs + vs_off(16 * i + 8 + vt, 32 * (mt + 1) + vd));
                }
            }
            const u32x2* a = va[mt & 1];
            oacc[mt] = mfma32(as_bf16x8(u32x4{a[0][0], a[0][1], a[1][0], a[1][1]}), pb[0], f32x16{});
#pragma unroll
            for (int i = 1; i < 8; ++i)
                oacc[mt] = mfma32(as_bf16x8(u32x4{a[2 * i][0], a[2 * i][1], a[2 * i + 1][0], a[2 * i + 1][1]}),
                                  pb[i], oacc[mt]);
            __builtin_amdgcn_sched_barrier(0);
        }
        sum += __shfl_xor(sum, 32, kWave);

        // normalised partial output.  Row rho = tile 32 + n of the bucket is
        // partial row (base + rho / G) G + rho % G = base G + rho, so a tile's
        // 32 rows are consecutive; padding rows write a trash row (-1).  Each
        // half row (dims 64hf .. 64hf + 63) goes accumulators -> this wave's
        // staging tile (lane (n, h) holds dims 32mt + 8qd + 4h .. +3 of row n;
        // 16-byte chunk c of row r sits at position c ^ (r % 8)) -> streaming
        // 16-byte stores, 8 lanes per 128-byte line: stores of 8 bytes per
        // lane, or streaming stores of partial lines, cost far more.
        const float inv = 1.0f / sum;
        const int orow = cur_ok ? base * G + tile * 32 + n : -1;
        uint16_t* sbuf = stg + wave * 32 * 64;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
            for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
                for (int qd = 0; qd < 4; ++qd) {
                    const int mt = 2 * hf + m2;
                    const int c = 4 * m2 + qd;
                    *reinterpret_cast<u32x2*>(sbuf + n * 64 + 8 * (c ^ (n & 7)) + 4 * h) =
                        u32x2{pack2_bf16(oacc[mt][4 * qd + 0] * inv, oacc[mt][4 * qd + 1] * inv),
                              pack2_bf16(oacc[mt][4 * qd + 2] * inv, oacc[mt][4 * qd + 3] * inv)};
                }
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const int r = lane / 8 + 8 * it;
                const int c = lane % 8;
                const int o = __shfl(orow, r, kWave);
                const u32x4 v = *reinterpret_cast<const u32x4*>(sbuf + r * 64 + 8 * (c ^ (r & 7)));
                uint16_t* dst = (o >= 0) ? w.part_o + (size_t)o * kHeadDim : w.trash_o;
                __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dst + 64 * hf + 8 * c));
            }
            __builtin_amdgcn_wave_barrier();
        }
        float* ldst = (cur_ok && h == 0) ? w.part_lse + orow : w.trash_lse + lane;
        *ldst = mx * scale_log2 * kLn2 + __logf(sum);
        __builtin_amdgcn_wave_barrier();
        };
    // whole pairs of this wavefront's tiles, then an odd last one: a loop with
    // no exit between its two steps, so that each step's wait is exact
    const int mine = (ceil_div(nrows, 32) - wave + kWaves - 1) / kWaves;  // >= 1
    for (int pair = 0; pair < mine / 2; ++pair) {
        step(qA, tA, hA, okA);
        tile += kWaves;
        step(qB, tB, hB, okB);
        tile += kWaves;
    }
    if (mine & 1) step(qA, tA, hA, okA);
}

// Small buckets (at most kSmallRows (query, head) rows): one 256-thread
// workgroup per bucket.  Each wavefront holds its 32 tokens of K as 16x16x32
// A operands straight from HBM; V goes to the swizzled LDS tile; the rows go
// 16 at a time as B-operand columns: S^T = K Q^T, a per-row causal cut, the
// row max and sum across the four wavefronts through LDS, P (bf16) through
// LDS, O^T = V^T P^T with each wavefront owning 32 dims.  Partial outputs and
// log-sum-exps go where the block-major kernel puts them.
//
// A block is loaded (load_small: V rows, tokens at or past nv zero, then K
// rows; tokens past nv are read from the page's padding and masked to -inf
// later) and then attended (compute_small) against nrows rows: row rho is
// head g G + rho % G of the (query << 4 | slot) entry entry_at(rho / G), and
// its partial output and log-sum-exp go to row row_of(rho).
// Every thread of the workgroup calls both; compute_small starts by writing
// the V tile, so a caller that attends several blocks puts a barrier between
// calls.
struct SmallRaw {
    u32x4 v[8];
    u32x4 k[8];
};

__device__ __forceinline__ void load_small(const uint16_t* __restrict__ kp,
                                           const uint16_t* __restrict__ vp, int nv, SmallRaw& r) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const int tok = tid / 16 + 16 * it;
        r.v[it] = (tok < nv) ? ld16_stream(vp + tok * kHeadDim + 8 * (tid % 16)) : u32x4{0u, 0u, 0u, 0u};
    }
    load_k_rows(kp, tid / kWave, tid % kWave, r.k);
}

template <class EntryAt, class RowOf>
__device__ __forceinline__ void compute_small(DecodeShared& sh, const SmallRaw& r,
                                              const uint16_t* __restrict__ q, int nv, int pos0,
                                              int b, int g, int G, int Hq, int nrows,
                                              EntryAt entry_at, RowOf row_of, const PrefillWs& w,
                                              float scale_log2) {
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = tid % kWave;
    const int n = lane % 16;   // row (B / result column) or row of A
    const int kg = lane / 16;  // lane group

    // K -> A operands of this wavefront's tokens 32w + 16j + n, dims 32i + 8kg
    // (operand order through the V tile), then V -> LDS
    bf16x8 ka[2][4];
    k_rows_to_operands(r.k, wave, lane, sh.vs, ka);
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 8; ++it)
        *reinterpret_cast<u32x4*>(sh.vs + vs_off(tid / 16 + 16 * it, 8 * (tid % 16))) = r.v[it];

    for (int r0 = 0; r0 < nrows; r0 += 16) {
        // row n of this group: its query and head (rows past the bucket
        // repeat its last row; their results are discarded)
        const int rho0 = r0 + n;
        const bool row_ok = rho0 < nrows;
        const int rho = row_ok ? rho0 : nrows - 1;
        const int t = entry_at(rho / G) >> 4;
        const int head = g * G + rho % G;
        bf16x8 qb[4];
        const uint16_t* qrow = q + ((size_t)t * Hq + head) * kHeadDim;
#pragma unroll
        for (int i = 0; i < 4; ++i) qb[i] = as_bf16x8(ld16(qrow + 32 * i + 8 * kg));
        __syncthreads();  // V staged (first group) / the previous group's LDS reads done

        // S^T for tokens 32w + 16j + 4kg + rr of row n; a token is visible iff
        // it is in the cache (< nv) and at or before the row's position
        const int lim = min(nv - 1, pos0 + t - b * kBlock);
        f32x4 sacc[2];
        float mx = -__builtin_inff();
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            sacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < 4; ++i) sacc[j] = mfma16(ka[j][i], qb[i], sacc[j]);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int tok = 32 * wave + 16 * j + 4 * kg + rr;
                if (tok > lim) sacc[j][rr] = -__builtin_inff();
                mx = fmaxf(mx, sacc[j][rr]);
            }
        }
        mx = wave_max_xor(mx, 16);
        mx = wave_max_xor(mx, 32);
        if (kg == 0) sh.red_max[wave][n] = mx;
        __syncthreads();
        const float m = fmaxf(fmaxf(sh.red_max[0][n], sh.red_max[1][n]),
                              fmaxf(sh.red_max[2][n], sh.red_max[3][n]));
        // P rounded to bf16; the sum uses the rounded weights
        float sum = 0.f;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int tok = 32 * wave + 16 * j + 4 * kg;
            uint32_t pw[2];
#pragma unroll
            for (int e2 = 0; e2 < 2; ++e2) {
                const float p0 = __builtin_amdgcn_exp2f((sacc[j][2 * e2] - m) * scale_log2);
                const float p1 = __builtin_amdgcn_exp2f((sacc[j][2 * e2 + 1] - m) * scale_log2);
                pw[e2] = pack2_bf16(p0, p1);
                sum += bf16_lo(pw[e2]) + bf16_hi(pw[e2]);
            }
            *reinterpret_cast<u32x2*>(sh.pl + n * kPStride + tok) = u32x2{pw[0], pw[1]};
        }
        sum += __shfl_xor(sum, 16, kWave);
        sum += __shfl_xor(sum, 32, kWave);
        if (kg == 0) sh.red_sum[wave][n] = sum;
        __syncthreads();

        // O^T = V^T P^T for dims 32w .. 32w+31; k-step ks covers tokens
        // 32ks + 4kg + 0..3 and 32ks + 16 + 4kg + 0..3
        f32x4 oacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int ta = 32 * ks + 4 * kg;
            const u32x2 p0 = *reinterpret_cast<const u32x2*>(sh.pl + n * kPStride + ta);
            const u32x2 p1 = *reinterpret_cast<const u32x2*>(sh.pl + n * kPStride + ta + 16);
            const bf16x8 pbv = as_bf16x8(u32x4{p0[0], p0[1], p1[0], p1[1]});
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                const uint16_t* src = sh.vs + vs_off(ta + n / 4, 32 * wave + 16 * mt + 4 * (n % 4));
                const u32x2 v0a = lds_read_tr16(src);
                const u32x2 v1a = lds_read_tr16(src + 16 * kHeadDim);
                oacc[mt] = mfma16(as_bf16x8(u32x4{v0a[0], v0a[1], v1a[0], v1a[1]}), pbv, oacc[mt]);
            }
        }
        const float l = sh.red_sum[0][n] + sh.red_sum[1][n] + sh.red_sum[2][n] + sh.red_sum[3][n];
        if (row_ok) {
            const size_t prow = row_of(rho);
            const float inv = 1.0f / l;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                const int d = 32 * wave + 16 * mt + 4 * kg;
                *reinterpret_cast<u32x2*>(w.part_o + prow * kHeadDim + d) =
                    u32x2{pack2_bf16(oacc[mt][0] * inv, oacc[mt][1] * inv),
                          pack2_bf16(oacc[mt][2] * inv, oacc[mt][3] * inv)};
            }
            if (wave == 0 && kg == 0) w.part_lse[prow] = m * scale_log2 * kLn2 + __logf(l);
        }
    }
}

__global__ __launch_bounds__(kDecThreads)
void bucket_small_kernel(const uint16_t* __restrict__ q,        // [T, Hq, 128]
                         const uint16_t* __restrict__ k_cache,  // [P, Hkv, 128, 128]
                         const uint16_t* __restrict__ v_cache,
                         const int32_t* __restrict__ block_table,
                         const int32_t* __restrict__ seq_lens,
                         const int32_t* __restrict__ cu_q, PrefillWs w, int Hq, int Hkv,
                         int maxblk, float scale_log2) {
    __shared__ __attribute__((aligned(16))) DecodeShared sh;
    if ((int)blockIdx.x >= w.small[0]) return;  // uniform
    const int bk = w.small[1 + blockIdx.x];
    const int cnt = w.counts[bk];
    const int base = w.offsets[bk];
    const int b = bk % maxblk;
    const int g = (bk / maxblk) % Hkv;
    const int s = bk / (maxblk * Hkv);
    const int G = Hq / Hkv;
    const int L = seq_lens[s];
    const int nq = cu_q[s + 1] - cu_q[s];
    const int pos0 = L - nq - cu_q[s];  // p = pos0 + t
    const int nv = min(kBlock, L - b * kBlock);
    const int page = block_table[(size_t)s * maxblk + b];
    const size_t page_off = ((size_t)page * Hkv + g) * kBlock * kHeadDim;
    SmallRaw raw;
    load_small(k_cache + page_off, v_cache + page_off, nv, raw);
    compute_small(sh, raw, q, nv, pos0, b, g, G, Hq, cnt * G,
                  [&](int i) { return w.entries[base + i]; },
                  [&](int rho) { return (size_t)base * G + rho; }, w, scale_log2);
}

// Few queries per sequence (multi-query decode: a handful of draft tokens
// per sequence): the inverse map's work moves into the attention kernel.
// Workgroup (s Hkv + g, p) marks the blocks that the queries of sequence s
// select in group g in a bitmap (in the V tile), ranks them by block index,
// and attends each block whose rank is p modulo P once, for every entry that
// selected it, as the block-major kernels do: one launch where the general
// path needs the map's launches and two attention kernels.  The pages of a
// workgroup's blocks are looked up together, in one round trip.  (Loading a
// block's K and V during the previous block's products gains nothing: the
// query rows each pass loads wait behind those loads.)
// With SELECT (the multi-query step) the workgroup first makes the top-k
// selection of its queries itself from their block scores, one query per
// wavefront at a time, with the selection rule of msa_topk_blocks (NPT
// candidates per lane, one wavefront per row); stripe 0 publishes them in
// sel.  Without it the selection is read from sel.
constexpr int kMqEntries = 4096;                        // queries of a sequence x k, at most
// The kernel is compiled for 1,024 entries too, used when the call's entries
// fit: fewer registers and LDS (at 8 x 60k with 4 and 8 drafts, 65.2 and
// 103.2 us per step against 65.8 and 104.4 us).
constexpr int kMqSmallEntries = 1024;
constexpr int kMqMaxOwn = 128;                          // blocks per workgroup, at most
constexpr int kMqMaxWords = kBlock * kHeadDim / 2;      // bitmap words the V tile holds

// The multi-query form serves calls whose every sequence's entries fit
// (total_q x k <= kMqEntries) with at most 32 queries per sequence on
// average.  Past that, blocks are chosen by enough of a sequence's queries
// that the inverse map and the block-major kernel win: at 60k, one sequence
// with 128 or 256 new tokens took 187 and 332 us in this form against 180
// and 306 us, while 8 sequences with 16 or 32 drafts each took 149 and 211
// us against 167 and 235 us.
inline bool mq_form(const MsaShape& s, int total_q) {
    return (int64_t)total_q * kTopK <= kMqEntries && total_q <= 32 * s.B &&
           ceil_div(s.maxblk, 32) <= kMqMaxWords;
}

template <bool SELECT, int NPT, int CAP>
__global__ __launch_bounds__(kDecThreads)
void mq_block_kernel(const uint16_t* __restrict__ q,        // [T, Hq, 128]
                     const uint16_t* __restrict__ k_cache,  // [P, Hkv, 128, 128]
                     const uint16_t* __restrict__ v_cache,
                     const int32_t* __restrict__ block_table,
                     const int32_t* __restrict__ seq_lens,
                     const int32_t* __restrict__ cu_q,
                     int32_t* __restrict__ sel,             // [T, Hkv, k]: read, or written with SELECT
                     const float* __restrict__ scores,      // [T, Hkv, maxblk] (SELECT only)
                     PrefillWs w, int Hq, int Hkv, int maxblk, int P, float scale_log2) {
    __shared__ __attribute__((aligned(16))) DecodeShared sh;
    constexpr int kMqPerThread = CAP / kDecThreads;  // entries held per thread
    __shared__ int32_t rsel[SELECT ? CAP : 1];  // this (sequence, group)'s selections
    __shared__ uint16_t rows[CAP];  // entry indices of the current block's rows
    __shared__ int own[kMqMaxOwn];         // this workgroup's blocks, in rank order
    __shared__ int own_page[kMqMaxOwn];    // their physical pages
    __shared__ int wtot[kDecThreads / kWave];
    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = tid / kWave;
    const int s = blockIdx.x / Hkv;
    const int g = blockIdx.x % Hkv;
    const int p = blockIdx.y;
    const int G = Hq / Hkv;
    const int t0 = cu_q[s];
    const int nq = cu_q[s + 1] - t0;
    const int n_e = min(nq * kTopK, CAP);  // the host takes this kernel only when
                                                  // every sequence's entries fit
    const int L = seq_lens[s];
    const int pos0 = L - nq - t0;  // position of query token t: pos0 + t

    if constexpr (SELECT) {
        // query t0 + i of this (sequence, group) by wavefront i mod 4; the
        // selection scratch lives in the V tile, free until the bitmap
        static_assert(4 * sizeof(SelectShared<1>) <= sizeof(sh.vs), "selection scratch");
        SelectShared<1>* ssh = reinterpret_cast<SelectShared<1>*>(sh.vs) + wave;
        const int nq_sel = min(nq, CAP / kTopK);
        for (int i = wave; i < nq_sel; i += kDecThreads / kWave) {
            const int t = t0 + i;
            float raw[NPT];
            int pg[NPT];
            load_candidates<NPT, 1, false>(scores + ((size_t)t * Hkv + g) * maxblk, nullptr, maxblk,
                                           0, lane, raw, pg);
            select_row<NPT, 1>(raw, pg, (pos0 + t) / kBlock, 0, lane, ssh,
                               [&](int pos, uint32_t, int b, int) {
                                   rsel[i * kTopK + pos] = b;
                                   if (p == 0) sel[((size_t)t * Hkv + g) * kTopK + pos] = b;
                               });
            wave_sync_lds();  // this wavefront's scratch is reused by its next query
        }
        __syncthreads();  // rsel complete; the selection scratch is free
    }

    // entry e = q_local k + slot of this thread: tid + 256 i; its block, or -1
    int eb[kMqPerThread];
#pragma unroll
    for (int i = 0; i < kMqPerThread; ++i) {
        const int e = tid + kDecThreads * i;
        int b = -1;
        if (e < n_e)
            b = SELECT ? rsel[e] : sel[((size_t)(t0 + e / kTopK) * Hkv + g) * kTopK + e % kTopK];
        eb[i] = (b >= 0 && b < maxblk) ? b : -1;
    }
    uint32_t* bits = reinterpret_cast<uint32_t*>(sh.vs);
    const int nw = ceil_div(maxblk, 32);  // <= kMqMaxWords
    for (int i = tid; i < nw; i += kDecThreads) bits[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kMqPerThread; ++i)
        if (eb[i] >= 0) atomicOr(&bits[eb[i] >> 5], 1u << (eb[i] & 31));
    __syncthreads();

    // a marked block's rank = the marked blocks below it: thread tid counts
    // words [tid wpt, (tid + 1) wpt), then an exclusive prefix over threads
    const int wpt = ceil_div(nw, kDecThreads);
    int cnt = 0;
    for (int k = 0; k < wpt; ++k) {
        const int wi = tid * wpt + k;
        if (wi < nw) cnt += __popc(bits[wi]);
    }
    const int incl = wave_inclusive_sum(cnt);
    if (lane == kWave - 1) wtot[wave] = incl;
    __syncthreads();
    int run = incl - cnt;
    int n_marked = 0;
#pragma unroll
    for (int k = 0; k < kDecThreads / kWave; ++k) {
        if (k < wave) run += wtot[k];
        n_marked += wtot[k];
    }
    for (int k = 0; k < wpt; ++k) {
        const int wi = tid * wpt + k;
        uint32_t m = wi < nw ? bits[wi] : 0u;
        while (m) {
            const int bit = __builtin_ctz(m);
            m &= m - 1;
            if (run % P == p) own[run / P] = wi * 32 + bit;
            ++run;
        }
    }
    // ranks p, p + P, ... below n_marked (at most kMqMaxOwn: the host sizes P)
    const int n_own = __builtin_amdgcn_readfirstlane(n_marked > p ? (n_marked - p + P - 1) / P : 0);
    __syncthreads();  // own[] written; every bitmap word read (the V tile is free)

    if (tid < n_own) own_page[tid] = block_table[(size_t)s * maxblk + own[tid]];
    __syncthreads();

    auto nv_of = [&](int b) { return min(kBlock, L - b * kBlock); };
    auto load_own = [&](int j, SmallRaw& r) {
        const size_t page_off = ((size_t)own_page[j] * Hkv + g) * kBlock * kHeadDim;
        load_small(k_cache + page_off, v_cache + page_off, nv_of(own[j]), r);
    };
    auto attend_own = [&](int j, const SmallRaw& r) {
        const int b = __builtin_amdgcn_readfirstlane(own[j]);
        // this block's rows: the entries that selected it, compacted in LDS
        int mine = 0;
#pragma unroll
        for (int i = 0; i < kMqPerThread; ++i) mine += (eb[i] == b);
        const int incl_b = wave_inclusive_sum(mine);
        __syncthreads();  // the previous block's reads of rows, wtot and the tiles are done
        if (lane == kWave - 1) wtot[wave] = incl_b;
        __syncthreads();
        int at = incl_b - mine;
        int n_rows_b = 0;
#pragma unroll
        for (int k = 0; k < kDecThreads / kWave; ++k) {
            if (k < wave) at += wtot[k];
            n_rows_b += wtot[k];
        }
#pragma unroll
        for (int i = 0; i < kMqPerThread; ++i)
            if (eb[i] == b) rows[at++] = (uint16_t)(tid + kDecThreads * i);
        n_rows_b = __builtin_amdgcn_readfirstlane(n_rows_b);
        __syncthreads();  // rows visible
        // partials at row (t, head, slot): this form has no entry list, and
        // its merge reads them there
        compute_small(sh, r, q, nv_of(b), pos0, b, g, G, Hq, n_rows_b * G,
                      [&](int i) {
                          const int e = rows[i];
                          return ((t0 + e / kTopK) << 4) | (e % kTopK);
                      },
                      [&](int rho) {
                          const int e = rows[rho / G];
                          return ((size_t)(t0 + e / kTopK) * Hq + g * G + rho % G) * kTopK + e % kTopK;
                      },
                      w, scale_log2);
    };
    for (int j = 0; j < n_own; ++j) {
        SmallRaw raw;
        load_own(j, raw);
        attend_own(j, raw);
    }
}

// 16 threads per (query, head), 8 dims each: merge the selected slots'
// partials.  Slot i's partial is at row pos_of[(t Hkv + g) k + i] G + n
// (pos_of -1: no selection), or, with DIRECT (the multi-query form, which
// has no entry list), at row (t Hq + h) k + i when sel names a block there.
template <bool DIRECT>
__global__ __launch_bounds__(256)
void prefill_merge_kernel(const int32_t* __restrict__ sel, PrefillWs w,
                          uint16_t* __restrict__ out, float* __restrict__ lse_out, int total_q,
                          int Hq, int Hkv, int maxblk) {
    const int idx = blockIdx.x * 256 + threadIdx.x;
    const int th = idx / 16;  // t * Hq + h
    const int part = idx % 16;
    if (th >= total_q * Hq) return;
    const int t = th / Hq;
    const int hh = th % Hq;
    const int G = Hq / Hkv;
    const size_t tg = ((size_t)t * Hkv + hh / G) * kTopK;
    // each slot's row, then every partial loaded together (a slot with no
    // selection reads a row of its own and is dropped by selects, never by a
    // multiply, so a stale non-finite value cannot leak in)
    bool ok[kTopK];
    size_t row[kTopK];
#pragma unroll
    for (int i = 0; i < kTopK; ++i) {
        if (DIRECT) {
            const int b = sel[tg + i];
            ok[i] = b >= 0 && b < maxblk;
            row[i] = (size_t)th * kTopK + i;
        } else {
            const int pe = w.pos_of[tg + i];
            ok[i] = pe >= 0;
            row[i] = (size_t)(ok[i] ? pe : 0) * G + hh % G;
        }
    }
    float li[kTopK];
    u32x4 oi[kTopK];
#pragma unroll
    for (int i = 0; i < kTopK; ++i) {
        li[i] = w.part_lse[row[i]];
        oi[i] = ld16_stream(w.part_o + row[i] * kHeadDim + 8 * part);
    }
    float mx = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < kTopK; ++i) mx = ok[i] ? fmaxf(mx, li[i]) : mx;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float den = 0.f;
#pragma unroll
    for (int i = 0; i < kTopK; ++i) {
        const float wi = __expf(li[i] - mx);
        den = ok[i] ? den + wi : den;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc[2 * e] = ok[i] ? acc[2 * e] + wi * bf16_lo(oi[i][e]) : acc[2 * e];
            acc[2 * e + 1] = ok[i] ? acc[2 * e + 1] + wi * bf16_hi(oi[i][e]) : acc[2 * e + 1];
        }
    }
    // a row with no selection attends nothing: out = 0, lse = -inf
    const bool empty = !(den > 0.f);
    const float inv = empty ? 0.f : 1.0f / den;
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = pack2_bf16(acc[2 * e] * inv, acc[2 * e + 1] * inv);
    *reinterpret_cast<u32x4*>(out + (size_t)th * kHeadDim + 8 * part) = o;
    if (lse_out && part == 0) lse_out[th] = empty ? -__builtin_inff() : mx + __logf(den);
}

}  // namespace
}  // namespace msa

size_t msa_prefill_ws_bytes(const MsaShape& s, int total_q) {
    using namespace msa;
    return prefill_ws_size(s.B, s.Hkv, s.maxblk, total_q, s.Hq);
}

hipError_t msa_launch_prefill(const MsaShape& s, int total_q, const uint16_t* q,
                              const uint16_t* k_cache, const uint16_t* v_cache,
                              const int32_t* block_table, const int32_t* seq_lens,
                              const int32_t* cu_q, const int32_t* sel, uint16_t* out, float* lse,
                              void* ws, hipStream_t st) {
    using namespace msa;
    if (total_q == 0) return hipSuccess;
    const int NB = s.B * s.Hkv * s.maxblk;
    PrefillWs w = prefill_ws(ws, s.B, s.Hkv, s.maxblk, total_q, s.Hq);
    const int tiles = max_tiles(total_q, s.B, s.Hkv);
    const size_t map_lds = (size_t)s.maxblk * sizeof(int32_t);
    // buckets of at most small_cnt entries (kSmallRows rows) are small
    const int small_cnt = kSmallRows / (s.Hq / s.Hkv);
    if (mq_form(s, total_q)) {
        // a few queries per sequence: one kernel finds each (sequence, group)'s
        // blocks and attends them.  P workgroups per (sequence, group): about
        // eight blocks each when the queries are spread evenly over the
        // sequences, and never more than kMqMaxOwn.  Each workgroup repeats
        // the union, so fewer and longer ones win up to a point: at 8 x 60k
        // with 4 drafts the attention call took 66.5, 58.5, 54.0 and 52.5 us
        // at 1, 2, 4 and 8 blocks per workgroup with the pages looked up per
        // block, and 48.6 and 59.8 us at 8 and 16 with the lookups together.
        const int u_avg = std::min(s.maxblk, ceil_div(total_q, s.B) * kTopK);
        const int u_max = std::min(s.maxblk, total_q * kTopK);
        const int P = std::max({1, ceil_div(u_avg, 8), ceil_div(u_max, kMqMaxOwn)});
        int32_t* sel_rw = const_cast<int32_t*>(sel);  // read only: no selection in this form
        if ((int64_t)total_q * kTopK <= kMqSmallEntries)
            hipLaunchKernelGGL((mq_block_kernel<false, 1, kMqSmallEntries>), dim3(s.B * s.Hkv, P),
                               dim3(kDecThreads), 0, st, q, k_cache, v_cache, block_table, seq_lens,
                               cu_q, sel_rw, nullptr, w, s.Hq, s.Hkv, s.maxblk, P, s.scale * kLog2e);
        else
            hipLaunchKernelGGL((mq_block_kernel<false, 1, kMqEntries>), dim3(s.B * s.Hkv, P),
                               dim3(kDecThreads), 0, st, q, k_cache, v_cache, block_table, seq_lens,
                               cu_q, sel_rw, nullptr, w, s.Hq, s.Hkv, s.maxblk, P, s.scale * kLog2e);
        const int nth = total_q * s.Hq * 16;
        hipLaunchKernelGGL(prefill_merge_kernel<true>, dim3(ceil_div(nth, 256)), dim3(256), 0, st, sel,
                           w, out, lse, total_q, s.Hq, s.Hkv, s.maxblk);
        return hipGetLastError();
    }
    if (NB <= kSmallMapBuckets && (int64_t)total_q * s.Hkv * kTopK <= kSmallMapSel) {
        hipLaunchKernelGGL(inverse_map_small_kernel, dim3(1), dim3(kSmallMapThreads), 0, st, sel, cu_q, w,
                           total_q, s.B, s.Hkv, s.maxblk, small_cnt);
    } else {
        hipLaunchKernelGGL(zero_kernel, dim3(min(1024, ceil_div(NB, 256))), dim3(256), 0, st,
                           w.counts, NB);
        hipLaunchKernelGGL(bucket_count_kernel, dim3(tiles), dim3(kMapThreads), map_lds, st, sel,
                           cu_q, w.counts, w.tile_base, s.B, s.Hkv, s.maxblk);
        hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, st, w.counts, w.offsets,
                           w.buckets, w.small, NB, small_cnt);
        hipLaunchKernelGGL(bucket_fill_kernel, dim3(tiles), dim3(kMapThreads), map_lds, st, sel,
                           cu_q, w.offsets, w.tile_base, w.entries, w.pos_of, s.B, s.Hkv, s.maxblk);
    }
    // at most one nonempty bucket per selection, and at most one bucket of
    // more than small_cnt entries per small_cnt + 1 selections
    const int64_t n_sel = (int64_t)total_q * s.Hkv * kTopK;
    const int n_bk = (int)std::min<int64_t>(NB, n_sel);
    const int n_large = (int)std::min<int64_t>(NB, n_sel / (small_cnt + 1));
    if (n_large > 0)
        hipLaunchKernelGGL(block_major_kernel, dim3(ceil_div(n_large, 8) * 8), dim3(kPfThreads), 0,
                           st, q, k_cache, v_cache, block_table, seq_lens, cu_q, w, s.Hq, s.Hkv, s.maxblk,
                           s.scale * kLog2e);
    hipLaunchKernelGGL(bucket_small_kernel, dim3(n_bk), dim3(kDecThreads), 0, st, q, k_cache,
                       v_cache, block_table, seq_lens, cu_q, w, s.Hq, s.Hkv, s.maxblk,
                       s.scale * kLog2e);
    const int nth = total_q * s.Hq * 16;
    hipLaunchKernelGGL(prefill_merge_kernel<false>, dim3(ceil_div(nth, 256)), dim3(256), 0, st, sel, w,
                       out, lse, total_q, s.Hq, s.Hkv, s.maxblk);
    return hipGetLastError();
}

// The multi-query step's workspace: block scores [T, Hkv, maxblk] fp32, the
// selection [T, Hkv, k] (used when the caller passes none), then the prefill
// workspace.
size_t msa_multi_query_ws_bytes(const MsaShape& s, int total_q) {
    using namespace msa;
    return align256((size_t)total_q * s.Hkv * s.maxblk * 4) +
           align256((size_t)total_q * s.Hkv * kTopK * 4) + msa_prefill_ws_bytes(s, total_q);
}

hipError_t msa_launch_multi_query_step(const MsaShape& s, int total_q, const uint16_t* q_idx,
                                       const uint16_t* kidx, const uint16_t* q,
                                       const uint16_t* k_cache, const uint16_t* v_cache,
                                       const int32_t* block_table, const int32_t* seq_lens,
                                       const int32_t* cu_q, uint16_t* out, float* lse,
                                       int32_t* sel_out, void* ws, hipStream_t st) {
    using namespace msa;
    if (total_q == 0) return hipSuccess;
    char* base = static_cast<char*>(ws);
    float* scores = reinterpret_cast<float*>(base);
    base += align256((size_t)total_q * s.Hkv * s.maxblk * 4);
    int32_t* sel = sel_out ? sel_out : reinterpret_cast<int32_t*>(base);
    base += align256((size_t)total_q * s.Hkv * kTopK * 4);
    hipError_t e = msa_launch_index_score(s, total_q, q_idx, kidx, block_table, seq_lens, cu_q,
                                          scores, st);
    if (e != hipSuccess) return e;
    // The attention kernel makes the selections itself when each wavefront
    // selects about one query: every stripe of a (sequence, group) repeats
    // them, which at 8 x 60k cost more than the separate selection launch with
    // 8 drafts per sequence (104.7 against 100.5 us) and saved it with 4
    // (64.8 against 66.7 us).
    const bool fused = mq_form(s, total_q) && total_q <= 4 * s.B && s.maxblk <= 16 * kWave;
    if (!fused) {  // the three calls: selection, then the prefill entry's own form
        e = msa_launch_topk(s, total_q, scores, seq_lens, cu_q, sel, st);
        if (e != hipSuccess) return e;
        return msa_launch_prefill(s, total_q, q, k_cache, v_cache, block_table, seq_lens, cu_q,
                                  sel, out, lse, base, st);
    }
    PrefillWs w = prefill_ws(base, s.B, s.Hkv, s.maxblk, total_q, s.Hq);
    // stripes as in msa_launch_prefill's multi-query form
    const int u_avg = std::min(s.maxblk, ceil_div(total_q, s.B) * kTopK);
    const int u_max = std::min(s.maxblk, total_q * kTopK);
    const int P = std::max({1, ceil_div(u_avg, 8), ceil_div(u_max, kMqMaxOwn)});
#define MSA_MQ(NPT, CAP)                                                                       \
    hipLaunchKernelGGL((mq_block_kernel<true, NPT, CAP>), dim3(s.B * s.Hkv, P), dim3(kDecThreads), \
                       0, st, q, k_cache, v_cache, block_table, seq_lens, cu_q, sel, scores, w,   \
                       s.Hq, s.Hkv, s.maxblk, P, s.scale * kLog2e)
    const bool small = (int64_t)total_q * kTopK <= kMqSmallEntries;
    if (s.maxblk <= 8 * kWave) {
        if (small) MSA_MQ(8, kMqSmallEntries);
        else MSA_MQ(8, kMqEntries);
    } else {
        if (small) MSA_MQ(16, kMqSmallEntries);
        else MSA_MQ(16, kMqEntries);
    }
#undef MSA_MQ
    const int nth = total_q * s.Hq * 16;
    hipLaunchKernelGGL(prefill_merge_kernel<true>, dim3(ceil_div(nth, 256)), dim3(256), 0, st, sel, w,
                       out, lse, total_q, s.Hq, s.Hkv, s.maxblk);
    return hipGetLastError();
}
