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
//
// Many queries per sequence (chunked prefill) make scoring a dense
// contraction, [tokens x 64] . [64 x (query, group) rows], reduced by a max
// over each 128-token block.  A second kernel handles that case as a GEMM:
// a workgroup of 8 wavefronts owns 1024 rows of one sequence (their q_idx
// held in registers as 32x32x16 B operands) and a chunk of 64 blocks; each
// block's index keys are staged once in LDS (double-buffered, rows padded so
// the A-operand reads are bank-conflict free) and used by all 8 wavefronts.
// The epilogue masks tokens past each row's position and keeps per-row block
// maxima in registers, so the 32x32 products never leave the chip.
#include <type_traits>

#include "msa_common.hpp"

namespace msa {
namespace {

constexpr int kScoreWaves = 4;  // blocks per workgroup (one per wavefront)

// The new decode tokens' rows, for the step that appends them to the caches
// as it scores (one token per sequence, at position seq_lens[s] - 1).
struct AppendRows {
    const uint16_t* kidx_new;  // [B, Hidx, 64]
    const uint16_t* k_new;     // [B, Hkv, 128]
    const uint16_t* v_new;     // [B, Hkv, 128]
    uint16_t* kidx_cache;      // [P, Hidx, 128, 64], the array scored
    uint16_t* k_cache;         // [P, Hkv, 128, 128]
    uint16_t* v_cache;
};

// kInvisible: write -inf for the blocks past every row's position (the ABI's
// score rows); the fused decode step, whose selection never reads them,
// skips those stores.  kAppend (decode only): the wavefront of each
// sequence's last block writes the new token's rows into the caches and
// scores its index-key row from the new values, so the cache slot is never
// read back in this launch; the attention launches that follow see the
// appended K/V.
template <bool kInvisible, bool kAppend>
__global__ __launch_bounds__(kScoreWaves * kWave)
void index_score_kernel(const uint16_t* __restrict__ q_idx,   // [T, Hkv, 64]
                        const uint16_t* kidx,                 // [P, Hidx, 128, 64]
                        const int32_t* __restrict__ block_table,
                        const int32_t* __restrict__ seq_lens,
                        const int32_t* __restrict__ cu_q,
                        float* __restrict__ scores,           // [T, Hkv, maxblk]
                        int Hkv, int Hidx, int maxblk, AppendRows ap) {
    // wave-uniform to the compiler too: the block's tests are scalar branches
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = threadIdx.x % kWave;
    // grid: x = (sequence, index head), y = block chunk, so the sequences vary
    // fastest in dispatch order; the pair is skewed by the chunk because
    // workgroups are dealt to the XCDs round-robin: without it sequence s
    // would always land on XCD s mod 8, and in a ragged batch the XCD holding
    // the longest rows would finish last
    const int SH = gridDim.x;
    const int xs = (int)((blockIdx.x + blockIdx.y) % (unsigned)SH);
    const int b = blockIdx.y * kScoreWaves + wave;
    const int s = xs / Hidx;
    const int ih = xs % Hidx;
    if (b >= maxblk) return;

    // The block-table entry is loaded only once the block is known to be
    // visible: in a ragged batch most of the grid, which is sized by the
    // longest row, holds blocks past their sequence's end, and a wavefront
    // that has issued a load keeps its slot until the load returns.  The
    // sequence length, which decides, is a scalar load (cached after its
    // first use).
    const int L = seq_lens[s];
    // cu_q == nullptr: decode, query token s is sequence s's only query
    const int q0 = cu_q ? cu_q[s] : s;
    const int nq = cu_q ? cu_q[s + 1] - q0 : 1;
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
        if (!kInvisible) return;
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
    const int page = block_table[(size_t)s * maxblk + b];  // b < maxblk: in bounds

    // A operands: the block's index keys.  Tile mt covers tokens 16*mt..16*mt+15;
    // k-step i of lane group kg takes dims 32*i + 8*kg .. +7 (16-byte chunk
    // 4i + kg) of the token row.  The 16 KB arrive in sixteen contiguous 1 KB
    // loads (load j: tokens 8j .. 8j+7; lane l: token 8j + l/8, chunk l % 8)
    // -- whole 128-byte lines per instruction, where loading in operand order
    // would request half lines -- and reach operand order through this
    // wavefront's 8 KB LDS tile, half a block at a time.  Chunk c of local
    // token t sits at chunk c ^ (t mod 8), so the operand reads of 8
    // consecutive tokens fall in 8 different bank groups.  LDS operations of
    // one wavefront complete in order, so the tile needs no barrier.
    __shared__ __attribute__((aligned(16))) u32x4 kstage[kScoreWaves][kBlock / 2 * 8];
    u32x4* st = kstage[wave];
    const u32x4* kb = reinterpret_cast<const u32x4*>(kidx + ((size_t)page * Hidx + ih) * kBlock * kIdxDim);
    // B operands of rows r0 .. r0+15 (lane row m_in, dims 32i + 8kg .. +7;
    // zero past the last row).  The first group's are loaded ahead of the
    // keys, each later group's during the products of the one before, so no
    // row waits for a query load after its keys arrive.
    auto load_rows = [&](int r0, bf16x8 (&bq)[2]) {
        const int rho = r0 + m_in;
        const bool ok = rho < nrows;
        const int qi = ok ? rho / R : 0;
        const int g = (Hidx == 1) ? (ok ? rho % R : 0) : ih;
        const uint16_t* qrow = q_idx + ((size_t)(q0 + qi) * Hkv + g) * kIdxDim;
#pragma unroll
        for (int i = 0; i < 2; ++i)
            bq[i] = as_bf16x8(ok ? ld16(qrow + 32 * i + 8 * kg) : u32x4{0u, 0u, 0u, 0u});
    };
    bf16x8 bq_next[2];
    load_rows(0, bq_next);
    u32x4 raw[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) raw[j] = ld16_stream(kb + kWave * j + lane);
    // kAppend: this wavefront's block holds the sequence's new token (decode:
    // position L - 1) in slot tn; lanes 0..7 fetch its 8 index-key pieces.
    const bool new_block = kAppend && b == last_pos / kBlock;  // wave-uniform
    const int tn = last_pos % kBlock;
    u32x4 knew = {0u, 0u, 0u, 0u};
    if (new_block && lane < 8)
        knew = ld16(ap.kidx_new + ((size_t)s * Hidx + ih) * kIdxDim + 8 * lane);
    bf16x8 a[8][2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            const int t = 8 * jj + lane / 8;  // local token (tokens 64 half + t)
            st[t * 8 + ((lane % 8) ^ (t & 7))] = raw[8 * half + jj];
        }
        if (new_block && tn / 64 == half && lane < 8) {
            // the slot's row comes from the new keys (this later LDS write of
            // the same wavefront lands after the stale one) and goes to the cache
            st[(tn % 64) * 8 + (lane ^ (tn & 7))] = knew;
            *reinterpret_cast<u32x4*>(ap.kidx_cache + (((size_t)page * Hidx + ih) * kBlock + tn) * kIdxDim +
                                      8 * lane) = knew;
        }
#pragma unroll
        for (int mq = 0; mq < 4; ++mq) {
            const int t = 16 * mq + m_in;
#pragma unroll
            for (int i = 0; i < 2; ++i) a[4 * half + mq][i] = as_bf16x8(st[t * 8 + ((4 * i + kg) ^ (t & 7))]);
        }
    }

    const int tok0 = b * kBlock;
    for (int r0 = 0; r0 < nrows; r0 += 16) {
        const int rho = r0 + m_in;
        const bool row_ok = rho < nrows;
        const int qi = row_ok ? rho / R : 0;
        const int t = q0 + qi;
        const int g = (Hidx == 1) ? (row_ok ? rho % R : 0) : ih;
        const int p = first_pos + qi;
        const bf16x8 bq[2] = {bq_next[0], bq_next[1]};
        if (r0 + 16 < nrows) load_rows(r0 + 16, bq_next);
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
    if (new_block && ih == 0) {
        // the new token's K and V rows (one per KV group), read by the
        // attention launches that follow
        constexpr int kPieces = kHeadDim / 8;  // 16-byte pieces per K or V row
        for (int c = lane; c < Hkv * kPieces; c += kWave) {
            const int g = c / kPieces;
            const size_t src = ((size_t)s * Hkv + g) * kHeadDim + 8 * (c % kPieces);
            const size_t dst = (((size_t)page * Hkv + g) * kBlock + tn) * kHeadDim + 8 * (c % kPieces);
            const u32x4 kv = ld16(ap.k_new + src);
            const u32x4 vv = ld16(ap.v_new + src);
            *reinterpret_cast<u32x4*>(ap.k_cache + dst) = kv;
            *reinterpret_cast<u32x4*>(ap.v_cache + dst) = vv;
        }
    }
}


// ---------------------------------------------------------------------------
// GEMM form for many queries per sequence
// ---------------------------------------------------------------------------
constexpr int kGWaves = 8;                       // wavefronts per workgroup
constexpr int kGTiles = 4;                       // 32-row tiles per wavefront
constexpr int kGRows = kGWaves * kGTiles * 32;   // rows per workgroup (1024)
constexpr int kGBlocks = 64;                     // blocks per workgroup chunk
constexpr int kKStrideB = kIdxDim * 2 + 16;      // bytes per LDS index-key row (padded)
constexpr int kStageBlocks = 16;                 // block maxima staged per row before a flush
constexpr int kStageStride = kStageBlocks + 1;   // floats per staged row (padded)
// s_waitcnt immediate: vector-memory count 0, the other counters unconstrained
// (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int kWaitVmcnt0 = 0x0F70;

// Which (sequence, row group) this workgroup serves.  Sequence s has
// ceil(nq_s * R / kGRows) row groups; group ids are dealt out in sequence order.
// Returns false if blockIdx.x is past the last group.
__device__ bool find_row_group(const int32_t* __restrict__ cu_q, int B, int R, int gid, int* s_out,
                               int* g_out) {
    const int lane = __lane_id();
    int base = 0;
    for (int c0 = 0; c0 < B; c0 += kWave) {
        const int i = c0 + lane;
        const int nq = (i < B) ? (cu_q[i + 1] - cu_q[i]) : 0;
        const int groups = (nq * R + kGRows - 1) / kGRows;
        int scan = groups;  // inclusive prefix over lanes
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const int v = __shfl_up(scan, off, kWave);
            if (lane >= off) scan += v;
        }
        const uint64_t hit = __ballot(base + scan > gid);
        if (hit) {
            const int first = __builtin_ctzll(hit);
            const int prev = __shfl(scan - groups, first, kWave);
            *s_out = c0 + first;
            *g_out = gid - base - prev;
            return true;
        }
        base += __shfl(scan, kWave - 1, kWave);
    }
    return false;
}

__global__ __launch_bounds__(kGWaves * kWave)
void index_score_gemm_kernel(const uint16_t* __restrict__ q_idx,   // [T, Hkv, 64]
                             const uint16_t* __restrict__ kidx,    // [P, Hidx, 128, 64]
                             const int32_t* __restrict__ block_table,
                             const int32_t* __restrict__ seq_lens,
                             const int32_t* __restrict__ cu_q,
                             float* __restrict__ scores,           // [T, Hkv, maxblk]
                             int B, int Hkv, int Hidx, int maxblk) {
    __shared__ __attribute__((aligned(16))) unsigned char ktile[4][kBlock * kKStrideB];
    // per-row block maxima of the current 16 blocks: each row's scores leave
    // as one 64-byte run instead of 8-byte pieces every second block
    __shared__ float stage[kGRows * kStageStride];
    __shared__ int grp[2];

    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = tid % kWave;
    const int ih = blockIdx.z;
    const int R = (Hidx == 1) ? Hkv : 1;
    if (wave == 0) {
        int s_, g_;
        const bool ok = find_row_group(cu_q, B, R, blockIdx.x, &s_, &g_);
        if (lane == 0) {
            grp[0] = ok ? s_ : -1;
            grp[1] = g_;
        }
    }
    __syncthreads();
    // workgroup-uniform: kept in scalar registers so that every test derived
    // from them is a scalar branch
    const int s = __builtin_amdgcn_readfirstlane(grp[0]);
    if (s < 0) return;
    const int rg = __builtin_amdgcn_readfirstlane(grp[1]);
    const int L = seq_lens[s];
    const int q0 = cu_q[s];
    const int nq = cu_q[s + 1] - q0;
    const int nrows = nq * R;
    const int row0 = rg * kGRows;                       // first row of the workgroup
    const int row_end = min(nrows, row0 + kGRows);
    const int p_first = L - nq + row0 / R;              // smallest position in the group
    const int p_last = L - nq + (row_end - 1) / R;      // largest
    const int b_begin = blockIdx.y * kGBlocks;
    const int b_end = min(maxblk, b_begin + kGBlocks);
    // blocks at or past b_vis_end are after every row's position: -inf
    const int b_vis_end = min(b_end, p_last / kBlock + 1);

    const int n = lane % 32;  // row within a tile / token within a token tile
    const int h = lane / 32;  // lane half: dims 32h .. 32h+31 of the reduction

    // B operands: q_idx of this wave's 4 row tiles
    bf16x8 qb[kGTiles][4];
    int prow[kGTiles];  // position of each lane's row (per tile)
    bool rok[kGTiles];
#pragma unroll
    for (int r = 0; r < kGTiles; ++r) {
        const int rho = row0 + (wave * kGTiles + r) * 32 + n;
        rok[r] = rho < row_end;
        const int qi = rok[r] ? rho / R : 0;
        const int g = (Hidx == 1) ? (rok[r] ? rho % R : 0) : ih;
        prow[r] = L - nq + qi;
        const uint16_t* qrow = q_idx + ((size_t)(q0 + qi) * Hkv + g) * kIdxDim + 32 * h;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            qb[r][i] = as_bf16x8(rok[r] ? ld16(qrow + 8 * i) : u32x4{0u, 0u, 0u, 0u});
    }

    // index-key tile staging: 16 KB per block, two 16-byte pieces per thread
    auto load_tile = [&](int b, u32x4* v) {
        const int page = block_table[(size_t)s * maxblk + b];
        const unsigned char* src =
            reinterpret_cast<const unsigned char*>(kidx + ((size_t)page * Hidx + ih) * kBlock * kIdxDim);
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int c = tid + kGWaves * kWave * it;  // 16-byte piece: row c/8, col c%8
            v[it] = ld16(src + c * 16);
        }
    };
    auto store_tile = [&](int buf, const u32x4* v) {
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int c = tid + kGWaves * kWave * it;
            *reinterpret_cast<u32x4*>(&ktile[buf][(c / 8) * kKStrideB + (c % 8) * 16]) = v[it];
        }
    };

    // Blocks go in pairs (b_begin is even) through four LDS tile buffers: the
    // pair (b0, b0 + 1) sits in buffers cur, cur + 1 while the next pair is
    // fetched into registers; at the end of the pair those registers go to the
    // other two buffers and one barrier publishes them.  Each fetch has two
    // blocks of work to arrive, and every load is waited for inside the
    // iteration that issued it.
    u32x4 stage0[2], stage1[2];
    if (b_begin < b_vis_end) load_tile(b_begin, stage0);
    if (b_begin + 1 < b_vis_end) load_tile(b_begin + 1, stage1);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // every path: nothing outstanding
    if (b_begin < b_vis_end) store_tile(0, stage0);
    if (b_begin + 1 < b_vis_end) store_tile(1, stage1);
    __syncthreads();

    // Block b from LDS buffer buf: per-row maxima over this lane half's tokens.
    // Per 32-token tile the four row tiles' products are independent chains,
    // issued interleaved; their maxima are taken after the last product.
    // Only blocks that reach past the group's first position need the causal
    // mask (a workgroup-uniform choice made once per block).
    auto block_body = [&](const unsigned char* kt, int tok_base, float (&mx)[kGTiles], auto masked) {
        // The 16 (token tile tt, row tile r) products of the block form one
        // rolling sequence: the four k-steps of each product are interleaved
        // with the reduction of the previous product (four of its values per
        // k-step), so the VALU maxima run while the matrix core works.
        // Value v of a 32x32 result is token tok_base + 32tt + 8(v/4) + 4h +
        // v%4 of row n.
        f32x16 prev = {};
        int prev_lim = 0;
        auto reduce4 = [&](float m, const f32x16& acc, int q, int lim) {
#pragma unroll
            for (int v = 4 * q; v < 4 * q + 4; ++v) {
                if constexpr (decltype(masked)::value)
                    m = fmaxf(m, (8 * (v / 4) + (v % 4) <= lim) ? acc[v] : -__builtin_inff());
                else
                    m = fmaxf(m, acc[v]);
            }
            return m;
        };
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            bf16x8 a[4];
            const unsigned char* arow = kt + (32 * tt + n) * kKStrideB + 64 * h;
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = as_bf16x8(*reinterpret_cast<const u32x4*>(arow + 16 * i));
#pragma unroll
            for (int r = 0; r < kGTiles; ++r) {
                const int j = tt * kGTiles + r;  // position in the sequence
                f32x16 acc = {};
                float m = -__builtin_inff();
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc = mfma32(a[i], qb[r][i], acc);
                    if (j > 0) m = reduce4(m, prev, i, prev_lim);
                    // keep the order: one product, then the VALU work beside it
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, decltype(masked)::value ? 8 : 2, 0);
                }
                if (j > 0) {
                    const int pr = (j - 1) % kGTiles;
                    mx[pr] = fmaxf(mx[pr], m);
                }
                prev = acc;
                prev_lim = prow[r] - tok_base - 32 * tt - 4 * h;
            }
        }
        float m = -__builtin_inff();
#pragma unroll
        for (int q = 0; q < 4; ++q) m = reduce4(m, prev, q, prev_lim);
        mx[kGTiles - 1] = fmaxf(mx[kGTiles - 1], m);
    };
    auto do_block = [&](int b, int buf, float (&mx)[kGTiles]) {
#pragma unroll
        for (int r = 0; r < kGTiles; ++r) mx[r] = -__builtin_inff();
        if (b >= b_vis_end) return;  // workgroup-uniform
        const int tok_base = b * kBlock;
        if (tok_base + kBlock - 1 > p_first)
            block_body(ktile[buf], tok_base, mx, std::true_type{});
        else
            block_body(ktile[buf], tok_base, mx, std::false_type{});
    };

    // This wavefront's 128 rows of the stage -> scores[.., fb .. fb + cnt - 1]:
    // 16 lanes per row, four rows per store instruction.  Row rho of the
    // group is score row (q0 + rho / R) * H_kv + g, i.e. q0 H_kv + rho when
    // one index head serves every group (R = H_kv), else (q0 + rho) H_kv + ih.
    const int wrow0 = wave * kGTiles * 32;  // first stage row of this wavefront
    auto flush = [&](int fb, int cnt) {
        const int col = lane % kStageBlocks;
#pragma unroll 4
        for (int k = 0; k < kGTiles * 32 * kStageBlocks / kWave; ++k) {
            const int rl = wrow0 + lane / kStageBlocks + (kWave / kStageBlocks) * k;
            const int rho = row0 + rl;
            if (col < cnt && rho < row_end) {
                const size_t srow = (Hidx == 1) ? (size_t)q0 * Hkv + rho : (size_t)(q0 + rho) * Hkv + ih;
                scores[srow * maxblk + fb + col] = stage[rl * kStageStride + col];
            }
        }
    };

    for (int b0 = b_begin, cur = 0; b0 < b_end; b0 += 2, cur ^= 2) {
        if (b0 + 2 < b_vis_end) load_tile(b0 + 2, stage0);
        if (b0 + 3 < b_vis_end) load_tile(b0 + 3, stage1);
        float m0[kGTiles], m1[kGTiles];
        do_block(b0, cur, m0);
        do_block(b0 + 1, cur + 1, m1);
        // both lane halves saw different tokens of the same row: combine, then
        // half h stages block b0 + h (a wavefront reads back only its own rows,
        // in order, so no barrier is needed before the flush)
        const int j = (b0 - b_begin) % kStageBlocks;
#pragma unroll
        for (int r = 0; r < kGTiles; ++r) {
            m0[r] = fmaxf(m0[r], __shfl_xor(m0[r], 32, kWave));
            m1[r] = fmaxf(m1[r], __shfl_xor(m1[r], 32, kWave));
            stage[(wrow0 + r * 32 + n) * kStageStride + j + h] = h ? m1[r] : m0[r];
        }
        if (j + 2 == kStageBlocks || b0 + 2 >= b_end) {
            const int fb = b0 - j;
            flush(fb, min(kStageBlocks, b_end - fb));
        }
        // buffers cur ^ 2, (cur ^ 2) + 1 were last read in the previous pair,
        // which every wavefront finished before that pair's barrier
        if (b0 + 2 < b_vis_end) store_tile(cur ^ 2, stage0);
        if (b0 + 3 < b_vis_end) store_tile((cur ^ 2) + 1, stage1);
        __syncthreads();
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
    const int R = (s.Hidx == 1) ? s.Hkv : 1;
    // Up to 128 queries per sequence on average the per-block kernel (each
    // block's keys loaded once for all of its sequence's rows) is faster:
    // scoring 8 x 60k with 8, 32, 128 or 256 queries per sequence took 16.6,
    // 38.0, 111.5 and 197 us there against 150, 151, 160 and 164 us in the
    // GEMM form, whose few 1,024-row groups leave most of the chip idle at
    // these sizes.
    if (total_q > 128 * s.B) {
        // many queries per sequence on average: GEMM form.  Upper bound on the
        // number of row groups: sum_s ceil(nq_s R / rows) <= total_q R / rows + B.
        const int groups = ceil_div(total_q * R, kGRows) + s.B;
        dim3 grid(groups, ceil_div(s.maxblk, kGBlocks), s.Hidx);
        hipLaunchKernelGGL(index_score_gemm_kernel, grid, dim3(kGWaves * kWave), 0, st, q_idx, kidx,
                           block_table, seq_lens, cu_q, scores, s.B, s.Hkv, s.Hidx, s.maxblk);
        return hipGetLastError();
    }
    dim3 grid(s.B * s.Hidx, ceil_div(s.maxblk, kScoreWaves));
    hipLaunchKernelGGL((index_score_kernel<true, false>), grid, dim3(kScoreWaves * kWave), 0, st,
                       q_idx, kidx, block_table, seq_lens, cu_q, scores, s.Hkv, s.Hidx, s.maxblk,
                       AppendRows{});
    return hipGetLastError();
}

hipError_t msa_launch_index_score_decode(const MsaShape& s, const uint16_t* q_idx,
                                         const uint16_t* kidx, const int32_t* block_table,
                                         const int32_t* seq_lens, float* scores,
                                         const DecodeAppend* app, hipStream_t st) {
    using namespace msa;
    if (s.B == 0) return hipSuccess;
    // scores past each row's own block stay unwritten: the decode step's
    // selection gives blocks past b_loc no key and never reads their values
    dim3 grid(s.B * s.Hidx, ceil_div(s.maxblk, kScoreWaves));
    if (app) {
        const AppendRows ap{app->kidx_new, app->k_new, app->v_new,
                            app->kidx_cache, app->k_cache, app->v_cache};
        hipLaunchKernelGGL((index_score_kernel<false, true>), grid, dim3(kScoreWaves * kWave), 0,
                           st, q_idx, static_cast<const uint16_t*>(app->kidx_cache), block_table,
                           seq_lens, static_cast<const int32_t*>(nullptr), scores, s.Hkv, s.Hidx,
                           s.maxblk, ap);
    } else {
        hipLaunchKernelGGL((index_score_kernel<false, false>), grid, dim3(kScoreWaves * kWave), 0,
                           st, q_idx, kidx, block_table, seq_lens,
                           static_cast<const int32_t*>(nullptr), scores, s.Hkv, s.Hidx, s.maxblk,
                           AppendRows{});
    }
    return hipGetLastError();
}
