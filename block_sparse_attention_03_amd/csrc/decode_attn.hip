// decode_attn.hip -- MSA sparse decode attention over the flattened page table.
//
// What it computes (aivizor serving-report news item, paragraph on MSA with
// paged attention): the KV-group dimension is flattened into the batch, so
// row r = s*H_kv + g is an ordinary paged sequence of row_lens[r] tokens whose
// pages are page_table[r][0..]; its G = H_q/H_kv query heads attend it with
// softmax(scale * q K^T) V.
//
// Mapping.  One workgroup (4 wavefronts) per (row, page): the page's K and V
// (2 x 32 KB) are read from HBM exactly once, and the row's G query heads are
// packed as the 16 columns of 16x16x32 bf16 matrix-core tiles, so one page
// load serves the whole GQA group.  Wavefront w scores tokens 32w..32w+31
// (S^T = K Q^T, fp32 accumulate); the page's per-head max and sum are
// combined through LDS; P is rounded to bf16 and shared through LDS; then
// wavefront w forms dims 32w..32w+31 of O^T = V^T P^T.  V is loaded with
// fully coalesced 16-byte reads into a row-major (swizzled) LDS tile, and the transposed
// matrix-core operand (4 consecutive tokens of one dim per lane) comes from
// the LDS transpose read.  Each page leaves a normalised partial
// output and its log-sum-exp in the workspace; a second kernel merges a row's
// pages with the Log-Sum-Exp rule (aivizor, KV-Block-Major paragraph).
#include "decode_tile.hpp"
#include "select.hpp"

namespace msa {
namespace {

struct DecodeWs {
    uint16_t* o;  // [R, k, G, 128] normalised partial outputs, bf16
    float* lse;   // [R, k, G]
};

__device__ __forceinline__ DecodeWs decode_ws(void* ws, int R, int G) {
    DecodeWs w;
    w.o = static_cast<uint16_t*>(ws);
    w.lse = reinterpret_cast<float*>(w.o + (size_t)R * kTopK * G * kHeadDim);
    return w;
}

// Q of row (sequence s, group g) as matrix-core B operands: head n of the
// group in column n (zero beyond G), dims 32i + 8kg .. +7 at k-step i.
__device__ __forceinline__ void load_q_operands(const uint16_t* __restrict__ q, int s, int g, int G,
                                                int Hq, bf16x8 (&qb)[4]) {
    const int lane = threadIdx.x % kWave;
    const int n = lane % 16;
    const int kg = lane / 16;
    const uint16_t* qrow = q + ((size_t)s * Hq + g * G + n) * kHeadDim;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        qb[i] = as_bf16x8(n < G ? ld16(qrow + 32 * i + 8 * kg) : u32x4{0u, 0u, 0u, 0u});
}

// One page's K and V in registers: K of this wavefront's 32 tokens as
// contiguous rows (operand order comes later, through the V tile), V rows
// with coalesced 16-byte loads (16 lanes per 256-byte row).  The whole page
// is loaded -- a page is always allocated in full, and unconditional loads
// keep the compiler from waiting on them early -- and tokens at or past the
// valid count are zeroed when V is written to LDS, so that P = 0 there never
// meets a non-finite V.
struct PageRegs {
    u32x4 k[8];
    u32x4 v[8];
};

__device__ __forceinline__ void load_page(const uint16_t* __restrict__ kp,
                                          const uint16_t* __restrict__ vp, PageRegs& pr) {
    const int tid = threadIdx.x;
    load_k_rows(kp, tid / kWave, tid % kWave, pr.k);
#pragma unroll
    for (int it = 0; it < 8; ++it)
        pr.v[it] = ld16_stream(vp + (tid / 16 + 16 * it) * kHeadDim + 8 * (tid % 16));
}

// The G query heads of row r (operands qb) against one page (in pr) holding
// nv valid tokens: writes the normalised partial output and log-sum-exp of
// page slot `slot`.  Every thread of the 256-thread workgroup calls it; the
// page's K goes through the V tile first, so a caller that attends another
// page with the same tile puts a barrier between the two.
__device__ __forceinline__ void compute_page(const bf16x8 (&qb)[4], const PageRegs& pr, int nv,
                                             int G, int r, int slot, void* __restrict__ ws, int R,
                                             float scale_log2, DecodeShared& sh) {
    uint16_t* vs = sh.vs;
    uint16_t* pl = sh.pl;
    auto& red_max = sh.red_max;
    auto& red_sum = sh.red_sum;
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = tid % kWave;
    const int n = lane % 16;   // head column (B / result) or row of A
    const int kg = lane / 16;  // lane group
    const u32x4 (&kraw)[8] = pr.k;
    const u32x4 (&vv)[8] = pr.v;
    bf16x8 ka[2][4];
    k_rows_to_operands(kraw, wave, lane, vs, ka);
    {
        // S^T = K Q^T for tokens 32w + 16j + 4kg + rr, head n
        f32x4 sacc[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            sacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < 4; ++i) sacc[j] = mfma16(ka[j][i], qb[i], sacc[j]);
        }
        float mx = -__builtin_inff();
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int tok = 32 * wave + 16 * j + 4 * kg + rr;
                if (tok >= nv) sacc[j][rr] = -__builtin_inff();
                mx = fmaxf(mx, sacc[j][rr]);
            }
        mx = wave_max_xor(mx, 16);
        mx = wave_max_xor(mx, 32);
        if (kg == 0) red_max[wave][n] = mx;
        // the maxima are visible and every wave has read its K out of the V tile
        __syncthreads();
        const float m = fmaxf(fmaxf(red_max[0][n], red_max[1][n]), fmaxf(red_max[2][n], red_max[3][n]));
        // P = exp(scale * (s - m)) rounded to bf16; the sum uses the rounded values
        float sum = 0.f;
        uint16_t pb[2][4];
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const float pv = __builtin_amdgcn_exp2f((sacc[j][rr] - m) * scale_log2);
                pb[j][rr] = f32_to_bf16(pv);
                sum += bf16_to_f32(pb[j][rr]);
            }
        sum += __shfl_xor(sum, 16, kWave);
        sum += __shfl_xor(sum, 32, kWave);
        if (kg == 0) red_sum[wave][n] = sum;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int tok = 32 * wave + 16 * j + 4 * kg;
            u32x2 w2 = {static_cast<uint32_t>(pb[j][0]) | (static_cast<uint32_t>(pb[j][1]) << 16),
                        static_cast<uint32_t>(pb[j][2]) | (static_cast<uint32_t>(pb[j][3]) << 16)};
            *reinterpret_cast<u32x2*>(pl + n * kPStride + tok) = w2;
        }
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const int tok = tid / 16 + 16 * it;
            *reinterpret_cast<u32x4*>(vs + vs_off(tok, 8 * (tid % 16))) =
                (tok < nv) ? vv[it] : u32x4{0u, 0u, 0u, 0u};
        }
        __syncthreads();

        // O^T = V^T P^T for dims 32w .. 32w+31; k-step ks covers tokens 32ks..32ks+31,
        // lane group kg taking tokens 32ks + 4kg + 0..3 and 32ks + 16 + 4kg + 0..3.
        f32x4 oacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int ta = 32 * ks + 4 * kg;
            const u32x2 p0 = *reinterpret_cast<const u32x2*>(pl + n * kPStride + ta);
            const u32x2 p1 = *reinterpret_cast<const u32x2*>(pl + n * kPStride + ta + 16);
            const bf16x8 pbv = as_bf16x8(u32x4{p0[0], p0[1], p1[0], p1[1]});
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                // lane j of group kg points at token 32ks + 4kg + j/4 (and +16),
                // dims d0 + 4(j%4); the transpose read hands lane i dim d0 + i
                const uint16_t* src = vs + vs_off(ta + n / 4, 32 * wave + 16 * mt + 4 * (n % 4));
                const u32x2 v0a = lds_read_tr16(src);
                const u32x2 v1a = lds_read_tr16(src + 16 * kHeadDim);  // token + 16: same swizzle
                oacc[mt] = mfma16(as_bf16x8(u32x4{v0a[0], v0a[1], v1a[0], v1a[1]}), pbv, oacc[mt]);
            }
        }
        const float l = red_sum[0][n] + red_sum[1][n] + red_sum[2][n] + red_sum[3][n];
        if (n < G) {
            DecodeWs w = decode_ws(ws, R, G);
            const float inv = 1.0f / l;
            uint16_t* orow = w.o + (((size_t)r * kTopK + slot) * G + n) * kHeadDim;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                const int d = 32 * wave + 16 * mt + 4 * kg;
                *reinterpret_cast<u32x2*>(orow + d) =
                    u32x2{pack2_bf16(oacc[mt][0] * inv, oacc[mt][1] * inv),
                          pack2_bf16(oacc[mt][2] * inv, oacc[mt][3] * inv)};
            }
            if (wave == 0 && kg == 0)
                w.lse[((size_t)r * kTopK + slot) * G + n] = m * scale_log2 * kLn2 + __logf(l);
        }
    }
}


// Q, the page's K, then its V -- loads in the order their data is needed,
// since vector loads retire in issue order: the scores and the softmax wait
// only for Q and K while V is still arriving -- then the page's attention.
__device__ __forceinline__ void attend_page(const uint16_t* __restrict__ q,
                                            const uint16_t* __restrict__ kp,
                                            const uint16_t* __restrict__ vp, int nv, int s, int g,
                                            int G, int Hq, int r, int slot, void* __restrict__ ws,
                                            int R, float scale_log2, DecodeShared& sh) {
    bf16x8 qb[4];
    load_q_operands(q, s, g, G, Hq, qb);
    PageRegs pr;
    load_page(kp, vp, pr);
    // keep every load issued here, ahead of the first wait
    __builtin_amdgcn_sched_barrier(0);
    compute_page(qb, pr, nv, G, r, slot, ws, R, scale_log2, sh);
}

// The (row, workgroup-within-row) of a page workgroup on an (n_x, R) grid.
// Workgroups reach the 8 XCDs round-robin by linear id; when R is a
// multiple of 8 the k-th workgroup on XCD x takes row (k / n_x) * 8 + x, so
// that all n_x workgroups of a row share one L2 and what they all read of
// the row (its scores and block-table entries, or its page-table row, and
// its queries) comes from memory once (same-box A/Bs: 4 x 1M decode
// 0.3-1% faster, ragged 16-sequence decode 0.6%, 8 x 60k within noise).
__device__ __forceinline__ void xcd_row(int n_x, int R, int* x, int* r) {
    if (R % 8 != 0) {
        *x = blockIdx.x;
        *r = blockIdx.y;
        return;
    }
    const int lin = blockIdx.y * n_x + blockIdx.x;
    *x = (lin / 8) % n_x;
    *r = (lin / 8 / n_x) * 8 + lin % 8;
}

__global__ __launch_bounds__(kDecThreads)
void decode_page_kernel(const uint16_t* __restrict__ q,        // [B, Hq, 128]
                        const uint16_t* __restrict__ k_cache,  // [P, Hkv, 128, 128]
                        const uint16_t* __restrict__ v_cache,
                        const int32_t* __restrict__ page_table,  // [R, k]
                        const int32_t* __restrict__ row_lens,    // [R]
                        void* __restrict__ ws, int Hq, int Hkv, int R, float scale_log2) {
    __shared__ __attribute__((aligned(16))) DecodeShared sh;
    int slot, r;
    xcd_row(kTopK, R, &slot, &r);
    const int n_tok = row_lens[r];
    if (slot * kBlock >= n_tok) return;  // page not used by this row (uniform)
    const int nv = min(kBlock, n_tok - slot * kBlock);
    const int G = Hq / Hkv;
    const int s = r / Hkv;
    const int g = r % Hkv;
    const int page = page_table[(size_t)r * kTopK + slot];
    const size_t page_off = ((size_t)page * Hkv + g) * kBlock * kHeadDim;
    attend_page(q, k_cache + page_off, v_cache + page_off, nv, s, g, G, Hq, r, slot, ws, R,
                scale_log2, sh);
}

// Fused decode: the workgroup of (row r = s*H_kv + g, slot i) selects the
// row's top-k blocks itself from the block scores (every workgroup of the row
// makes the same, deterministic selection), maps its i-th selected block to
// a physical page through the block table -- the row's page table, kept on
// chip -- and attends that page.  Slot 0 also publishes the row's selection
// and length.  With PAGES the block-table entries are loaded beside the
// scores, so the selection hands over pages directly.
template <int NPT, int W, bool PAGES>
__global__ __launch_bounds__(kDecThreads)
void decode_fused_kernel(const float* __restrict__ scores,     // [B, Hkv, maxblk]
                         const int32_t* __restrict__ block_table,
                         const int32_t* __restrict__ seq_lens,
                         const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
                         const uint16_t* __restrict__ v_cache, int32_t* __restrict__ row_lens,
                         int32_t* __restrict__ sel_out, void* __restrict__ ws, int Hq, int Hkv,
                         int R, int maxblk, float scale_log2) {
    __shared__ __attribute__((aligned(16))) DecodeShared sh;
    __shared__ int32_t sel_idx[kTopK];
    __shared__ int32_t sel_page[kTopK];
    // the selection's LDS lives in the V tile, which is written only after
    // the barrier that ends the selection
    static_assert(sizeof(SelectShared<W>) <= sizeof(sh.vs), "selection scratch");
    SelectShared<W>* ssh = reinterpret_cast<SelectShared<W>*>(sh.vs);
    int slot, r;
    xcd_row(kTopK, R, &slot, &r);
    const int s = r / Hkv;
    const int g = r % Hkv;
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int w = (W == 1) ? 0 : wave;
    // W = 1: wavefront 0 selects alone (no barriers inside the search) while
    // the others wait; W = 4: all four wavefronts share a long row.  The
    // candidate loads are issued before the sequence length arrives.
    const bool selecting = (W == 4 || wave == 0);
    float raw[NPT];
    int page[NPT];
    if (selecting)
        load_candidates<NPT, W, PAGES>(scores + (size_t)r * maxblk, block_table + (size_t)s * maxblk,
                                       maxblk, w, lane, raw, page);
    const int p = seq_lens[s] - 1;
    const int b_loc = p / kBlock;
    const int n_sel = min(kTopK, b_loc + 1);
    if (selecting)
        select_row<NPT, W>(raw, page, b_loc, w, lane, ssh, [&](int pos, uint32_t, int b, int pg) {
            sel_idx[pos] = b;
            sel_page[pos] = pg;
        });
    __syncthreads();
    if (slot >= n_sel) return;  // uniform
    const int b = sel_idx[slot];
    if (slot == 0) {
        if (threadIdx.x < kTopK && sel_out) sel_out[(size_t)r * kTopK + threadIdx.x] = sel_idx[threadIdx.x];
        if (threadIdx.x == 0) row_lens[r] = (n_sel - 1) * kBlock + (p - kBlock * b_loc + 1);
    }
    // ascending order puts the own (partial) block last
    const int nv = (slot == n_sel - 1) ? p - kBlock * b_loc + 1 : kBlock;
    const int pg = PAGES ? sel_page[slot] : block_table[(size_t)s * maxblk + b];
    const size_t page_off = ((size_t)pg * Hkv + g) * kBlock * kHeadDim;
    attend_page(q, k_cache + page_off, v_cache + page_off, nv, s, g, Hq / Hkv, Hq, r, slot, ws, R,
                scale_log2, sh);
}

// Fused decode for batches with more page workgroups than the chip holds at
// once: the workgroup of (row r, slots PPW*x .. PPW*x + PPW-1) makes the
// row's selection once, as decode_fused_kernel does, keeps the row's query
// operands, and attends its pages one after the other with the next page's
// K and V loads issued before the current page's products, so that each
// compute unit keeps a page in flight while it computes.  Each page leaves
// the same partial output and log-sum-exp as in decode_fused_kernel, for the
// same merge.
template <int NPT, int W, bool PAGES, int PPW>
__global__ __launch_bounds__(kDecThreads)
void decode_multi_kernel(const float* __restrict__ scores,     // [B, Hkv, maxblk]
                         const int32_t* __restrict__ block_table,
                         const int32_t* __restrict__ seq_lens,
                         const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
                         const uint16_t* __restrict__ v_cache, int32_t* __restrict__ row_lens,
                         int32_t* __restrict__ sel_out, void* __restrict__ ws, int Hq, int Hkv,
                         int R, int maxblk, float scale_log2) {
    __shared__ __attribute__((aligned(16))) DecodeShared sh;
    __shared__ int32_t sel_idx[kTopK];
    __shared__ int32_t sel_page[kTopK];
    static_assert(sizeof(SelectShared<W>) <= sizeof(sh.vs), "selection scratch");
    SelectShared<W>* ssh = reinterpret_cast<SelectShared<W>*>(sh.vs);
    int x, r;
    xcd_row(kTopK / PPW, R, &x, &r);
    const int slot0 = x * PPW;
    const int s = r / Hkv;
    const int g = r % Hkv;
    const int G = Hq / Hkv;
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int w = (W == 1) ? 0 : wave;
    const bool selecting = (W == 4 || wave == 0);
    float raw[NPT];
    int page[NPT];
    if (selecting)
        load_candidates<NPT, W, PAGES>(scores + (size_t)r * maxblk, block_table + (size_t)s * maxblk,
                                       maxblk, w, lane, raw, page);
    const int p = seq_lens[s] - 1;
    const int b_loc = p / kBlock;
    const int n_sel = min(kTopK, b_loc + 1);
    if (selecting)
        select_row<NPT, W>(raw, page, b_loc, w, lane, ssh, [&](int pos, uint32_t, int b, int pg) {
            sel_idx[pos] = b;
            sel_page[pos] = pg;
        });
    __syncthreads();
    if (slot0 >= n_sel) return;  // uniform
    if (slot0 == 0) {
        if (threadIdx.x < kTopK && sel_out) sel_out[(size_t)r * kTopK + threadIdx.x] = sel_idx[threadIdx.x];
        if (threadIdx.x == 0) row_lens[r] = (n_sel - 1) * kBlock + (p - kBlock * b_loc + 1);
    }
    // pages of this workgroup, wave-uniform to the compiler (scalar loop
    // control, exact load waits across the loop)
    const int npg = __builtin_amdgcn_readfirstlane(min(PPW, n_sel - slot0));
    auto page_ptr = [&](int slot, const uint16_t* cache) {
        const int pg = PAGES ? sel_page[slot] : block_table[(size_t)s * maxblk + sel_idx[slot]];
        return cache + ((size_t)pg * Hkv + g) * kBlock * kHeadDim;
    };
    // ascending order puts the own (partial) block last
    auto valid = [&](int slot) { return (slot == n_sel - 1) ? p - kBlock * b_loc + 1 : kBlock; };
    bf16x8 qb[4];
    load_q_operands(q, s, g, G, Hq, qb);
    PageRegs pa, pb;
    load_page(page_ptr(slot0, k_cache), page_ptr(slot0, v_cache), pa);
    // pairs of pages through two register sets, then an odd last page
    for (int k = 0; k + 1 < npg; k += 2) {
        load_page(page_ptr(slot0 + k + 1, k_cache), page_ptr(slot0 + k + 1, v_cache), pb);
        __builtin_amdgcn_sched_barrier(0);
        compute_page(qb, pa, valid(slot0 + k), G, r, slot0 + k, ws, R, scale_log2, sh);
        __syncthreads();  // this page's reads of the V tile are done
        if (k + 2 < npg)
            load_page(page_ptr(slot0 + k + 2, k_cache), page_ptr(slot0 + k + 2, v_cache), pa);
        __builtin_amdgcn_sched_barrier(0);
        compute_page(qb, pb, valid(slot0 + k + 1), G, r, slot0 + k + 1, ws, R, scale_log2, sh);
        __syncthreads();
    }
    if (npg & 1) compute_page(qb, pa, valid(slot0 + npg - 1), G, r, slot0 + npg - 1, ws, R,
                              scale_log2, sh);
}

// Log-Sum-Exp merge of a row's pages: 16 threads per (row, head), each
// merging 8 dims (one 16-byte piece of every page's bf16 partial); four
// (row, head) pairs per 64-thread workgroup.
constexpr int kMergeThreads = 64;

__global__ __launch_bounds__(kMergeThreads)
void decode_merge_kernel(const int32_t* __restrict__ row_lens, const void* __restrict__ ws,
                         uint16_t* __restrict__ out, float* __restrict__ lse_out, int Hq,
                         int Hkv, int R) {
    const int idx = blockIdx.x * kMergeThreads + threadIdx.x;
    const int G = Hq / Hkv;
    const int rn = idx / 16;  // r * G + n
    const int part = idx % 16;
    if (rn >= R * G) return;
    const int r = rn / G;
    const int n = rn % G;
    DecodeWs w = decode_ws(const_cast<void*>(ws), R, G);
    const float* lp = w.lse + (size_t)r * kTopK * G + n;
    // every slot's partial is loaded together with the row length (slots past
    // the row's pages hold stale workspace values and are dropped by selects,
    // never by a multiply, so a stale non-finite value cannot leak in)
    float li[kTopK];
    u32x4 oi[kTopK];
#pragma unroll
    for (int i = 0; i < kTopK; ++i) {
        li[i] = lp[i * G];
        oi[i] = ld16(w.o + (((size_t)r * kTopK + i) * G + n) * kHeadDim + 8 * part);
    }
    const int npages = min(kTopK, ceil_div(row_lens[r], kBlock));
    float mx = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < kTopK; ++i) mx = (i < npages) ? fmaxf(mx, li[i]) : mx;
    float den = 0.f;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < kTopK; ++i) {
        const float wi = __expf(li[i] - mx);
        const bool ok = i < npages;
        den = ok ? den + wi : den;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc[2 * e] = ok ? acc[2 * e] + wi * bf16_lo(oi[i][e]) : acc[2 * e];
            acc[2 * e + 1] = ok ? acc[2 * e + 1] + wi * bf16_hi(oi[i][e]) : acc[2 * e + 1];
        }
    }
    const float inv = 1.0f / den;
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = pack2_bf16(acc[2 * e] * inv, acc[2 * e + 1] * inv);
    const int s = r / Hkv;
    const int h = (r % Hkv) * G + n;
    *reinterpret_cast<u32x4*>(out + ((size_t)s * Hq + h) * kHeadDim + 8 * part) = o;
    if (lse_out && part == 0) lse_out[(size_t)s * Hq + h] = mx + __logf(den);
}

hipError_t launch_merge(const MsaShape& s, const int32_t* row_lens, const void* ws, uint16_t* out,
                        float* lse, hipStream_t st) {
    const int R = s.B * s.Hkv;
    const int n = R * (s.Hq / s.Hkv) * 16;
    hipLaunchKernelGGL(decode_merge_kernel, dim3(ceil_div(n, kMergeThreads)), dim3(kMergeThreads),
                       0, st, row_lens, ws, out, lse, s.Hq, s.Hkv, R);
    return hipGetLastError();
}

}  // namespace
}  // namespace msa

size_t msa_decode_ws_bytes(const MsaShape& s) {
    using namespace msa;
    const size_t R = (size_t)s.B * s.Hkv;
    const size_t G = (size_t)(s.Hq / s.Hkv);
    const size_t bytes = R * kTopK * G * (kHeadDim * sizeof(uint16_t) + sizeof(float));
    return (bytes + 255) / 256 * 256;
}

hipError_t msa_launch_decode(const MsaShape& s, const uint16_t* q, const uint16_t* k_cache,
                             const uint16_t* v_cache, const int32_t* page_table,
                             const int32_t* row_lens, uint16_t* out, float* lse, void* ws,
                             hipStream_t st) {
    using namespace msa;
    const int R = s.B * s.Hkv;
    if (R == 0) return hipSuccess;
    const float scale_log2 = s.scale * kLog2e;
    hipLaunchKernelGGL(decode_page_kernel, dim3(kTopK, R), dim3(kDecThreads), 0, st, q, k_cache,
                       v_cache, page_table, row_lens, ws, s.Hq, s.Hkv, R, scale_log2);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_merge(s, row_lens, ws, out, lse, st);
}

namespace {
size_t align256(size_t x) { return (x + 255) / 256 * 256; }
}  // namespace

// Rows longer than this many blocks select in the standalone kernel (one
// 1024-thread workgroup per row) rather than inside the page workgroups.
constexpr int kFusedMaxBlocks = 32 * msa::kDecThreads;

// Workspace of the decode step: page partials, block scores, row lengths and,
// for rows past kFusedMaxBlocks, the selection and page table.
size_t msa_decode_step_ws_bytes(const MsaShape& s) {
    const size_t R = (size_t)s.B * s.Hkv;
    size_t bytes = msa_decode_ws_bytes(s) + align256(R * s.maxblk * sizeof(float)) +
                   align256(R * sizeof(int32_t));
    if (s.maxblk > kFusedMaxBlocks) bytes += 2 * align256(R * msa::kTopK * sizeof(int32_t));
    return bytes;
}

// Compute units, and the page workgroups the chip holds at once (LDS for four
// of 37.6 KB each per compute unit).
constexpr int kComputeUnits = 256;
constexpr int kResidentPageWorkgroups = kComputeUnits * 4;

template <int NPT, int W, bool PAGES>
static hipError_t launch_fused(const MsaShape& s, const float* scores, const int32_t* block_table,
                               const int32_t* seq_lens, const uint16_t* q, const uint16_t* k_cache,
                               const uint16_t* v_cache, int32_t* row_lens, int32_t* sel_out,
                               void* ws, hipStream_t st) {
    using namespace msa;
    const int R = s.B * s.Hkv;
#define MSA_MULTI(PPW)                                                                           \
    hipLaunchKernelGGL((decode_multi_kernel<NPT, W, PAGES, PPW>), dim3(kTopK / PPW, R),              \
                       dim3(kDecThreads), 0, st, scores, block_table, seq_lens, q, k_cache, v_cache, \
                       row_lens, sel_out, ws, s.Hq, s.Hkv, R, s.maxblk, s.scale * kLog2e)
    // One page per workgroup while every page workgroup fits on the chip at
    // once; past that, several slots per workgroup (one selection each), as
    // many as still leave two workgroups per compute unit.
    if (R * kTopK >= 8 * 2 * kComputeUnits) MSA_MULTI(8);
    else if (R * kTopK >= 4 * 2 * kComputeUnits) MSA_MULTI(4);
    else if (R * kTopK > kResidentPageWorkgroups) MSA_MULTI(2);
#undef MSA_MULTI
    else
        hipLaunchKernelGGL((decode_fused_kernel<NPT, W, PAGES>), dim3(kTopK, R),
                           dim3(kDecThreads), 0, st, scores, block_table, seq_lens, q, k_cache,
                           v_cache, row_lens, sel_out, ws, s.Hq, s.Hkv, R, s.maxblk,
                           s.scale * kLog2e);
    return hipGetLastError();
}

hipError_t msa_launch_decode_step(const MsaShape& s, const uint16_t* q_idx, const uint16_t* kidx,
                                  const uint16_t* q, const uint16_t* k_cache,
                                  const uint16_t* v_cache, const int32_t* block_table,
                                  const int32_t* seq_lens, uint16_t* out, float* lse,
                                  int32_t* sel_out, void* ws, const DecodeAppend* app,
                                  hipStream_t st) {
    using namespace msa;
    const int R = s.B * s.Hkv;
    if (R == 0) return hipSuccess;
    char* base = static_cast<char*>(ws);
    float* scores = reinterpret_cast<float*>(base + msa_decode_ws_bytes(s));
    int32_t* row_lens = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(scores) +
                                                   align256((size_t)R * s.maxblk * sizeof(float)));
    hipError_t e = msa_launch_index_score_decode(s, q_idx, kidx, block_table, seq_lens, scores, app, st);
    if (e != hipSuccess) return e;
    const int m = s.maxblk;
    if (m > kFusedMaxBlocks) {
        char* extra = reinterpret_cast<char*>(row_lens) + align256((size_t)R * sizeof(int32_t));
        int32_t* page_table = reinterpret_cast<int32_t*>(extra);
        int32_t* sel = sel_out ? sel_out
                               : reinterpret_cast<int32_t*>(extra + align256((size_t)R * kTopK * sizeof(int32_t)));
        e = msa_launch_topk(s, s.B, scores, seq_lens, nullptr, sel, st);
        if (e != hipSuccess) return e;
        e = msa_launch_page_table(s, sel, block_table, seq_lens, page_table, row_lens, st);
        if (e != hipSuccess) return e;
        return msa_launch_decode(s, q, k_cache, v_cache, page_table, row_lens, out, lse, ws, st);
    }
#define MSA_FUSED(NPT, W, PAGES) \
    launch_fused<NPT, W, PAGES>(s, scores, block_table, seq_lens, q, k_cache, v_cache, row_lens, sel_out, ws, st)
    if (m <= 4 * kWave) e = MSA_FUSED(4, 1, true);
    else if (m <= 8 * kWave) e = MSA_FUSED(8, 1, true);
    else if (m <= 16 * kWave) e = MSA_FUSED(16, 1, true);
    else if (m <= 8 * kDecThreads) e = MSA_FUSED(8, 4, true);
    else if (m <= 16 * kDecThreads) e = MSA_FUSED(16, 4, true);
    else e = MSA_FUSED(32, 4, false);
#undef MSA_FUSED
    if (e != hipSuccess) return e;
    return launch_merge(s, row_lens, ws, out, lse, st);
}
