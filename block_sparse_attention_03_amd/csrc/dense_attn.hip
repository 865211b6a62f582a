// dense_attn.hip -- dense GQA decode attention: the comparison baseline for
// MSA's sparse decode.
//
// What it computes: every query head of sequence s attends all L_s cached
// tokens of its KV group, softmax(scale * q K^T) V, with the log-sum-exp.
// This is the "dense GQA with the same heads" that the youmind page's
// bullet "Rápido en producción" measures MSA's decode speedup against; the
// KV layout and the flattened (sequence, group) rows are those of the sparse
// path, so the two are compared on the same caches.
//
// Mapping.  A row r = s*H_kv + g is split into contiguous chunks of pages;
// one 256-thread workgroup per (chunk, row) walks its pages with the online
// softmax (running max and sum per head, output rescaled when the max grows),
// using the same page tile as the sparse kernel: the row's G heads are the 16
// columns of 16x16x32 bf16 matrix-core tiles, K arrives in contiguous pieces
// and reaches operand order through LDS, V is staged in LDS with coalesced
// loads and read back transposed; the next page's K and V are in flight while
// the current page is multiplied.
// Each chunk leaves a normalised partial output and its log-sum-exp; a second
// kernel merges a row's chunks with the Log-Sum-Exp rule.
#include "decode_tile.hpp"

namespace msa {
namespace {

// Pages per chunk: at least 4, and at most 64 chunks per row.
__host__ __device__ inline int dense_chunk_pages(int maxblk) {
    const int c = (maxblk + 63) / 64;
    return c < 4 ? 4 : c;
}

struct DenseWs {
    float* o;    // [R, chunks, G, 128] normalised partial outputs
    float* lse;  // [R, chunks, G]
};

__host__ __device__ inline DenseWs dense_ws(void* ws, int R, int chunks, int G) {
    DenseWs w;
    w.o = static_cast<float*>(ws);
    w.lse = w.o + (size_t)R * chunks * G * kHeadDim;
    return w;
}

// Three wavefronts per SIMD (at most 168 VGPRs) with the next page's K and V
// held in registers measured faster than two with more registers.
__global__ __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(3, 3)))
void dense_decode_kernel(const uint16_t* __restrict__ q,        // [B, Hq, 128]
                         const uint16_t* __restrict__ k_cache,  // [P, Hkv, 128, 128]
                         const uint16_t* __restrict__ v_cache,
                         const int32_t* __restrict__ block_table,  // [B, maxblk]
                         const int32_t* __restrict__ seq_lens,     // [B]
                         void* __restrict__ ws, int Hq, int Hkv, int R, int maxblk, int chunk,
                         int chunks, float scale_log2) {
    __shared__ __attribute__((aligned(16))) DecodeShared sh;
    const int c = blockIdx.x;
    const int r = blockIdx.y;
    const int s = r / Hkv;
    const int g = r % Hkv;
    const int L = seq_lens[s];
    const int npages = ceil_div(L, kBlock);
    const int p0 = c * chunk;
    const int p1 = min(npages, p0 + chunk);
    if (p0 >= p1) return;  // chunk past the sequence (uniform)
    const int G = Hq / Hkv;
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = tid % kWave;
    const int n = lane % 16;   // head column (B / result) or row of A
    const int kg = lane / 16;  // lane group

    // Q operands: head n of this group, zero beyond G
    bf16x8 qb[4];
    const uint16_t* qrow = q + ((size_t)s * Hq + g * G + n) * kHeadDim;
#pragma unroll
    for (int i = 0; i < 4; ++i) qb[i] = as_bf16x8(n < G ? ld16(qrow + 32 * i + 8 * kg) : u32x4{0u, 0u, 0u, 0u});

    float m_run = -__builtin_inff(), l_run = 0.f;  // per head n, in scaled-log2 units for m
    f32x4 o_run[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};

    // A page's K (contiguous 1 KB loads, see load_k_rows) and V (16 lanes per
    // 256-byte row), the whole page: pages are allocated in full, and loads
    // with no condition keep the compiler from waiting on them early.  Page
    // i + 1 is loaded while page i is in its softmax and products; its
    // block-table entry one page earlier still.
    const int32_t* bt = block_table + (size_t)s * maxblk;
    auto load_page = [&](int page, u32x4 (&kraw)[8], u32x4 (&vv)[8]) {
        const size_t off = ((size_t)page * Hkv + g) * kBlock * kHeadDim;
        load_k_rows(k_cache + off, wave, lane, kraw);
#pragma unroll
        for (int it = 0; it < 8; ++it)
            vv[it] = ld16_stream(v_cache + off + (tid / 16 + 16 * it) * kHeadDim + 8 * (tid % 16));
    };
    u32x4 kraw[8], vv[8];
    load_page(bt[p0], kraw, vv);
    int next_page = (p0 + 1 < p1) ? bt[p0 + 1] : 0;

    for (int pi = p0; pi < p1; ++pi) {
        const int nv = min(kBlock, L - pi * kBlock);
        __syncthreads();  // the previous page's LDS reads are done
        // K -> operands through this wavefront's quarter of the V tile
        bf16x8 ka[2][4];
        k_rows_to_operands(kraw, wave, lane, sh.vs, ka);

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
                sacc[j][rr] = (tok < nv) ? sacc[j][rr] * scale_log2 : -__builtin_inff();
                mx = fmaxf(mx, sacc[j][rr]);
            }
        mx = wave_max_xor(mx, 16);
        mx = wave_max_xor(mx, 32);
        if (kg == 0) sh.red_max[wave][n] = mx;
        // the maxima are visible and every wavefront has read its K out of the
        // V tile: V goes in (tokens at or past nv zero, so that P = 0 there
        // never meets a non-finite V), and the next page's loads go out
        __syncthreads();
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const int tok = tid / 16 + 16 * it;
            *reinterpret_cast<u32x4*>(sh.vs + vs_off(tok, 8 * (tid % 16))) =
                (tok < nv) ? vv[it] : u32x4{0u, 0u, 0u, 0u};
        }
        if (pi + 1 < p1) {  // uniform
            load_page(next_page, kraw, vv);
            next_page = (pi + 2 < p1) ? bt[pi + 2] : 0;
        }
        const float m_page = fmaxf(fmaxf(sh.red_max[0][n], sh.red_max[1][n]),
                                   fmaxf(sh.red_max[2][n], sh.red_max[3][n]));
        const float m_new = fmaxf(m_run, m_page);  // finite: every page has a valid token
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 on the first page
        // P = 2^(s - m_new) rounded to bf16; the sum uses the rounded values
        float sum = 0.f;
        uint16_t pb[2][4];
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                pb[j][rr] = f32_to_bf16(__builtin_amdgcn_exp2f(sacc[j][rr] - m_new));
                sum += bf16_to_f32(pb[j][rr]);
            }
        sum += __shfl_xor(sum, 16, kWave);
        sum += __shfl_xor(sum, 32, kWave);
        if (kg == 0) sh.red_sum[wave][n] = sum;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int tok = 32 * wave + 16 * j + 4 * kg;
            u32x2 w2 = {static_cast<uint32_t>(pb[j][0]) | (static_cast<uint32_t>(pb[j][1]) << 16),
                        static_cast<uint32_t>(pb[j][2]) | (static_cast<uint32_t>(pb[j][3]) << 16)};
            *reinterpret_cast<u32x2*>(sh.pl + n * kPStride + tok) = w2;
        }
        __syncthreads();

        // O^T += V^T P^T for dims 32w .. 32w+31 (see the sparse page kernel)
        f32x4 oacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int ta = 32 * ks + 4 * kg;
            const u32x2 p0v = *reinterpret_cast<const u32x2*>(sh.pl + n * kPStride + ta);
            const u32x2 p1v = *reinterpret_cast<const u32x2*>(sh.pl + n * kPStride + ta + 16);
            const bf16x8 pbv = as_bf16x8(u32x4{p0v[0], p0v[1], p1v[0], p1v[1]});
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                const uint16_t* src = sh.vs + vs_off(ta + n / 4, 32 * wave + 16 * mt + 4 * (n % 4));
                const u32x2 v0a = lds_read_tr16(src);
                const u32x2 v1a = lds_read_tr16(src + 16 * kHeadDim);  // token + 16: same swizzle
                oacc[mt] = mfma16(as_bf16x8(u32x4{v0a[0], v0a[1], v1a[0], v1a[1]}), pbv, oacc[mt]);
            }
        }
        const float l_page = sh.red_sum[0][n] + sh.red_sum[1][n] + sh.red_sum[2][n] + sh.red_sum[3][n];
        l_run = l_run * alpha + l_page;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) o_run[mt] = o_run[mt] * alpha + oacc[mt];
        m_run = m_new;
    }

    if (n < G) {
        DenseWs w = dense_ws(ws, R, chunks, G);
        const float inv = 1.0f / l_run;
        float* orow = w.o + (((size_t)r * chunks + c) * G + n) * kHeadDim;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            const int d = 32 * wave + 16 * mt + 4 * kg;
            *reinterpret_cast<f32x4*>(orow + d) = o_run[mt] * inv;
        }
        if (wave == 0 && kg == 0) w.lse[((size_t)r * chunks + c) * G + n] = m_run * kLn2 + __logf(l_run);
    }
}

// One thread per (row, head, dim): Log-Sum-Exp merge of the row's chunks (at
// most kDenseMaxChunks), every chunk's partial loaded together.
constexpr int kDenseMaxChunks = 64;
__global__ __launch_bounds__(kHeadDim)
void dense_merge_kernel(const int32_t* __restrict__ seq_lens, const void* __restrict__ ws,
                        uint16_t* __restrict__ out, float* __restrict__ lse_out, int Hq, int Hkv,
                        int R, int chunk, int chunks) {
    __shared__ float lse_s[kDenseMaxChunks];
    const int rn = blockIdx.x;  // r * G + n
    const int G = Hq / Hkv;
    const int r = rn / G;
    const int n = rn % G;
    const int d = threadIdx.x;
    const int s = r / Hkv;
    const int used = ceil_div(ceil_div(seq_lens[s], kBlock), chunk);  // chunks with pages
    const int last = max(used, 1) - 1;  // clamped index: every load in bounds
    DenseWs w = dense_ws(const_cast<void*>(ws), R, chunks, G);
    const float* lp = w.lse + (size_t)r * chunks * G + n;
    const float* op = w.o + ((size_t)r * chunks * G + n) * kHeadDim + d;
    float oi[kDenseMaxChunks];
#pragma unroll
    for (int i = 0; i < kDenseMaxChunks; ++i) oi[i] = op[(size_t)min(i, last) * G * kHeadDim];
    if (d < kDenseMaxChunks) lse_s[d] = lp[(size_t)min(d, last) * G];
    __syncthreads();
    float mx = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < kDenseMaxChunks; ++i) mx = (i < used) ? fmaxf(mx, lse_s[i]) : mx;
    float den = 0.f, acc = 0.f;
#pragma unroll
    for (int i = 0; i < kDenseMaxChunks; ++i) {
        const float wi = __expf(lse_s[i] - mx);
        den = (i < used) ? den + wi : den;
        acc = (i < used) ? __builtin_fmaf(wi, oi[i], acc) : acc;
    }
    const int h = (r % Hkv) * G + n;
    out[((size_t)s * Hq + h) * kHeadDim + d] = f32_to_bf16(acc / den);
    if (lse_out && d == 0) lse_out[(size_t)s * Hq + h] = mx + __logf(den);
}

}  // namespace
}  // namespace msa

size_t msa_dense_decode_ws_bytes(const MsaShape& s) {
    using namespace msa;
    const size_t R = (size_t)s.B * s.Hkv;
    const size_t G = (size_t)(s.Hq / s.Hkv);
    const int chunk = dense_chunk_pages(s.maxblk);
    const size_t chunks = (size_t)ceil_div(s.maxblk, chunk);
    const size_t bytes = R * chunks * G * (kHeadDim + 1) * sizeof(float);
    return (bytes + 255) / 256 * 256;
}

hipError_t msa_launch_dense_decode(const MsaShape& s, const uint16_t* q, const uint16_t* k_cache,
                                   const uint16_t* v_cache, const int32_t* block_table,
                                   const int32_t* seq_lens, uint16_t* out, float* lse, void* ws,
                                   hipStream_t st) {
    using namespace msa;
    const int R = s.B * s.Hkv;
    if (R == 0) return hipSuccess;
    const int G = s.Hq / s.Hkv;
    const int chunk = dense_chunk_pages(s.maxblk);
    const int chunks = ceil_div(s.maxblk, chunk);
    hipLaunchKernelGGL(dense_decode_kernel, dim3(chunks, R), dim3(kDecThreads), 0, st, q, k_cache,
                       v_cache, block_table, seq_lens, ws, s.Hq, s.Hkv, R, s.maxblk, chunk, chunks,
                       s.scale * kLog2e);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(dense_merge_kernel, dim3(R * G), dim3(kHeadDim), 0, st, seq_lens, ws, out,
                       lse, s.Hq, s.Hkv, R, chunk, chunks);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Dense causal prefill: the baseline for MSA's chunked-prefill speedup
// ---------------------------------------------------------------------------
//
// Query token t of sequence s (position p = L_s - nq_s + (t - q0_s)) attends
// every cached token j <= p of its group.  One 512-thread workgroup owns 256
// (query, head) rows of one (sequence, group) -- eight 32-row tiles, one per
// wavefront, rows ordered query-major with the group's G heads adjacent -- and
// walks the KV blocks 0 .. (its last row's own block), each block's K and V
// loaded once into LDS for all its rows, straight from global memory into the
// second of two buffers while the first is multiplied.  Per block and tile:
// S^T = K Q^T with 32x32x16 bf16 products, the causal cut where a row's own
// block is reached, the online softmax (running max and sum per row,
// accumulators rescaled), P rounded to bf16 as the B operand of
// O^T += V^T P^T with V^T from LDS transpose reads.  The output staging tiles
// reuse the K/V buffers after the last block.
namespace msa {
namespace {

constexpr int kDpThreads = 512;
constexpr int kDpRows = (kDpThreads / kWave) * 32;  // rows per workgroup (256)
constexpr int kDKStride = kHeadDim + 8;   // bf16 per output staging row (272 B)

// Two K/V block buffers, loaded straight from global memory into LDS: while
// block b is multiplied from one, block b + 1 arrives in the other.  Rows are
// unpadded (256 B); 16-byte chunk c of K token t sits at chunk c ^ (t mod 16)
// and of V token t at c ^ 2(t mod 8) (vs_off), which makes the K operand reads
// and the V transpose reads conflict-free.  Each lane of a direct load writes
// the 16 bytes at (instruction base + 16 lane), so the swizzle is chosen by
// which global chunk a lane reads.
struct DenseKV {
    uint16_t k[kBlock * kHeadDim];
    uint16_t v[kBlock * kHeadDim];
};
struct DenseShared {
    DenseKV buf[2];
};
static_assert((kDpThreads / kWave) * 32 * kDKStride * 2 <= (int)sizeof(DenseShared),
              "output staging fits over the K/V buffers");
__device__ __forceinline__ int dk_off(int t, int d) {  // bf16 offset of K (token t, dim d)
    return t * kHeadDim + ((((d >> 3) ^ (t & 15))) << 3) + (d & 7);
}

__device__ bool dense_row_chunk(const int32_t* __restrict__ cu_q, int B, int Hkv, int G, int id,
                                int* s_out, int* g_out, int* r0_out) {
    const int lane = __lane_id();
    int base = 0;
    for (int c0 = 0; c0 < B; c0 += kWave) {
        const int i = c0 + lane;
        const int nq = (i < B) ? (cu_q[i + 1] - cu_q[i]) : 0;
        const int per_group = ceil_div(nq * G, kDpRows);
        const int n = per_group * Hkv;
        int scan = n;  // inclusive prefix over lanes
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const int v = __shfl_up(scan, off, kWave);
            if (lane >= off) scan += v;
        }
        const uint64_t hit = __ballot(base + scan > id);
        if (hit) {
            const int first = __builtin_ctzll(hit);
            const int rem = id - base - __shfl(scan - n, first, kWave);
            const int pg = __shfl(per_group, first, kWave);
            *s_out = c0 + first;
            *g_out = rem / pg;
            *r0_out = (rem % pg) * kDpRows;
            return true;
        }
        base += __shfl(scan, kWave - 1, kWave);
    }
    return false;
}

__global__ __launch_bounds__(kDpThreads, 1)
void dense_prefill_kernel(const uint16_t* __restrict__ q,        // [T, Hq, 128]
                          const uint16_t* __restrict__ k_cache,  // [P, Hkv, 128, 128]
                          const uint16_t* __restrict__ v_cache,
                          const int32_t* __restrict__ block_table,
                          const int32_t* __restrict__ seq_lens,
                          const int32_t* __restrict__ cu_q, uint16_t* __restrict__ out,
                          float* __restrict__ lse_out, int B, int Hq, int Hkv, int maxblk,
                          float scale_log2) {
    __shared__ __attribute__((aligned(16))) DenseShared sh;
    __shared__ int info[3];
    const int G = Hq / Hkv;
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = tid % kWave;
    if (wave == 0) {
        int s_, g_, r0_;
        const bool ok = dense_row_chunk(cu_q, B, Hkv, G, blockIdx.x, &s_, &g_, &r0_);
        if (lane == 0) {
            info[0] = ok ? s_ : -1;
            info[1] = g_;
            info[2] = r0_;
        }
    }
    __syncthreads();
    const int s = info[0];
    if (s < 0) return;  // uniform
    const int g = info[1];
    const int q0 = cu_q[s];
    const int nq = cu_q[s + 1] - q0;
    const int L = seq_lens[s];
    const int nrows = nq * G;
    const int wg_row0 = info[2];
    const int n = lane % 32;  // row of this lane within the wave's tile
    const int h = lane / 32;  // lane half

    // this lane's row (rows past the sequence repeat its last row; results discarded)
    const int rho0 = wg_row0 + wave * 32 + n;
    const bool row_ok = rho0 < nrows;
    const int rho = row_ok ? rho0 : nrows - 1;
    const int t = q0 + rho / G;
    const int head = g * G + rho % G;
    const int p = L - nq + rho / G;
    const int last_row = min(wg_row0 + kDpRows, nrows) - 1;
    const int b_last = (L - nq + last_row / G) / kBlock;  // the workgroup's last block

    // K/V block -> LDS buffer: wavefront w's four direct loads per tile fill
    // its 16-byte chunks 256w .. 256w + 255 (tokens 16w .. 16w + 15); lane l
    // of load j fills chunk position l % 16 of token (256w + 64j + l) / 16 and
    // so reads that token's global chunk (l % 16) ^ swizzle
    const int32_t* bt = block_table + (size_t)s * maxblk;
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    auto load_block = [&](int page, DenseKV& dst) {
        const size_t page_off = ((size_t)page * Hkv + g) * kBlock * kHeadDim;
        const uint16_t* kp = k_cache + page_off;
        const uint16_t* vp = v_cache + page_off;
#pragma unroll
        for (int jl = 0; jl < 4; ++jl) {
            const int chunk0 = (wv * 4 + jl) * kWave;  // first 16-byte chunk of this load
            const int tok = (chunk0 + lane) / 16, pos = lane % 16;
            __builtin_amdgcn_global_load_lds(
                kp + tok * kHeadDim + 8 * (pos ^ (tok & 15)),
                (__attribute__((address_space(3))) void*)(dst.k + chunk0 * 8), 16, 0, 0);
            __builtin_amdgcn_global_load_lds(
                vp + tok * kHeadDim + 8 * (pos ^ ((tok & 7) << 1)),
                (__attribute__((address_space(3))) void*)(dst.v + chunk0 * 8), 16, 0, 0);
        }
    };
    load_block(bt[0], sh.buf[0]);
    int next_page = (b_last >= 1) ? bt[1] : 0;

    // Q: B operands straight from the row (k-step i of lane half h: dims
    // 64h + 8i .. +7)
    bf16x8 qb[8];
    {
        const uint16_t* qrow = q + ((size_t)t * Hq + head) * kHeadDim + 64 * h;
#pragma unroll
        for (int i = 0; i < 8; ++i) qb[i] = as_bf16x8(ld16(qrow + 8 * i));
    }

    float m_run = -__builtin_inff();  // running max of this lane's row, scaled log2 units
    float l_run = 0.f;
    f32x16 o_run[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) o_run[mt] = f32x16{};
    const int j = lane % 16;

    for (int b = 0; b <= b_last; ++b) {
        DenseKV& cur = sh.buf[b & 1];
        // s_waitcnt immediate: vector-memory count 0, other counters free
        __builtin_amdgcn_s_waitcnt(0x0F70);  // this wavefront's loads of block b are in LDS ...
        __syncthreads();  // ... and every wavefront's; block b - 1's buffer is free
        const int nv = min(kBlock, L - b * kBlock);
        if (nv < kBlock) {  // uniform: the sequence's partial last block
            // V rows past the cache's tokens -> 0, so that P = 0 there never
            // meets a non-finite value (K rows there are masked: they are past
            // every row's position)
            for (int c = tid; c < (kBlock - nv) * (kHeadDim / 8); c += kDpThreads)
                *reinterpret_cast<u32x4*>(cur.v + (nv + c / 16) * kHeadDim + 8 * (c % 16)) =
                    u32x4{0u, 0u, 0u, 0u};
            __syncthreads();
        }
        if (b < b_last) {  // uniform: block b + 1 arrives while block b is multiplied
            load_block(next_page, sh.buf[(b + 1) & 1]);
            next_page = (b + 2 <= b_last) ? bt[b + 2] : 0;
        }

        // S^T = K Q^T: tile mt = tokens 32mt..32mt+31; value v of the lane is
        // token 32mt + 8(v/4) + 4h + v%4 of row n
        f32x16 sacc[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            sacc[mt] = f32x16{};
#pragma unroll
            for (int i = 0; i < 8; ++i)
                sacc[mt] = mfma32(as_bf16x8(*reinterpret_cast<const u32x4*>(
                                      cur.k + dk_off(32 * mt + n, 64 * h + 8 * i))),
                                  qb[i], sacc[mt]);
        }
        // causal cut: token b*128 + tk visible iff <= p (all of a block before
        // the row's own block is visible)
        const int lim = p - b * kBlock;
        if (__ballot(lim < kBlock - 1)) {
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
        // block 0 always holds token 0 <= p, so m_new is finite from the first block on
        const float m_new = fmaxf(m_run, mx * scale_log2);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 on block 0

        // P (bf16) as the B operand: k-step i covers tokens 16i..16i+15, i.e.
        // accumulator values 8(i%2)..8(i%2)+7 of S^T tile i/2; the row sum uses
        // the rounded weights the product uses
        bf16x8 pb[8];
        float sum = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            u32x4 pw;
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                const float p0 = __builtin_amdgcn_exp2f(sacc[i / 2][8 * (i % 2) + 2 * e2] * scale_log2 - m_new);
                const float p1 = __builtin_amdgcn_exp2f(sacc[i / 2][8 * (i % 2) + 2 * e2 + 1] * scale_log2 - m_new);
                pw[e2] = pack2_bf16(p0, p1);
                sum += bf16_lo(pw[e2]) + bf16_hi(pw[e2]);
            }
            pb[i] = as_bf16x8(pw);
        }
        sum += __shfl_xor(sum, 32, kWave);
        l_run = l_run * alpha + sum;
        m_run = m_new;

        // O^T = alpha O^T + V^T P^T; dim tile mt: the A operand is the same
        // tokens of dims 32mt + n from transpose reads of row-major V
        // (tokens 16i + 4h + j/4 and 8 later, dims 32mt + 16((lane/16) % 2) +
        // 4(j % 4): 4 dims of one 16-byte chunk, swizzled by token as vs_off)
        const int vt = 4 * h + j / 4;
        const int vd = 16 * ((lane / 16) % 2) + 4 * (j % 4);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            f32x16 acc = o_run[mt] * alpha;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const u32x2 a0 = lds_read_tr16(cur.v + vs_off(16 * i + vt, 32 * mt + vd));
                const u32x2 a1 = lds_read_tr16(cur.v + vs_off(16 * i + 8 + vt, 32 * mt + vd));
                acc = mfma32(as_bf16x8(u32x4{a0[0], a0[1], a1[0], a1[1]}), pb[i], acc);
            }
            o_run[mt] = acc;
        }
    }

    // normalised output: O^T fragments -> staging tile (row n, padded rows,
    // over the K/V buffers) -> coalesced 16-byte stores of 4 rows x 256 bytes
    // per instruction
    __syncthreads();  // every wave is done with the last block's K/V
    uint16_t* tbuf = reinterpret_cast<uint16_t*>(&sh) + wave * 32 * kDKStride;
    const float inv = 1.0f / l_run;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
            const int d = 32 * mt + 8 * qd + 4 * h;
            *reinterpret_cast<u32x2*>(tbuf + n * kDKStride + d) =
                u32x2{pack2_bf16(o_run[mt][4 * qd + 0] * inv, o_run[mt][4 * qd + 1] * inv),
                      pack2_bf16(o_run[mt][4 * qd + 2] * inv, o_run[mt][4 * qd + 3] * inv)};
        }
    __builtin_amdgcn_wave_barrier();
    const int orow = row_ok ? t * Hq + head : -1;
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const int r = lane / 16 + 4 * it;
        const int o = __shfl(orow, r, kWave);
        const u32x4 v = *reinterpret_cast<const u32x4*>(tbuf + r * kDKStride + 8 * (lane % 16));
        if (o >= 0) *reinterpret_cast<u32x4*>(out + (size_t)o * kHeadDim + 8 * (lane % 16)) = v;
    }
    if (lse_out && row_ok && h == 0) lse_out[(size_t)t * Hq + head] = m_run * kLn2 + __logf(l_run);
}

}  // namespace
}  // namespace msa

hipError_t msa_launch_dense_prefill(const MsaShape& s, int total_q, const uint16_t* q,
                                    const uint16_t* k_cache, const uint16_t* v_cache,
                                    const int32_t* block_table, const int32_t* seq_lens,
                                    const int32_t* cu_q, uint16_t* out, float* lse,
                                    hipStream_t st) {
    using namespace msa;
    if (total_q == 0) return hipSuccess;
    const int G = s.Hq / s.Hkv;
    // upper bound on the row chunks: sum_s H_kv ceil(nq_s G / 128) <= H_kv (total_q G / 128 + B)
    const int64_t chunks = (int64_t)s.Hkv * (ceil_div(total_q * G, kDpRows) + s.B);
    hipLaunchKernelGGL(dense_prefill_kernel, dim3((unsigned)chunks), dim3(kDpThreads), 0, st, q,
                       k_cache, v_cache, block_table, seq_lens, cu_q, out, lse, s.B, s.Hq, s.Hkv,
                       s.maxblk, s.scale * kLog2e);
    return hipGetLastError();
}
