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
// columns of 16x16x32 bf16 matrix-core tiles, K operands come straight from
// HBM, V is staged in LDS with coalesced loads and read back transposed.
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

__global__ __launch_bounds__(kDecThreads)
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

    for (int pi = p0; pi < p1; ++pi) {
        const int nv = min(kBlock, L - pi * kBlock);
        const int page = block_table[(size_t)s * maxblk + pi];
        const size_t page_off = ((size_t)page * Hkv + g) * kBlock * kHeadDim;
        const uint16_t* kp = k_cache + page_off;
        const uint16_t* vp = v_cache + page_off;
        __syncthreads();  // the previous page's LDS reads are done
        u32x4 vv[8];
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const int tok = tid / 16 + 16 * it;
            vv[it] = (tok < nv) ? ld16_stream(vp + tok * kHeadDim + 8 * (tid % 16)) : u32x4{0u, 0u, 0u, 0u};
        }
        bf16x8 ka[2][4];
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                ka[j][i] = as_bf16x8(ld16_stream(kp + (32 * wave + 16 * j + n) * kHeadDim + 32 * i + 8 * kg));
#pragma unroll
        for (int it = 0; it < 8; ++it)
            *reinterpret_cast<u32x4*>(sh.vs + vs_off(tid / 16 + 16 * it, 8 * (tid % 16))) = vv[it];

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
        __syncthreads();
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

// One thread per (row, head, dim): Log-Sum-Exp merge of the row's chunks.
__global__ __launch_bounds__(kHeadDim)
void dense_merge_kernel(const int32_t* __restrict__ seq_lens, const void* __restrict__ ws,
                        uint16_t* __restrict__ out, float* __restrict__ lse_out, int Hq, int Hkv,
                        int R, int chunk, int chunks) {
    const int rn = blockIdx.x;  // r * G + n
    const int G = Hq / Hkv;
    const int r = rn / G;
    const int n = rn % G;
    const int d = threadIdx.x;
    const int s = r / Hkv;
    const int used = ceil_div(ceil_div(seq_lens[s], kBlock), chunk);  // chunks with pages
    DenseWs w = dense_ws(const_cast<void*>(ws), R, chunks, G);
    const float* lp = w.lse + (size_t)r * chunks * G + n;
    const float* op = w.o + ((size_t)r * chunks * G + n) * kHeadDim + d;
    float mx = -__builtin_inff();
    for (int i = 0; i < used; ++i) mx = fmaxf(mx, lp[(size_t)i * G]);
    float den = 0.f, acc = 0.f;
    for (int i = 0; i < used; ++i) {
        const float wi = __expf(lp[(size_t)i * G] - mx);
        den += wi;
        acc += wi * op[(size_t)i * G * kHeadDim];
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
