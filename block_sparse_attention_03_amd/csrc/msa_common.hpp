// msa_common.hpp -- shared device helpers of the MSA HIP kernels (gfx950).
//
// Vector types for the CDNA4 bf16 matrix-core builtins, bf16 <-> fp32
// conversion, wavefront helpers, and the internal launcher declarations used
// by msa_api.cpp.  Nothing here is part of the public C ABI (include/msa.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

constexpr int kWave = 64;        // CDNA wavefront width
constexpr int kBlock = 128;      // Bk: tokens per KV block (= page)
constexpr int kHeadDim = 128;    // D
constexpr int kIdxDim = 64;      // d
constexpr int kTopK = 16;        // k
constexpr int kMaxGroup = 16;    // G = H_q / H_kv handled by one matrix-core tile

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even fp32 -> bf16 bits (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    __bf16 h = static_cast<__bf16>(f);
    return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ u32x4 ld16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

// 16-byte load of data that is read once (K/V pages, index keys): the
// nontemporal hint keeps it from displacing reusable lines in the caches.
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> two bf16 (RNE) in one 32-bit word, low half first.
__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// 8 fp32 -> 8 bf16 (RNE) packed for a matrix-core operand.
__device__ __forceinline__ bf16x8 pack_bf16x8(float a0, float a1, float a2, float a3, float a4,
                                              float a5, float a6, float a7) {
    bf16x8 r;
    r[0] = static_cast<__bf16>(a0);
    r[1] = static_cast<__bf16>(a1);
    r[2] = static_cast<__bf16>(a2);
    r[3] = static_cast<__bf16>(a3);
    r[4] = static_cast<__bf16>(a4);
    r[5] = static_cast<__bf16>(a5);
    r[6] = static_cast<__bf16>(a6);
    r[7] = static_cast<__bf16>(a7);
    return r;
}

// D(16x16, fp32) += A(16x32) * B(32x16).  Lane l supplies A row l%16 and
// B column l%16, each with 8 consecutive reduction-index values of lane group
// l/16; the result holds D[4*(l/16) + r][l%16] for r = 0..3.  Callers feed A
// and B through the same (lane, element) -> reduction-index map, so the
// product does not depend on how the hardware orders that index.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// D(32x32, fp32) += A(32x16) * B(16x32).  Lane l supplies A row l%32 and B
// column l%32 with 8 reduction-index values of lane half l/32; the result
// holds D[8*(v/4) + 4*(l/32) + v%4][l%32] for v = 0..15.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// LDS transpose read (gfx950 ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane j supplies the LDS address of 4 consecutive bf16 values; lane i
// receives element i%4 of the values supplied by lanes i/4, i/4+4, i/4+8 and
// i/4+12 (in that order).  With lane j pointing at row R0 + j/4, columns
// C0 + 4*(j%4) .. +3 of a row-major tile, lane i therefore receives column
// C0 + i of rows R0 .. R0+3: a column slice, i.e. the transposed operand.
typedef short i16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* lds_ptr) {
    i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(lds_ptr));
    return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ float wave_max_xor(float v, int mask) {
    return fmaxf(v, __shfl_xor(v, mask, kWave));
}

// Number of set bits of `m` in lanes below this one.
__device__ __forceinline__ int mbcnt(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                     __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0));
}

__host__ __device__ constexpr int ceil_div(int a, int b) { return (a + b - 1) / b; }

}  // namespace msa

// ---------------------------------------------------------------------------
// Internal launchers (defined in the .hip files, called by msa_api.cpp).
// Each returns hipSuccess or the launch error.
// ---------------------------------------------------------------------------
struct MsaShape {
    int B, Hq, Hkv, Hidx, maxblk, num_pages;
    float scale;  // resolved softmax scale (> 0)
};

hipError_t msa_launch_append_kv(const MsaShape& s, int total_q, const uint16_t* k_new,
                                const uint16_t* v_new, const uint16_t* kidx_new,
                                const int32_t* block_table, const int32_t* seq_lens,
                                const int32_t* cu_q, uint16_t* k_cache, uint16_t* v_cache,
                                uint16_t* kidx_cache, hipStream_t st);
hipError_t msa_launch_validate(const MsaShape& s, int total_q, const int32_t* block_table,
                               const int32_t* seq_lens, const int32_t* cu_q, int32_t* status,
                               hipStream_t st);
hipError_t msa_launch_index_score(const MsaShape& s, int total_q, const uint16_t* q_idx,
                                  const uint16_t* kidx, const int32_t* block_table,
                                  const int32_t* seq_lens, const int32_t* cu_q, float* scores,
                                  hipStream_t st);
hipError_t msa_launch_topk(const MsaShape& s, int total_q, const float* scores,
                           const int32_t* seq_lens, const int32_t* cu_q, int32_t* sel,
                           hipStream_t st);
hipError_t msa_launch_page_table(const MsaShape& s, const int32_t* sel,
                                 const int32_t* block_table, const int32_t* seq_lens,
                                 int32_t* page_table, int32_t* row_lens, hipStream_t st);
size_t msa_decode_ws_bytes(const MsaShape& s);
hipError_t msa_launch_decode(const MsaShape& s, const uint16_t* q, const uint16_t* k_cache,
                             const uint16_t* v_cache, const int32_t* page_table,
                             const int32_t* row_lens, uint16_t* out, float* lse, void* ws,
                             hipStream_t st);
size_t msa_prefill_ws_bytes(const MsaShape& s, int total_q);
size_t msa_multi_query_ws_bytes(const MsaShape& s, int total_q);
hipError_t msa_launch_multi_query_step(const MsaShape& s, int total_q, const uint16_t* q_idx,
                                       const uint16_t* kidx, const uint16_t* q,
                                       const uint16_t* k_cache, const uint16_t* v_cache,
                                       const int32_t* block_table, const int32_t* seq_lens,
                                       const int32_t* cu_q, uint16_t* out, float* lse,
                                       int32_t* sel_out, void* ws, hipStream_t st);
hipError_t msa_launch_prefill(const MsaShape& s, int total_q, const uint16_t* q,
                              const uint16_t* k_cache, const uint16_t* v_cache,
                              const int32_t* block_table, const int32_t* seq_lens,
                              const int32_t* cu_q, const int32_t* sel, uint16_t* out, float* lse,
                              void* ws, hipStream_t st);
// The new decode tokens (one per sequence) that a decode step writes into the
// caches while it scores.
struct DecodeAppend {
    const uint16_t* k_new;     // [B, Hkv, 128]
    const uint16_t* v_new;     // [B, Hkv, 128]
    const uint16_t* kidx_new;  // [B, Hidx, 64]
    uint16_t* k_cache;
    uint16_t* v_cache;
    uint16_t* kidx_cache;
};
hipError_t msa_launch_index_score_decode(const MsaShape& s, const uint16_t* q_idx,
                                         const uint16_t* kidx, const int32_t* block_table,
                                         const int32_t* seq_lens, float* scores,
                                         const DecodeAppend* app, hipStream_t st);
size_t msa_dense_decode_ws_bytes(const MsaShape& s);
hipError_t msa_launch_dense_decode(const MsaShape& s, const uint16_t* q, const uint16_t* k_cache,
                                   const uint16_t* v_cache, const int32_t* block_table,
                                   const int32_t* seq_lens, uint16_t* out, float* lse, void* ws,
                                   hipStream_t st);
hipError_t msa_launch_dense_prefill(const MsaShape& s, int total_q, const uint16_t* q,
                                    const uint16_t* k_cache, const uint16_t* v_cache,
                                    const int32_t* block_table, const int32_t* seq_lens,
                                    const int32_t* cu_q, uint16_t* out, float* lse,
                                    hipStream_t st);
size_t msa_decode_step_ws_bytes(const MsaShape& s);
hipError_t msa_launch_decode_step(const MsaShape& s, const uint16_t* q_idx, const uint16_t* kidx,
                                  const uint16_t* q, const uint16_t* k_cache,
                                  const uint16_t* v_cache, const int32_t* block_table,
                                  const int32_t* seq_lens, uint16_t* out, float* lse,
                                  int32_t* sel_out, void* ws, const DecodeAppend* app,
                                  hipStream_t st);
// The library's static device scratch (static_scratch.hip): its size, and its
// device address on the device of `st`, looked up once per device.
size_t msa_static_scratch_bytes();
hipError_t msa_static_scratch(hipStream_t st, void** out);
