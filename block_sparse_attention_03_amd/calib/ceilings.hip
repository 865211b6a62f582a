// ceilings.hip -- measured ceilings for the roofline fractions: a streaming
// HBM read, a device copy (reads and writes at once) and a bf16 matrix-core
// loop on MI355X (gfx950), each in the forms that probes found fastest.  Not part of the
// MSA library: the benchmark loads this separate libmsa_calib.so to report
// achieved bandwidth and FLOP rate against what the chip actually sustains,
// next to the published peaks.
#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;

// The sink store depends on every load, so none can be dropped; it runs only
// if the XOR of a thread's words equals this value, which never happens for
// the zero-filled buffers the benchmark reads, so the reads are the only
// traffic.
constexpr uint32_t kNever = 0x12345678u;

// Every 16-byte chunk of buf read once with streaming (non-temporal) loads,
// eight in flight per thread, grid-stride.
__global__ __launch_bounds__(kThreads) void read_kernel(const u32x4* __restrict__ buf, size_t n16,
                                                        uint32_t* __restrict__ sink) {
    const size_t stride = (size_t)gridDim.x * kThreads;
    size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 7 * stride < n16; i += 8 * stride) {
        u32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(buf + i + u * stride);
#pragma unroll
        for (int u = 0; u < 8; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    for (; i < n16; i += stride) {
        const u32x4 v = __builtin_nontemporal_load(buf + i);
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    if (acc == kNever) sink[(size_t)blockIdx.x * kThreads + threadIdx.x] = acc;
}

// Workgroup b reads the chunk [b chunk, (b + 1) chunk) of 16-byte units, four
// loads in flight per thread: many short-lived workgroups, the form that
// streams fastest on this chip.
__global__ __launch_bounds__(kThreads) void read_chunk_kernel(const u32x4* __restrict__ buf,
                                                              size_t n16, size_t chunk,
                                                              uint32_t* __restrict__ sink) {
    const size_t b0 = (size_t)blockIdx.x * chunk;
    const size_t b1 = b0 + chunk < n16 ? b0 + chunk : n16;
    size_t i = b0 + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 3 * kThreads < b1; i += 4 * kThreads) {
        u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(buf + i + u * kThreads);
#pragma unroll
        for (int u = 0; u < 4; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    for (; i < b1; i += kThreads) {
        const u32x4 v = __builtin_nontemporal_load(buf + i);
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    if (acc == kNever) sink[threadIdx.x] = acc;
}

// dst = src by chunks as read_chunk_kernel reads, with streaming stores.
__global__ __launch_bounds__(kThreads) void copy_chunk_kernel(const u32x4* __restrict__ src,
                                                              u32x4* __restrict__ dst, size_t n16,
                                                              size_t chunk) {
    const size_t b0 = (size_t)blockIdx.x * chunk;
    const size_t b1 = b0 + chunk < n16 ? b0 + chunk : n16;
    size_t i = b0 + threadIdx.x;
    for (; i + 3 * kThreads < b1; i += 4 * kThreads) {
        u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(src + i + u * kThreads);
#pragma unroll
        for (int u = 0; u < 4; ++u) __builtin_nontemporal_store(v[u], dst + i + u * kThreads);
    }
    for (; i < b1; i += kThreads) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// dst = src, 16-byte chunks with streaming loads, eight in flight per thread:
// the rate of traffic that is half reads and half writes.
__global__ __launch_bounds__(kThreads) void copy_kernel(const u32x4* __restrict__ src,
                                                        u32x4* __restrict__ dst, size_t n16) {
    const size_t stride = (size_t)gridDim.x * kThreads;
    size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
    for (; i + 7 * stride < n16; i += 8 * stride) {
        u32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < 8; ++u) dst[i + u * stride] = v[u];
    }
    for (; i < n16; i += stride) dst[i] = __builtin_nontemporal_load(src + i);
}

// Four independent chains of 32x32x16 bf16 products per wavefront, iters
// rounds: the matrix core's sustained rate with 4 waves per SIMD.
__global__ __launch_bounds__(kThreads) void mfma_kernel(float* __restrict__ out, int iters) {
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(0.001f * (threadIdx.x + i));
        b[i] = (__bf16)(0.002f * (blockIdx.x % 7 - i));
    }
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < iters; ++it) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
    out[(size_t)blockIdx.x * kThreads + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Workgroups of the read kernel; sink must hold msa_calib_read_sink_len() words.
int msa_calib_read_blocks(void) { return 4096; }
size_t msa_calib_read_sink_len(void) { return (size_t)4096 * kThreads; }

// Streams `bytes` (a multiple of 16) of device memory at buf.  Returns a
// hipError_t value (0 = launched).
int msa_calib_read(const void* buf, size_t bytes, uint32_t* sink, size_t sink_len, void* stream) {
    if (!buf || !sink || bytes % 16 != 0 || sink_len < msa_calib_read_sink_len())
        return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(read_kernel, dim3(msa_calib_read_blocks()), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4*>(buf), bytes / 16,
                       sink);
    return (int)hipGetLastError();
}

// The same read with `blocks` workgroups (1 .. msa_calib_read_blocks()), for
// reads of a few tens of MB where the grid size sets how fast the chip fills.
int msa_calib_read_grid(const void* buf, size_t bytes, int blocks, uint32_t* sink, size_t sink_len,
                        void* stream) {
    if (!buf || !sink || bytes % 16 != 0 || blocks <= 0 || blocks > msa_calib_read_blocks() ||
        sink_len < msa_calib_read_sink_len())
        return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(read_kernel, dim3(blocks), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4*>(buf), bytes / 16,
                       sink);
    return (int)hipGetLastError();
}

// Copies `bytes` (a multiple of 16) from src to dst (not overlapping) with
// `blocks` workgroups (1 .. msa_calib_read_blocks()).
int msa_calib_copy_grid(const void* src, void* dst, size_t bytes, int blocks, void* stream) {
    if (!src || !dst || bytes % 16 != 0 || blocks <= 0 || blocks > msa_calib_read_blocks())
        return (int)hipErrorInvalidValue;
    const char* a = static_cast<const char*>(src);
    const char* b = static_cast<const char*>(dst);
    if (a < b + bytes && b < a + bytes) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(copy_kernel, dim3(blocks), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src),
                       static_cast<u32x4*>(dst), bytes / 16);
    return (int)hipGetLastError();
}

// Streams `bytes` (a multiple of 16) at buf, one workgroup per `chunk_bytes`
// (a multiple of 16, at least 4096) of it.
int msa_calib_read_chunked(const void* buf, size_t bytes, size_t chunk_bytes, uint32_t* sink,
                           size_t sink_len, void* stream) {
    if (!buf || !sink || bytes % 16 != 0 || chunk_bytes % 16 != 0 || chunk_bytes < 4096 ||
        sink_len < (size_t)kThreads)
        return (int)hipErrorInvalidValue;
    const size_t chunk = chunk_bytes / 16;
    const size_t grid = (bytes / 16 + chunk - 1) / chunk;
    if (grid == 0) return 0;
    if (grid > 0x7FFFFFFF) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(read_chunk_kernel, dim3((unsigned)grid), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4*>(buf), bytes / 16,
                       chunk, sink);
    return (int)hipGetLastError();
}

// Copies `bytes` from src to dst (not overlapping), one workgroup per
// `chunk_bytes` (as msa_calib_read_chunked).
int msa_calib_copy_chunked(const void* src, void* dst, size_t bytes, size_t chunk_bytes,
                           void* stream) {
    if (!src || !dst || bytes % 16 != 0 || chunk_bytes % 16 != 0 || chunk_bytes < 4096)
        return (int)hipErrorInvalidValue;
    const char* a = static_cast<const char*>(src);
    const char* b = static_cast<const char*>(dst);
    if (a < b + bytes && b < a + bytes) return (int)hipErrorInvalidValue;
    const size_t chunk = chunk_bytes / 16;
    const size_t grid = (bytes / 16 + chunk - 1) / chunk;
    if (grid == 0) return 0;
    if (grid > 0x7FFFFFFF) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(copy_chunk_kernel, dim3((unsigned)grid), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src),
                       static_cast<u32x4*>(dst), bytes / 16, chunk);
    return (int)hipGetLastError();
}

// bf16 FLOP of one msa_calib_mfma launch of `blocks` workgroups.
double msa_calib_mfma_flop(int blocks, int iters) {
    return (double)blocks * (kThreads / 64) * iters * 4 * (32.0 * 32.0 * 16.0 * 2.0);
}

// out must hold blocks * 256 floats.
int msa_calib_mfma(float* out, int blocks, int iters, void* stream) {
    if (!out || blocks <= 0 || iters <= 0) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(mfma_kernel, dim3(blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       out, iters);
    return (int)hipGetLastError();
}

}  // extern "C"
