// static_scratch.hip -- the library's own device scratch, for the one entry
// point that takes no workspace (msa_decode_step_noalloc): callers that cannot
// allocate device memory (code under graph capture, serving loops that forbid
// allocation) still get the decode step's partials, block scores and row
// lengths.
//
// The array lives in the code object, so every GPU the library runs on holds
// its own copy at its own address from the first use until the process ends.
// In host code `scratch` names a host-side stand-in, not that address: the
// device address is looked up once per device with hipGetSymbolAddress (with
// that device current) and cached; only the cached pointer is ever handed to
// kernels.
#include <mutex>

#include "msa.h"
#include "msa_common.hpp"

static __device__ __align__(256) unsigned char scratch[MSA_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];  // device address of `scratch` per device, once looked up

}  // namespace

size_t msa_static_scratch_bytes() { return sizeof(scratch); }

// Device address of this GPU's scratch array for work enqueued on `st`: the
// array of the stream's device (the current device for the null stream).
// The lookup runs once per device, with that device made current for the
// call and the caller's current device restored after it.
hipError_t msa_static_scratch(hipStream_t st, void** out) {
    hipDevice_t dev = -1;
    hipError_t e = st ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        int cur = -1;
        if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return hipSuccess;
}
