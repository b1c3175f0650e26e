// Fixed device scratch of the allocation-free decode entry point (nsa_decode_noalloc).
//
// The library never allocates device memory; its entry points take a caller workspace.
// For callers that cannot allocate one (work under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc) the decode step's scratch lives in a file-scope
// device array instead.  Every GPU the library runs on holds its own copy at its own
// address, from the code object's load until the process ends.  In host code the
// array's name stands for a host-side shadow, not a device address: the address is
// taken once per device with hipGetSymbolAddress (with that device current) and only
// that pointer is ever handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.hpp"

namespace nsa {

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;   // 64 MiB per device
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

}  // namespace

size_t static_scratch_bytes() { return kScratchBytes; }

// Device address of the current device's scratch array (resolved on the first call made
// with that device current, then cached).  Returns nullptr and sets *err on failure.
void* static_scratch(hipError_t* err) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        *err = e;
        return nullptr;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::call_once(g_once[dev], [dev]() {
        void* p = nullptr;
        g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_ptr[dev] = g_err[dev] == hipSuccess ? p : nullptr;
    });
    *err = g_err[dev];
    return g_ptr[dev];
}

}  // namespace nsa
