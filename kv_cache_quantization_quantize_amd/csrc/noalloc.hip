// noalloc.hip -- the workspace of kivi_decode_attend_noalloc: a device array
// the library owns, for callers that cannot allocate (code under graph
// capture, tight serving loops, harnesses that forbid hipMalloc).  The array
// is part of the library's code object, so every GPU the library runs on
// holds its own copy from the moment the code object loads until the
// process ends; nothing is allocated at call time.
#include <mutex>

#include "kivi_launch.h"

namespace kivi {

namespace {

constexpr size_t kScratchBytes = size_t{32} << 20;          // 32 MiB per GPU

// In host code `scratch` names a host-side stand-in, not device memory: its
// device address comes from hipGetSymbolAddress (per device, below), and
// only that address may reach a kernel.
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void* g_scratch[kMaxDevices];                                // per device, once resolved

}  // namespace

size_t static_attend_scratch_bytes() { return kScratchBytes; }

hipError_t static_attend_scratch(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> guard(g_lock);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch[dev] = p;
    }
    *ptr = g_scratch[dev];
    return hipSuccess;
}

}  // namespace kivi
