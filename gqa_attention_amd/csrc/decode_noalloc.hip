// decode_noalloc.hip -- the decode workspace as a device array of the library itself, for
// callers that cannot allocate device memory (code under stream capture, serving loops
// that forbid allocation): gqa_attn_decode_noalloc runs the same split plan and kernels
// as gqa_attn_decode with this array as its workspace.
//
// The array is a file-scope __device__ variable, so every GPU the library runs on holds
// its own copy, at its own address, until the process ends.  Host code never uses the
// array's name as an address (on the host it only names the symbol): the first call on a
// device looks the device copy up with hipGetSymbolAddress, with that device current, and
// every later use goes through that pointer.  All calls on one GPU share its copy, so
// calls that overlap on one GPU race; the decode overwrites every byte it later reads, so
// nothing needs clearing between calls.
#include <mutex>

#include "gqa_launch.h"

namespace gqa {

constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;   // 16 MiB per device

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];   // device address of `scratch` on each device, once known

}  // namespace

size_t noalloc_scratch_bytes() { return kNoAllocScratchBytes; }

hipError_t noalloc_scratch(void **ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace gqa
