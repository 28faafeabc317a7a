// ttq_linear_noalloc: the whole-layer call for callers that cannot allocate
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).  Its workspace is a file-scope device array, `scratch`, of
// kNoallocScratchBytes; each GPU the library runs on holds its own copy until
// the process ends.  The array's device address is resolved once per device
// (hipGetSymbolAddress with that device current) and kept; host code only
// ever passes that address, never the array's name, to the kernels.
//
// Every call on a GPU shares that GPU's array and leaves its contents behind;
// nothing in ttq_linear needs zeroed scratch (no counters, no flags), so no
// clearing is required.  Calls that overlap on one GPU (different streams,
// or host threads without ordering) race on the array.
#include <atomic>
#include <mutex>

#include <hip/hip_runtime.h>

#include "ttq.h"
#include "launch.hpp"

constexpr size_t kNoallocScratchBytes = TTQ_NOALLOC_SCRATCH_BYTES;

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;

std::atomic<void*> g_ptr[kMaxDevices];
std::mutex g_init;

// The current device's copy of `scratch` (nullptr on failure).
void* scratch_ptr(int dev) {
    void* p = g_ptr[dev].load(std::memory_order_acquire);
    if (p != nullptr) return p;
    std::lock_guard<std::mutex> lock(g_init);
    p = g_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
        void* q = nullptr;
        if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        p = q;
        g_ptr[dev].store(p, std::memory_order_release);
    }
    return p;
}

}  // namespace

extern "C" ttq_status ttq_linear_noalloc(const ttq_linear_args* a, void* stream) {
    size_t need = 0;
    if (ttq_status e = ttq::linear_check(a, &need)) return e;
    if (need > kNoallocScratchBytes)
        return ttq::set_error(TTQ_ERR_INVALID,
                              "ttq_linear_noalloc: the layer needs more workspace than the library's "
                              "scratch array holds (TTQ_NOALLOC_SCRATCH_BYTES)");
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return ttq::set_error(TTQ_ERR_DEVICE, "ttq_linear_noalloc: no usable current device");
    void* ws = scratch_ptr(dev);
    if (ws == nullptr)
        return ttq::set_error(TTQ_ERR_DEVICE, "ttq_linear_noalloc: hipGetSymbolAddress of the scratch array failed");
    return ttq_linear(a, ws, kNoallocScratchBytes, stream);
}
