// Scratch of the no-allocation prefill entry point (lt_prefill_noalloc).
//
// Some callers cannot allocate device memory at call time (code under HIP graph
// capture, tight serving loops, harnesses that forbid it). For them the
// segmented prefill plan takes its workspace from a fixed static array instead
// of a caller buffer. The array lives in this code object; each GPU that the
// library runs on holds its own copy, at its own address, until the process
// ends. In host code the array's name is only a stand-in, so its device
// address is looked up once per device with hipGetSymbolAddress (with that
// device current) and kept; kernels receive that address, never the name.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"

namespace {

// 64 MiB. The coarsest segmented plan (one pre-pass piece per segment) holds
// 2G - 1 states of 64 KiB per (sequence, head) pair, with at most
// G = ceil(256 / u) segments for u < 256 pairs; u (2 ceil(256 / u) - 1) peaks
// at u = 255 (765 states, 47.8 MiB), so every accepted call fits and the
// planner takes the finest pieces that do.
constexpr size_t kScratchBytes = size_t(64) << 20;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void *g_scratch[kMaxDevices] = {};

// Restores the caller's current device on scope exit.
struct CurrentDevice {
    int saved = -1;
    ~CurrentDevice() {
        if (saved >= 0) (void)hipSetDevice(saved);
    }
};

}  // namespace

namespace lt {

hipError_t noalloc_scratch(hipStream_t stream, void **ptr, size_t *bytes) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    int dev = cur;
    if (stream) {  // the stream's device, which need not be the current one
        e = hipStreamGetDevice(stream, &dev);
        if (e != hipSuccess) return e;
    }
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_lock);
    if (!g_scratch[dev]) {
        CurrentDevice restore;
        if (dev != cur) {
            e = hipSetDevice(dev);
            if (e != hipSuccess) return e;
            restore.saved = cur;
        }
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch[dev] = p;
    }
    *ptr = g_scratch[dev];
    *bytes = kScratchBytes;
    return hipSuccess;
}

}  // namespace lt
