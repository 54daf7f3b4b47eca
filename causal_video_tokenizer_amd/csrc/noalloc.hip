// The factorized causal convolution with its scratch memory in the library: the packed
// weights and the bf16 spatial->temporal intermediate that cvt_causal_conv3d_fact keeps in
// the caller's workspace live here in a file-scope device array, so the call needs no
// allocation from anyone (code under HIP graph capture, loops that must not allocate).
//
// Each GPU the library runs on holds its own copy of the array until the process ends.
// Host code never passes the array's name to a kernel or a copy (on the host that name is
// a stand-in, not a device address): the address comes from hipGetSymbolAddress, taken
// once per device with that device current, and kept per device.
#include <atomic>
#include <mutex>

#include "cvt_internal.h"

static __device__ __align__(256) uint8_t scratch[CVT_NOALLOC_SCRATCH_BYTES];

namespace cvt {
namespace {

constexpr int MAX_DEVICES = 64;
std::atomic<void*> g_scratch[MAX_DEVICES];
std::mutex g_scratch_mu;

// Device address of the current device's copy of `scratch`.
hipError_t scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (!p) return hipErrorInvalidSymbol;
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return hipSuccess;
}

}  // namespace

// The caller has validated the arguments and checked that conv_workspace_bytes() fits
// CVT_NOALLOC_SCRATCH_BYTES.  Nothing in the array must start at zero: the weight repack
// writes every packed byte (padding included) and the spatial part writes the whole
// intermediate before the temporal part reads it.
hipError_t launch_conv_fact_noalloc(const void* x, const void* w_s, const void* w_t, const float* b_s,
                                    const float* b_t, void* y, int B, int Cin, int Cout, int T, int H, int W, int k,
                                    hipStream_t s) {
    void* ws = nullptr;
    hipError_t e = scratch_address(&ws);
    if (e != hipSuccess) return e;
    return launch_conv_fact(x, w_s, w_t, b_s, b_t, y, B, Cin, Cout, T, H, W, k, ws, s);
}

}  // namespace cvt
