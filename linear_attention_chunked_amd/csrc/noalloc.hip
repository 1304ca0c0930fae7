// noalloc.hip -- scratch memory for the allocation-free forward entry point.
//
// ttt_fwd_chunked_noalloc runs the same kernels as ttt_fwd_chunked, for
// callers that cannot allocate (code under graph capture, tight serving
// loops).  The only scratch those kernels use is the segmented look-back's
// flags, ticket counter, error word and exchanged states; here it lives in
// a file-scope device array instead of a caller's workspace.  Every GPU the
// library runs on holds its own copy of the array until the process ends,
// and every call on that GPU shares it: the look-back clears its flags at
// the start of each call (a fill kernel), and calls that overlap in time on
// one GPU race on the array.
//
// The worst case of the look-back's workspace is below 64 MiB: a call is
// only segmented while its (head, value-column tile) grid is short of the
// chip, so it runs fewer than 2 x 256 workgroups of the 64-column form (or
// 2 x 512 of the 32-column form), each exchanging two state blocks of at
// most 128 x 64 x 2 (or 128 x 32 x 2) floats.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"

namespace ttt {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

// the array's device address per device, set once (the only state the
// library keeps; guarded by g_mu)
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

// The device address of `scratch` on the current device.  In host code the
// array's name is only a stand-in for the symbol, so its address is looked
// up once per device with hipGetSymbolAddress and kept.
hipError_t noalloc_scratch(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return hipSuccess;
}

}  // namespace ttt
