// noalloc.hip -- the forward entry point that allocates nothing.
//
// The segmented plan keeps the fp32 states of its segments and their
// log-decays in a workspace.  Callers that cannot allocate get that workspace
// from one file-scope device array per GPU: each device holds its own copy of
// `scratch` (SSD_NOALLOC_SCRATCH_BYTES) until the process ends.  In host code
// the array's name is only a stand-in, so its device address is looked up
// once per device (hipGetSymbolAddress with that device current) and only
// that address is passed to kernels.  The kernels ignore the region's
// contents on entry (every state slot they read is written earlier in the
// same call), so nothing is cleared.  Calls that overlap on one device share
// the region and race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "ssd.h"
#include "ssd_launch.hpp"

static __device__ __align__(256) unsigned char scratch[SSD_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 256;
std::mutex g_mu;
void* g_scratch[kMaxDevices];   // device address of each device's copy, once looked up

hipError_t scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

}  // namespace

extern "C" ssd_status ssd_chunk_scan_fwd_noalloc(const ssd_fwd_desc* desc, const void* X, const float* a,
                                                 const void* B, const void* C, const float* initial_state,
                                                 void* Y, float* final_state, void* stream) {
    return ssd::fwd_with_fixed_workspace(desc, X, a, B, C, initial_state, Y, final_state,
                                         SSD_NOALLOC_SCRATCH_BYTES, scratch_address, stream);
}
