// abi_stubs.cpp -- kernel launchers for a host-only build of the C ABI
// (api.cpp + shapes.cpp) under AddressSanitizer / UndefinedBehaviorSanitizer.
// That build exercises argument validation and planning on the CPU; every
// call it is given fails validation or is host-only, so none of these should
// run.  If one does, it reports hipErrorNotSupported instead of launching.
#include "ssd_launch.hpp"

extern "C" const char* hipGetErrorString(hipError_t) { return "stub launcher (host-only build)"; }

// the allocation-free forward over a host stand-in for its device array
// (the launch stubs never touch it)
static hipError_t fake_scratch(void** p) {
    static unsigned char region[256];
    *p = region;
    return hipSuccess;
}
extern "C" ssd_status ssd_chunk_scan_fwd_noalloc(const ssd_fwd_desc* desc, const void* X, const float* a,
                                                 const void* B, const void* C, const float* initial_state,
                                                 void* Y, float* final_state, void* stream) {
    return ssd::fwd_with_fixed_workspace(desc, X, a, B, C, initial_state, Y, final_state,
                                         SSD_NOALLOC_SCRATCH_BYTES, fake_scratch, stream);
}

namespace ssd {
#define SSD_STUB return hipErrorNotSupported
hipError_t launch_valu_fwd(const FwdShape&, bool, const void*, const float*, const void*, const void*,
                           const float*, void*, float*, hipStream_t, float*, bool) { SSD_STUB; }
hipError_t launch_chunk_cumsum(const FwdShape&, const float*, float*, float*, hipStream_t) { SSD_STUB; }
hipError_t launch_state_scan(const FwdShape&, int64_t, int64_t, const float*, const float*, int64_t,
                             int64_t, const float*, float*, int64_t, float*, int64_t, hipStream_t) { SSD_STUB; }
hipError_t launch_state_scan_pair(const FwdShape&, int64_t, int64_t, const ScanJob&, const ScanJob&,
                                  const CbJob*, hipStream_t) { SSD_STUB; }
hipError_t launch_mfma_state(const FwdShape&, int64_t, int64_t, int64_t, const void*, const float*,
                             const void*, float*, float*, hipStream_t, bool) { SSD_STUB; }
hipError_t launch_mfma_state_pair(const FwdShape&, int64_t, int64_t, int64_t, const StatePass&,
                                  const StatePass&, hipStream_t) { SSD_STUB; }
hipError_t launch_fwd(const FwdShape&, int, int64_t, int64_t, const void*, const float*, const void*,
                      const void*, StateSrc, void*, float*, hipStream_t, bool, const float*,
                      int64_t) { SSD_STUB; }
int64_t fwd_workgroups(const FwdShape&, int64_t, int) { return 0; }
hipError_t launch_mfma_out_xg_pair(const FwdShape&, int64_t, const XgPass&, const XgPass&, hipStream_t) { SSD_STUB; }
hipError_t launch_step(int64_t, int64_t, int64_t, int64_t, int64_t, bool, float*, const void*,
                       const float*, const void*, const void*, void*, hipStream_t) { SSD_STUB; }
hipError_t launch_stream_rmw(float*, int64_t, float, int, bool, hipStream_t) { SSD_STUB; }
hipError_t launch_remap_rows(void*, const void*, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t,
                             hipStream_t) { SSD_STUB; }
hipError_t launch_bcast_heads(void*, const void*, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t,
                              int64_t, int64_t, hipStream_t) { SSD_STUB; }
hipError_t launch_remap_a(float*, const float*, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t,
                          int64_t, hipStream_t) { SSD_STUB; }
hipError_t launch_state_transpose(float*, const float*, int64_t, int64_t, int64_t, hipStream_t) { SSD_STUB; }
hipError_t launch_group_sum(void*, const void*, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t,
                            int64_t, int64_t, bool, bool, hipStream_t) { SSD_STUB; }
hipError_t launch_group_sum_pair(const GsJob&, const GsJob&, int64_t, int64_t, int64_t, int64_t, int64_t, bool,
                                 bool, hipStream_t) { SSD_STUB; }
hipError_t launch_scale_state_by_a0(float*, const float*, int64_t, int64_t, int64_t, int64_t,
                                    hipStream_t) { SSD_STUB; }
hipError_t launch_bwd_da_valu(const FwdShape&, const float*, const float*, const float*, const float*,
                              const float*, const float*, const float*, float*, hipStream_t) { SSD_STUB; }
hipError_t launch_bwd_da(const FwdShape&, const void*, const void*, const float*, const void*,
                         const void*, const float*, const float*, const float*, bool, float*,
                         hipStream_t) { SSD_STUB; }
hipError_t launch_cb_tiles(const CbJob&, hipStream_t) { SSD_STUB; }
hipError_t launch_fill_zero(float*, int64_t, hipStream_t) { SSD_STUB; }
hipError_t launch_copy_f32(float*, const float*, int64_t, hipStream_t) { SSD_STUB; }
#undef SSD_STUB
}  // namespace ssd
