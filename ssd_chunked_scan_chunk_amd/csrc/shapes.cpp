// shapes.cpp -- host-side description of the compiled kernel set: which
// shapes each kernel family takes and how the forward MFMA kernel groups
// heads into workgroups.  Host code only (no kernels), so the C ABI's
// planning can also be built and checked without a GPU toolchain.
#include "ssd_launch.hpp"

namespace ssd {

bool mfma_supported(int64_t Q, int64_t P, int64_t N) {
    return (Q == 64 || Q == 128 || Q == 256) && (P == 32 || P == 64) && (N == 64 || N == 128);
}

int64_t mfma_heads_per_workgroup(int64_t P, int64_t N) {
    (void)N;
    return kMfmaStateWaves / (P / 32);
}

// The fused pass's units per workgroup: 4, 5 or 6 for headdim 64; 4 or 5
// for headdim 32 (six single-unit heads would need more LDS for their
// per-head stage-1 results than a CU has).
bool fwd_units_supported(int64_t P, int sw) {
    return sw == 4 || sw == 5 || (sw == 6 && P == 64);
}

bool valu_fwd_supported(const FwdShape& s) {
    return s.Q >= 1 && s.Q <= 256 && s.P * s.N <= 16384;
}

bool bwd_da_supported(int64_t Q, int64_t P, int64_t N) {
    return (Q == 64 || Q == 128 || Q == 256) && (P == 32 || P == 64) && (N == 64 || N == 128);
}

// bytes of the da kernel's C B^T tiles: every (batch, chunk, group) holds the
// T(T+1)/2 lower-triangle 32x32 fp32 tiles of its chunk, T = chunk / 32
int64_t cb_tiles_bytes(const FwdShape& s) {
    const int64_t nI = s.Q / 32;
    return s.Bz * s.nc * s.G * (nI * (nI + 1) / 2) * 1024 * 4;
}

}  // namespace ssd
