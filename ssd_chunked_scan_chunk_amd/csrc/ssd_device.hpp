// ssd_device.hpp -- device-side building blocks shared by the gfx950 kernels:
// bf16 storage conversion, wavefront/workgroup fp32 prefix sums and the MFMA
// fragment types.  gfx950 only (wave64, v_mfma_f32_16x16x32_bf16).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16;

constexpr float kLog2e = 1.4426950408889634f;

// ---- storage conversion ------------------------------------------------------
__device__ __forceinline__ float bf_bits_to_f32(u16 v) {
    return __uint_as_float(static_cast<uint32_t>(v) << 16);
}
// float32 -> bfloat16, round to nearest even (gfx950 converts in hardware).
__device__ __forceinline__ u16 f32_to_bf_bits(float f) {
    __bf16 b = static_cast<__bf16>(f);
    return __builtin_bit_cast(u16, b);
}
__device__ __forceinline__ __bf16 f32_to_bf(float f) { return static_cast<__bf16>(f); }

template <typename T> struct Elem;
template <> struct Elem<float> {
    __device__ __forceinline__ static float load(const float* p) { return *p; }
    __device__ __forceinline__ static void store(float* p, float v) { *p = v; }
};
template <> struct Elem<u16> {
    __device__ __forceinline__ static float load(const u16* p) { return bf_bits_to_f32(*p); }
    __device__ __forceinline__ static void store(u16* p, float v) { *p = f32_to_bf_bits(v); }
};

// Workgroup barrier that orders LDS accesses only.  __syncthreads() also
// waits for every outstanding global load and store of the wave, which would
// serialise each chunk's HBM traffic with its compute.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---- prefix sums ---------------------------------------------------------------
// Inclusive prefix sum across the 64 lanes of a wavefront (Hillis-Steele over
// lane shuffles: log2(64) = 6 rounds, each adding the value `d` lanes below).
__device__ __forceinline__ float wave_inclusive_scan(float v) {
    const int lane = __lane_id();
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const float t = __shfl_up(v, d, 64);
        if (lane >= d) v += t;
    }
    return v;
}

// Inclusive prefix sum of one value per thread over the first `nwaves_used`
// wavefronts of the workgroup (threads beyond contribute nothing).  `s_tot`
// is LDS scratch of at least nwaves_used floats.  Contains two barriers, so
// every thread of the workgroup must call it.
__device__ __forceinline__ float block_inclusive_scan(float v, float* s_tot, int nwaves_used) {
    const int lane = __lane_id();
    const int wave = threadIdx.x >> 6;
    v = wave_inclusive_scan(v);
    if (lane == 63 && wave < nwaves_used) s_tot[wave] = v;
    lds_barrier();
    float add = 0.f;
    for (int w = 0; w < wave && w < nwaves_used; ++w) add += s_tot[w];
    lds_barrier();
    return v + add;
}

// 2^x on the hardware v_exp_f32 (about 1 ulp).  Arguments here are decay
// exponents, <= 0 for a <= 0; results below the fp32 normal range flush to 0,
// which only drops contributions smaller than 2^-126 relative.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

}  // namespace ssd
