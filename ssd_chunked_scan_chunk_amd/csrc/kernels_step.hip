// kernels_step.hip -- single-token recurrent decode step on gfx950.
//
// The constant-memory inference mode of the layer (CiteArk page of
// "Transformers are SSMs", section "what this means"): the fp32 P x N state of
// every (batch, head) is read once, decayed and given the rank-1 update, written
// back in place, and contracted with C for the output:
//     S <- exp(a) S + x (x) B ;   y[p] = sum_n S[p][n] C[n]
// 0.5 flop per byte: a pure HBM stream, no MFMA.  Each workgroup owns one
// (b, h): thread t covers 4 consecutive n of rows p = t / (N/4) + k * (256 /
// (N/4)), so every wave-wide access is one contiguous 1 KiB run; all of a
// thread's state loads are issued before any arithmetic, and the row sums over
// n finish with lane shuffles inside groups of N/4 lanes.
#include <type_traits>

#include "ssd_device.hpp"
#include "ssd_launch.hpp"

#ifndef SSD_STEP_ROWS
#define SSD_STEP_ROWS 2
#endif

namespace ssd {

template <typename T> __device__ __forceinline__ float4 load4(const T* p);
template <> __device__ __forceinline__ float4 load4<float>(const float* p) {
    return *reinterpret_cast<const float4*>(p);
}
template <> __device__ __forceinline__ float4 load4<u16>(const u16* p) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
                       __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u));
}

template <typename T> struct AccOf;
template <> struct AccOf<float> {
    typedef double type;
    __device__ __forceinline__ static double exp(float a) { return ::exp((double)a); }
};
template <> struct AccOf<u16> {
    typedef float type;
    __device__ __forceinline__ static float exp(float a) { return expf(a); }
};

// The sum of v over each group of LPR consecutive lanes (LPR a power of two,
// at most 64), in every lane of the group.  fp32: within 16 lanes by DPP
// moves (quad exchanges, then the half-row and row mirrors, each pairing a
// lane with one of the other half of its group), across 16-lane rows by lane
// shuffles; fp64 by lane shuffles.
template <typename Acc, int LPR>
__device__ __forceinline__ Acc row_sum(Acc v)
{
#pragma unroll
    for (int off = LPR / 2; off >= 1; off >>= 1) {
        if constexpr (std::is_same<Acc, float>::value) {
            if (off >= 16) {
                v += __shfl_xor(v, off, 64);
            } else {
                int t;   // row_mirror, row_half_mirror, quad_perm [2,3,0,1], quad_perm [1,0,3,2]
                if (off == 8) t = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xf, 0xf, false);
                else if (off == 4) t = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xf, 0xf, false);
                else if (off == 2) t = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xf, 0xf, false);
                else t = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xf, 0xf, false);
                v += __int_as_float(t);
            }
        } else {
            v += __shfl_xor(v, off, 64);
        }
    }
    return v;
}

// Fast path: N/4 lanes per state row (N in {16, 32, 64, 128, 256}); a
// workgroup covers ROWS * 256 / (N/4) consecutive rows of one (b, h), so that
// SPLIT = P / that workgroups share a (b, h) and each thread streams only ROWS
// float4 of the state (fewer per thread keep more of them in flight across
// the chip: the in-place stream of the same array reaches its best rate at
// one float4 per thread).
template <typename T, int N, int ROWS>
__global__ __launch_bounds__(256) void k_step(float* __restrict__ state, const T* __restrict__ x,
                                              const float* __restrict__ a, const T* __restrict__ B,
                                              const T* __restrict__ C, T* __restrict__ y, int H, int G,
                                              int P, int split)
{
    constexpr int LPR = N / 4;           // lanes per row
    constexpr int RPP = 256 / LPR;       // rows per pass of the workgroup
    const int bh = blockIdx.x / split, part = blockIdx.x - bh * split;
    const int b = bh / H, h = bh - b * H, g = h / (H / G);
    const int tid = threadIdx.x;
    const int nq = tid % LPR, r0 = part * (RPP * ROWS) + tid / LPR;

    float* Sb = state + (int64_t)bh * P * N;
    f32x4 s[ROWS];
#pragma unroll
    for (int k = 0; k < ROWS; ++k)
        s[k] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Sb + (r0 + k * RPP) * N) + nq);

    // fp32 inputs update and contract in fp64 (free here: the kernel is HBM
    // bound) so a dot product that cancels does not lose the fp32 digits;
    // bf16 inputs use fp32 arithmetic.
    using Acc = typename AccOf<T>::type;
    const float4 Bf = load4<T>(B + ((int64_t)b * G + g) * N + 4 * nq);
    const float4 Cf = load4<T>(C + ((int64_t)b * G + g) * N + 4 * nq);
    const Acc Bn[4] = {Bf.x, Bf.y, Bf.z, Bf.w}, Cn[4] = {Cf.x, Cf.y, Cf.z, Cf.w};
    const Acc e = AccOf<T>::exp(a[bh]);
    const T* xb = x + (int64_t)bh * P;
    T* yb = y + (int64_t)bh * P;
    // every row's x before any store (a store in flight would otherwise be
    // waited for, as loads and stores share one counter)
    Acc xp[ROWS];
#pragma unroll
    for (int k = 0; k < ROWS; ++k) xp[k] = Elem<T>::load(xb + r0 + k * RPP);

    Acc acc[ROWS];
#pragma unroll
    for (int k = 0; k < ROWS; ++k) {
        const int p = r0 + k * RPP;
        f32x4 v;
        acc[k] = 0;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const Acc nv = e * (Acc)s[k][c] + xp[k] * Bn[c];
            v[c] = (float)nv;
            acc[k] += nv * Cn[c];
        }
        __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(Sb + p * N) + nq);
    }
#pragma unroll
    for (int k = 0; k < ROWS; ++k) acc[k] = row_sum<Acc, LPR>(acc[k]);
#pragma unroll
    for (int k = 0; k < ROWS; ++k)
        if (nq == 0) Elem<T>::store(yb + r0 + k * RPP, (float)acc[k]);
}

// General path: one thread per state row, any P and N.
template <typename T>
__global__ __launch_bounds__(256) void k_step_any(float* __restrict__ state, const T* __restrict__ x,
                                                  const float* __restrict__ a, const T* __restrict__ B,
                                                  const T* __restrict__ C, T* __restrict__ y,
                                                  int64_t rows, int H, int P, int N, int G)
{
    const int64_t row = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (row >= rows) return;
    const int64_t bh = row / P;
    const int b = (int)(bh / H), h = (int)(bh - (int64_t)b * H), g = h / (H / G);
    using Acc = typename AccOf<T>::type;
    const Acc e = AccOf<T>::exp(a[bh]);
    const Acc xp = Elem<T>::load(x + row);
    const T* Bt = B + ((int64_t)b * G + g) * N;
    const T* Ct = C + ((int64_t)b * G + g) * N;
    float* S = state + row * N;
    Acc acc = 0;
    for (int n = 0; n < N; ++n) {
        const Acc v = e * (Acc)S[n] + xp * (Acc)Elem<T>::load(Bt + n);
        S[n] = (float)v;
        acc += v * (Acc)Elem<T>::load(Ct + n);
    }
    Elem<T>::store(y + row, (float)acc);
}

// The practical HBM ceiling of the decode step: the same in-place fp32
// read-modify-write (every element multiplied by s), with no other traffic.
// V float4 per thread, all loads issued before any store; NT selects the
// nontemporal hints the decode kernel uses.
template <int V, bool NT>
__global__ __launch_bounds__(256) void k_stream_rmw(float* __restrict__ data, int64_t n4, float s)
{
    f32x4* p = reinterpret_cast<f32x4*>(data);
    const int64_t base = (int64_t)blockIdx.x * (256 * V) + threadIdx.x;
    f32x4 v[V];
#pragma unroll
    for (int k = 0; k < V; ++k) {
        const int64_t i = base + (int64_t)k * 256;
        if (i < n4) v[k] = NT ? __builtin_nontemporal_load(p + i) : p[i];
    }
#pragma unroll
    for (int k = 0; k < V; ++k) {
        const int64_t i = base + (int64_t)k * 256;
        if (i < n4) {
            const f32x4 w = v[k] * s;
            if (NT) __builtin_nontemporal_store(w, p + i);
            else p[i] = w;
        }
    }
}

hipError_t launch_stream_rmw(float* data, int64_t n4, float s, int per_thread, bool nontemporal,
                             hipStream_t st)
{
    const int64_t per_block = 256 * (int64_t)per_thread;
    const dim3 grid((unsigned)((n4 + per_block - 1) / per_block)), blk(256);
#define SSD_RMW(VV)                                                                          \
    if (per_thread == VV) {                                                                  \
        if (nontemporal) hipLaunchKernelGGL((k_stream_rmw<VV, true>), grid, blk, 0, st, data, n4, s); \
        else hipLaunchKernelGGL((k_stream_rmw<VV, false>), grid, blk, 0, st, data, n4, s);  \
        return hipGetLastError();                                                            \
    }
    SSD_RMW(1) SSD_RMW(2) SSD_RMW(4) SSD_RMW(8)
#undef SSD_RMW
    return hipErrorInvalidValue;
}

template <typename T>
static hipError_t launch_step_t(int64_t Bz, int64_t H, int64_t P, int64_t N, int64_t G,
                                float* state, const T* x, const float* a, const T* B,
                                const T* C, T* y, hipStream_t st)
{
    const dim3 blk(256);
    // SSD_STEP_ROWS float4 per thread where the rows allow it
#define SSD_STEP_CASE(NN, PP)                                                                 \
    if (N == NN && P == PP) {                                                                 \
        constexpr int rpp = 256 / (NN / 4), rows = SSD_STEP_ROWS < PP / rpp ? SSD_STEP_ROWS : PP / rpp; \
        constexpr int split = PP / (rpp * rows);                                              \
        hipLaunchKernelGGL((k_step<T, NN, rows>), dim3((unsigned)(Bz * H * split)), blk, 0, st, state, x, \
                           a, B, C, y, (int)H, (int)G, (int)PP, split);                       \
        return hipGetLastError();                                                             \
    }
    SSD_STEP_CASE(128, 64)
    SSD_STEP_CASE(64, 64)
    SSD_STEP_CASE(128, 128)
#undef SSD_STEP_CASE
    const int64_t rows = Bz * H * P;
    hipLaunchKernelGGL(k_step_any<T>, dim3((unsigned)((rows + 255) / 256)), blk, 0, st, state, x,
                       a, B, C, y, rows, (int)H, (int)P, (int)N, (int)G);
    return hipGetLastError();
}

hipError_t launch_step(int64_t Bz, int64_t H, int64_t P, int64_t N, int64_t G, bool bf16,
                       float* state, const void* x, const float* a, const void* B,
                       const void* C, void* y, hipStream_t st)
{
    if (bf16)
        return launch_step_t<u16>(Bz, H, P, N, G, state, (const u16*)x, a, (const u16*)B,
                                  (const u16*)C, (u16*)y, st);
    return launch_step_t<float>(Bz, H, P, N, G, state, (const float*)x, a, (const float*)B,
                                (const float*)C, (float*)y, st);
}

}  // namespace ssd
