// kernels_scan.hip -- the VALU kernels of the SSD layer for gfx950:
//   * k_valu_fwd       per-(batch, head) sequential walk over chunks with fp32
//                      arithmetic and exact segment sums (fp32 inputs, and any
//                      shape the MFMA kernels are not compiled for);
//   * k_chunk_cumsum   stage 1, in-chunk prefix sums of a on wavefront scans;
//   * k_state_scan     stage 4, the inter-chunk (or inter-segment) state scan,
//                      streaming the fp32 states once with 16-byte accesses;
//   * k_fill / k_copy  trivial helpers.
//
// Decomposition (wiki review of "Transformers are SSMs", section "Core
// concepts": semiseparable matrices and the block-decomposition SSD
// algorithm): within a chunk of Q steps the output is the masked quadratic
// form, across chunks it flows through the carried P x N state.
#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {

// ---------------------------------------------------------------------------
// VALU forward.  One workgroup per (b, h) walks every chunk in order and keeps
// the fp32 state in LDS.  Intra-chunk decays exp(a_{j+1} + ... + a_i) and the
// chunk-state decays exp(a_{j+1} + ... + a_{end}) are accumulated term by term
// from the diagonal outwards, so no decay is ever formed as a difference of
// two large prefix sums (fp32 cancellation would cost ~1e-5 relative).
// ---------------------------------------------------------------------------
constexpr int kValuThreads = 256;

// Y (of type TY) may be null (only the states are wanted); S_chunks
// (optional) receives the state entering every chunk, [Bz][nc][H][P*N].
template <typename T, typename TY = T>
__global__ __launch_bounds__(kValuThreads) void k_valu_fwd(
    const T* __restrict__ X, const float* __restrict__ a, const T* __restrict__ B,
    const T* __restrict__ C, const float* __restrict__ S0, TY* __restrict__ Y,
    float* __restrict__ S_fin, float* __restrict__ S_chunks, int64_t L, int H, int P, int N,
    int G, int Q)
{
    extern __shared__ float smem[];
    float* sA = smem;           // [Q] a of the chunk
    float* sCs = sA + Q;        // [Q] inclusive prefix sums
    float* sS = sCs + Q;        // [P*N] carried state
    float* sTot = sS + P * N;   // [4] scan scratch

    const int h = blockIdx.x, b = blockIdx.y, g = h * G / H;
    const int tid = threadIdx.x;
    const int PN = P * N;
    const int64_t bh = (int64_t)b * H + h;

    for (int k = tid; k < PN; k += kValuThreads) sS[k] = S0 ? S0[bh * PN + k] : 0.f;

    const int64_t nc = (L + Q - 1) / Q;
    for (int64_t c = 0; c < nc; ++c) {
        const int64_t t0 = c * Q;
        const int Lc = (int)((L - t0 < Q) ? (L - t0) : Q);
        __syncthreads();
        float av = 0.f;
        if (tid < Lc) av = a[((int64_t)b * L + t0 + tid) * H + h];
        if (tid < Q) sA[tid] = av;
        const float cs = block_inclusive_scan(av, sTot, (Q + 63) / 64);
        if (tid < Q) sCs[tid] = cs;
        __syncthreads();
        if (S_chunks)
            for (int k = tid; k < PN; k += kValuThreads)
                S_chunks[(((int64_t)b * nc + c) * H + h) * PN + k] = sS[k];

        // outputs of the chunk: intra-chunk masked product + carried state
        for (int idx = tid; Y && idx < Lc * P; idx += kValuThreads) {
            const int i = idx / P, p = idx - i * P;
            const T* Ci = C + (((int64_t)b * L + t0 + i) * G + g) * N;
            float acc = 0.f, seg = 0.f;
            for (int j = i; j >= 0; --j) {
                if (j < i) seg += sA[j + 1];
                const T* Bj = B + (((int64_t)b * L + t0 + j) * G + g) * N;
                float cb = 0.f;
                for (int n = 0; n < N; ++n) cb += Elem<T>::load(Ci + n) * Elem<T>::load(Bj + n);
                acc += expf(seg) * cb * Elem<T>::load(X + (((int64_t)b * L + t0 + j) * H + h) * P + p);
            }
            float off = 0.f;
            for (int n = 0; n < N; ++n) off += Elem<T>::load(Ci + n) * sS[p * N + n];
            Elem<TY>::store(Y + (((int64_t)b * L + t0 + i) * H + h) * P + p, acc + expf(sCs[i]) * off);
        }
        __syncthreads();
        // chunk state and the hand-off across the chunk boundary
        const float chunk_decay = expf(sCs[Lc - 1]);
        for (int idx = tid; idx < PN; idx += kValuThreads) {
            const int p = idx / N, n = idx - p * N;
            float ds = 0.f, suffix = 0.f;
            for (int j = Lc - 1; j >= 0; --j) {
                if (j < Lc - 1) suffix += sA[j + 1];
                const float xj = Elem<T>::load(X + (((int64_t)b * L + t0 + j) * H + h) * P + p);
                const float bj = Elem<T>::load(B + (((int64_t)b * L + t0 + j) * G + g) * N + n);
                ds += expf(suffix) * xj * bj;
            }
            sS[idx] = chunk_decay * sS[idx] + ds;
        }
    }
    __syncthreads();
    if (S_fin)
        for (int k = tid; k < PN; k += kValuThreads) S_fin[bh * PN + k] = sS[k];
}

bool valu_fwd_supported(const FwdShape& s) {
    return s.Q >= 1 && s.Q <= 256 && s.P * s.N <= 16384;
}

hipError_t launch_valu_fwd(const FwdShape& s, bool bf16, const void* X, const float* a,
                           const void* B, const void* C, const float* S0, void* Y,
                           float* S_fin, hipStream_t st, float* S_chunks, bool y_f32)
{
    const size_t lds = (size_t)(2 * s.Q + s.P * s.N + 4) * sizeof(float);
    dim3 grid((unsigned)s.H, (unsigned)s.Bz);
    if (bf16 && y_f32) {
        auto k = k_valu_fwd<u16, float>;
        hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(k, grid, dim3(kValuThreads), lds, st, (const u16*)X, a, (const u16*)B,
                           (const u16*)C, S0, (float*)Y, S_fin, S_chunks, s.L, (int)s.H, (int)s.P,
                           (int)s.N, (int)s.G, (int)s.Q);
    } else if (bf16) {
        auto k = k_valu_fwd<u16>;
        hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(k, grid, dim3(kValuThreads), lds, st, (const u16*)X, a, (const u16*)B,
                           (const u16*)C, S0, (u16*)Y, S_fin, S_chunks, s.L, (int)s.H, (int)s.P,
                           (int)s.N, (int)s.G, (int)s.Q);
    } else {
        auto k = k_valu_fwd<float>;
        hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(k, grid, dim3(kValuThreads), lds, st, (const float*)X, a, (const float*)B,
                           (const float*)C, S0, (float*)Y, S_fin, S_chunks, s.L, (int)s.H,
                           (int)s.P, (int)s.N, (int)s.G, (int)s.Q);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Stage 1: cs[b][h][c][i] = a_{cQ} + ... + a_{cQ+i}; lam[b][h][c] = chunk total.
// One workgroup of 256 threads per (c, h, b); fp32 wavefront scans.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_chunk_cumsum(const float* __restrict__ a,
                                                      float* __restrict__ cs,
                                                      float* __restrict__ lam, int64_t L,
                                                      int H, int Q, int64_t nc)
{
    __shared__ float sTot[4];
    const int64_t c = blockIdx.x;
    const int h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x;
    const int64_t t0 = c * Q;
    const int Lc = (int)((L - t0 < Q) ? (L - t0) : Q);
    float v = 0.f;
    if (tid < Lc) v = a[((int64_t)b * L + t0 + tid) * H + h];
    const float r = block_inclusive_scan(v, sTot, (Q + 63) / 64);
    const int64_t row = ((int64_t)b * H + h) * nc + c;
    if (tid < Q) cs[row * Q + tid] = (tid < Lc) ? r : 0.f;
    if (tid == Lc - 1) lam[row] = r;
}

hipError_t launch_chunk_cumsum(const FwdShape& s, const float* a, float* cs, float* lam,
                               hipStream_t st)
{
    dim3 grid((unsigned)s.nc, (unsigned)s.H, (unsigned)s.Bz);
    hipLaunchKernelGGL(k_chunk_cumsum, grid, dim3(256), 0, st, a, cs, lam, s.L, (int)s.H,
                       (int)s.Q, s.nc);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Stage 4: sequential over units (chunks or segments), parallel over
// (b, h, 4-float groups of the state).  Each thread streams its float4 of
// every unit: read D_u, write the entering state, fold.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_state_scan(
    const float* D, const float* __restrict__ lam, int64_t lam_bs, int64_t lam_hs,
    const float* __restrict__ S0, float* Sout, int64_t u_write, float* __restrict__ fin,
    int64_t fin_bs, int64_t nu, int64_t ustride, int H, int PN)
{
    const int h = blockIdx.y, b = blockIdx.z;
    const int q = blockIdx.x * blockDim.x + threadIdx.x;  // float4 index
    if (q * 4 >= PN) return;
    const int64_t bh = (int64_t)b * H + h;
    float4 S = S0 ? reinterpret_cast<const float4*>(S0 + bh * PN)[q] : make_float4(0.f, 0.f, 0.f, 0.f);
    const float* lrow = lam + b * lam_bs + h * lam_hs;
    for (int64_t u = 0; u < nu; ++u) {
        const int64_t off = (((int64_t)b * ustride + u) * H + h) * PN;
        const float4 d = reinterpret_cast<const float4*>(D + off)[q];
        if (u >= u_write) reinterpret_cast<float4*>(Sout + off)[q] = S;
        const float e = expf(lrow[u]);
        S.x = e * S.x + d.x;
        S.y = e * S.y + d.y;
        S.z = e * S.z + d.z;
        S.w = e * S.w + d.w;
    }
    if (fin) reinterpret_cast<float4*>(fin + b * fin_bs + (int64_t)h * PN)[q] = S;
}

hipError_t launch_state_scan(const FwdShape& s, int64_t nu, int64_t ustride, const float* D,
                             const float* lam,
                             int64_t lam_bstride, int64_t lam_hstride, const float* S0,
                             float* Sout, int64_t u_write, float* final_, int64_t final_bstride,
                             hipStream_t st)
{
    const int PN = (int)(s.P * s.N);
    dim3 grid((unsigned)((PN / 4 + 255) / 256), (unsigned)s.H, (unsigned)s.Bz);
    hipLaunchKernelGGL(k_state_scan, grid, dim3(256), 0, st, D, lam, lam_bstride, lam_hstride,
                       S0, Sout, u_write, final_, final_bstride, nu, ustride, (int)s.H, PN);
    return hipGetLastError();
}

__global__ void k_fill_zero(float* p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0.f;
}
__global__ void k_copy_f32(float* d, const float* s, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        d[i] = s[i];
}

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    const int64_t blocks = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
    hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)blocks), dim3(256), 0, st, p, n);
    return hipGetLastError();
}
hipError_t launch_copy_f32(float* dst, const float* src, int64_t n, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    const int64_t blocks = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
    hipLaunchKernelGGL(k_copy_f32, dim3((unsigned)blocks), dim3(256), 0, st, dst, src, n);
    return hipGetLastError();
}

}  // namespace ssd
