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
#include "cb_tiles.hpp"
#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {

// ---------------------------------------------------------------------------
// VALU forward.  One workgroup per (b, h) walks every chunk in order and keeps
// the fp32 state in LDS.  Intra-chunk decays exp(a_{j+1} + ... + a_i) and the
// chunk-state decays exp(a_{j+1} + ... + a_{end}) are accumulated term by term
// from the diagonal outwards, so no decay is ever formed as a difference of
// two large prefix sums (fp32 cancellation would cost ~1e-5 relative).
// The chunk's masked, decayed scores exp(a_{j+1} + ... + a_i) (C_i . B_j) are
// formed once per (i, j), kValuRows rows at a time into LDS (thread j owns
// column j and carries its segment sum down the rows), and then shared by
// every head-dim entry p of those rows.
// ---------------------------------------------------------------------------
constexpr int kValuThreads = 256;
constexpr int kValuRows = 16;

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
    float* sM = sTot + 4;       // [kValuRows][Q] decayed scores of a row block

    const int h = blockIdx.x, b = blockIdx.y, g = h / (H / G);
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

        // outputs of the chunk: intra-chunk masked product + carried state,
        // a block of kValuRows rows at a time
        float seg = 0.f;   // thread j: a_{j+1} + ... + a_i for the latest row i
        for (int i0 = 0; Y && i0 < Lc; i0 += kValuRows) {
            const int nr = Lc - i0 < kValuRows ? Lc - i0 : kValuRows;
            if (tid < Lc) {
                const int j = tid;
                const T* Bj = B + (((int64_t)b * L + t0 + j) * G + g) * N;
                for (int r = 0; r < nr; ++r) {
                    const int i = i0 + r;
                    float m = 0.f;
                    if (j <= i) {
                        if (j < i) seg += sA[i];
                        const T* Ci = C + (((int64_t)b * L + t0 + i) * G + g) * N;
                        float cb = 0.f;
                        for (int n = 0; n < N; ++n) cb += Elem<T>::load(Ci + n) * Elem<T>::load(Bj + n);
                        m = expf(seg) * cb;
                    }
                    sM[r * Q + j] = m;
                }
            }
            __syncthreads();
            for (int idx = tid; idx < nr * P; idx += kValuThreads) {
                const int r = idx / P, p = idx - r * P, i = i0 + r;
                const T* Ci = C + (((int64_t)b * L + t0 + i) * G + g) * N;
                float acc = 0.f;
                for (int j = i; j >= 0; --j)
                    acc += sM[r * Q + j] * Elem<T>::load(X + (((int64_t)b * L + t0 + j) * H + h) * P + p);
                float off = 0.f;
                for (int n = 0; n < N; ++n) off += Elem<T>::load(Ci + n) * sS[p * N + n];
                Elem<TY>::store(Y + (((int64_t)b * L + t0 + i) * H + h) * P + p, acc + expf(sCs[i]) * off);
            }
            __syncthreads();
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

// ---------------------------------------------------------------------------
// VALU forward, staged variant for the shapes whose chunk fits in LDS (N <= 128,
// Q <= 256, P*N a multiple of 256 with each thread's 32 or fewer state entries
// in one row).  Same per-(b, h) walk and the same fp32 products, but every
// operand of an inner loop comes from LDS or registers: the chunk's X in LDS,
// thread j's B row in registers for the scores, C rows per row block and B
// rows per 64-step block in LDS.  Decays come from fp64 prefix sums of a:
// exp(cs_i - cs_j) with the difference taken in fp64 has no cancellation
// (the fp32 sums above were built term by term for the same reason), and each
// step's state weight exp(cs_end - cs_j) is formed once per step instead of
// once per state entry.
// ---------------------------------------------------------------------------
constexpr int kValuNMax = 128, kValuNRMax = 32, kValuJB = 64;

__device__ __forceinline__ double block_scan_f64(double v, double* s_tot) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const double u = __shfl_up(v, d, 64);
        if (lane >= d) v += u;
    }
    if (lane == 63) s_tot[wave] = v;
    lds_barrier();
    double add = 0.0;
    for (int w = 0; w < wave; ++w) add += s_tot[w];
    lds_barrier();
    return v + add;
}

static size_t valu_fast_lds(const FwdShape& s) {
    const size_t work = (size_t)kValuRows * s.Q + (size_t)kValuRows * s.N;
    const size_t bblk = (size_t)kValuJB * s.N;
    return ((size_t)s.Q * s.P + (size_t)s.P * s.N + (work > bblk ? work : bblk) + s.Q) * sizeof(float) +
           ((size_t)s.Q + 4) * sizeof(double);
}

static bool valu_fast_ok(const FwdShape& s) {
    // (Q and N multiples of 4 keep every 16-byte LDS read aligned)
    if (s.N > kValuNMax || s.Q > kValuThreads || (s.P * s.N) % kValuThreads != 0 || s.Q % 4 != 0 ||
        s.N % 4 != 0)
        return false;
    const int64_t nr = s.P * s.N / kValuThreads;
    return nr <= kValuNRMax && s.N % nr == 0 && valu_fast_lds(s) <= 160 * 1024;
}

template <typename T, typename TY = T>
__global__ __launch_bounds__(kValuThreads) void k_valu_fwd_staged(
    const T* __restrict__ X, const float* __restrict__ a, const T* __restrict__ B,
    const T* __restrict__ C, const float* __restrict__ S0, TY* __restrict__ Y,
    float* __restrict__ S_fin, float* __restrict__ S_chunks, int64_t L, int H, int P, int N,
    int G, int Q)
{
    extern __shared__ double smem64[];
    double* sCs = smem64;                 // [Q] fp64 inclusive prefix sums of a
    double* sTot = sCs + Q;               // [4] scan scratch
    float* sX = reinterpret_cast<float*>(sTot + 4);   // [Q][P] the chunk's X
    float* sS = sX + Q * P;               // [P][N] carried state
    float* sW = sS + P * N;               // [Q] state weights of the chunk's steps
    float* sWork = sW + Q;                // scores [kValuRows][Q] + C rows [kValuRows][N], or B rows [kValuJB][N]
    float* sM = sWork;
    float* sC = sWork + kValuRows * Q;

    const int h = blockIdx.x, b = blockIdx.y, g = h / (H / G);
    const int tid = threadIdx.x;
    const int PN = P * N;
    const int NR = PN / kValuThreads;     // state entries per thread, one row
    const int sp = tid * NR / N, sn0 = (tid * NR) % N;
    const int64_t bh = (int64_t)b * H + h;
    auto xrow = [&](int64_t t) { return X + (((int64_t)b * L + t) * H + h) * P; };
    auto brow = [&](int64_t t) { return B + (((int64_t)b * L + t) * G + g) * N; };
    auto crow = [&](int64_t t) { return C + (((int64_t)b * L + t) * G + g) * N; };

    for (int k = tid; k < PN; k += kValuThreads) sS[k] = S0 ? S0[bh * PN + k] : 0.f;

    const int64_t nc = (L + Q - 1) / Q;
    for (int64_t c = 0; c < nc; ++c) {
        const int64_t t0 = c * Q;
        const int Lc = (int)((L - t0 < Q) ? (L - t0) : Q);
        __syncthreads();
        const double av = tid < Lc ? (double)a[((int64_t)b * L + t0 + tid) * H + h] : 0.0;
        const double cs = block_scan_f64(av, sTot);
        if (tid < Q) sCs[tid] = cs;
        for (int k = tid; k < Q * P; k += kValuThreads) {
            const int i = k / P;
            sX[k] = i < Lc ? Elem<T>::load(xrow(t0 + i) + (k - i * P)) : 0.f;
        }
        if (S_chunks)
            for (int k = tid; k < PN; k += kValuThreads)
                S_chunks[(((int64_t)b * nc + c) * H + h) * PN + k] = sS[k];
        __syncthreads();

        // ---- outputs: masked decayed scores per row block, then Y rows ----
        if (Y) {
            float bj[kValuNMax];
#pragma unroll
            for (int n = 0; n < kValuNMax; ++n)
                bj[n] = (tid < Lc && n < N) ? Elem<T>::load(brow(t0 + tid) + n) : 0.f;
            for (int i0 = 0; i0 < Lc; i0 += kValuRows) {
                const int nr = Lc - i0 < kValuRows ? Lc - i0 : kValuRows;
                for (int k = tid; k < nr * N; k += kValuThreads) {
                    const int r = k / N;
                    sC[k] = Elem<T>::load(crow(t0 + i0 + r) + (k - r * N));
                }
                __syncthreads();
                if (tid < Lc) {
                    for (int r = 0; r < nr; ++r) {
                        const int i = i0 + r;
                        float m = 0.f;
                        if (tid <= i) {
                            // four partial sums over n = 4k + e (16-byte reads of C)
                            float cb4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                            for (int n = 0; n < kValuNMax; n += 4)
                                if (n < N) {
                                    const float4 cv = *reinterpret_cast<const float4*>(&sC[r * N + n]);
                                    cb4[0] += cv.x * bj[n];
                                    cb4[1] += cv.y * bj[n + 1];
                                    cb4[2] += cv.z * bj[n + 2];
                                    cb4[3] += cv.w * bj[n + 3];
                                }
                            m = expf((float)(sCs[i] - sCs[tid])) * ((cb4[0] + cb4[1]) + (cb4[2] + cb4[3]));
                        }
                        sM[r * Q + tid] = m;
                    }
                }
                __syncthreads();
                for (int idx = tid; idx < nr * P; idx += kValuThreads) {
                    const int r = idx / P, p = idx - r * P, i = i0 + r;
                    // four partial sums each (j = 4k + e; n = 4k + e with 16-byte reads)
                    float acc4[4] = {0.f, 0.f, 0.f, 0.f};
                    int j = 0;
                    for (; j + 3 <= i; j += 4) {
                        const float4 mv = *reinterpret_cast<const float4*>(&sM[r * Q + j]);
                        acc4[0] += mv.x * sX[j * P + p];
                        acc4[1] += mv.y * sX[(j + 1) * P + p];
                        acc4[2] += mv.z * sX[(j + 2) * P + p];
                        acc4[3] += mv.w * sX[(j + 3) * P + p];
                    }
                    for (; j <= i; ++j) acc4[0] += sM[r * Q + j] * sX[j * P + p];
                    const float acc = (acc4[0] + acc4[1]) + (acc4[2] + acc4[3]);
                    float off4[4] = {0.f, 0.f, 0.f, 0.f};
                    for (int n = 0; n < N; n += 4) {
                        const float4 cv = *reinterpret_cast<const float4*>(&sC[r * N + n]);
                        const float4 sv = *reinterpret_cast<const float4*>(&sS[p * N + n]);
                        off4[0] += cv.x * sv.x;
                        off4[1] += cv.y * sv.y;
                        off4[2] += cv.z * sv.z;
                        off4[3] += cv.w * sv.w;
                    }
                    const float off = (off4[0] + off4[1]) + (off4[2] + off4[3]);
                    Elem<TY>::store(Y + (((int64_t)b * L + t0 + i) * H + h) * P + p,
                                    acc + expf((float)sCs[i]) * off);
                }
                __syncthreads();
            }
        }

        // ---- chunk state: dS[p][n] = sum_j w_j X[j][p] B[j][n], B rows staged
        // kValuJB at a time; S <- exp(cs_end) S + dS ----
        if (tid < Q) sW[tid] = tid < Lc ? expf((float)(sCs[Lc - 1] - sCs[tid])) : 0.f;
        float ds[kValuNRMax];
#pragma unroll
        for (int e = 0; e < kValuNRMax; ++e) ds[e] = 0.f;
        for (int j0 = 0; j0 < Lc; j0 += kValuJB) {
            const int nj = Lc - j0 < kValuJB ? Lc - j0 : kValuJB;
            __syncthreads();
            for (int k = tid; k < nj * N; k += kValuThreads) {
                const int r = k / N;
                sWork[k] = Elem<T>::load(brow(t0 + j0 + r) + (k - r * N));
            }
            __syncthreads();
            if (NR % 4 == 0) {   // 16-byte reads of the B rows
                for (int jj = 0; jj < nj; ++jj) {
                    const float xw = sW[j0 + jj] * sX[(j0 + jj) * P + sp];
                    const float* brw = sWork + jj * N + sn0;
#pragma unroll
                    for (int e = 0; e < kValuNRMax; e += 4)
                        if (e < NR) {
                            const float4 bv = *reinterpret_cast<const float4*>(brw + e);
                            ds[e] += xw * bv.x;
                            ds[e + 1] += xw * bv.y;
                            ds[e + 2] += xw * bv.z;
                            ds[e + 3] += xw * bv.w;
                        }
                }
            } else {
                for (int jj = 0; jj < nj; ++jj) {
                    const float xw = sW[j0 + jj] * sX[(j0 + jj) * P + sp];
                    const float* brw = sWork + jj * N + sn0;
#pragma unroll
                    for (int e = 0; e < kValuNRMax; ++e)
                        if (e < NR) ds[e] += xw * brw[e];
                }
            }
        }
        __syncthreads();
        const float decay = expf((float)sCs[Lc - 1]);
#pragma unroll
        for (int e = 0; e < kValuNRMax; ++e)
            if (e < NR) sS[sp * N + sn0 + e] = decay * sS[sp * N + sn0 + e] + ds[e];
    }
    __syncthreads();
    if (S_fin)
        for (int k = tid; k < PN; k += kValuThreads) S_fin[bh * PN + k] = sS[k];
}

hipError_t launch_valu_fwd(const FwdShape& s, bool bf16, const void* X, const float* a,
                           const void* B, const void* C, const float* S0, void* Y,
                           float* S_fin, hipStream_t st, float* S_chunks, bool y_f32)
{
    dim3 grid((unsigned)s.H, (unsigned)s.Bz);
    if (valu_fast_ok(s)) {
        const size_t lds = valu_fast_lds(s);
#define SSD_VALU_STAGED(TT, TYY)                                                                       \
    do {                                                                                               \
        auto k = k_valu_fwd_staged<TT, TYY>;                                                           \
        hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, \
                                           (int)lds);                                                  \
        if (e != hipSuccess) return e;                                                                 \
        hipLaunchKernelGGL(k, grid, dim3(kValuThreads), lds, st, (const TT*)X, a, (const TT*)B,        \
                           (const TT*)C, S0, (TYY*)Y, S_fin, S_chunks, s.L, (int)s.H, (int)s.P,        \
                           (int)s.N, (int)s.G, (int)s.Q);                                              \
    } while (0)
        if (bf16 && y_f32) SSD_VALU_STAGED(u16, float);
        else if (bf16) SSD_VALU_STAGED(u16, u16);
        else SSD_VALU_STAGED(float, float);
#undef SSD_VALU_STAGED
        return hipGetLastError();
    }
    const size_t lds = (size_t)(2 * s.Q + s.P * s.N + 4 + kValuRows * s.Q) * sizeof(float);
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
// every unit: read D_u, write the entering state, fold.  The reads of a window
// of kScanWin units are issued before any of its stores, so one memory round
// trip covers the window (the entering states may overwrite D in place: a
// thread writes only locations it has already read).
// ---------------------------------------------------------------------------
constexpr int kScanWin = 8;

// NCB (the dstate of the C B^T tiles, 0 for none): the first zcb planes of
// workgroups (blockIdx.z < zcb) form the da kernel's C B^T tiles instead
// (four per workgroup); dispatched first, their MFMA and latency-bound work
// overlaps the scan's streaming
template <int NCB>
__global__ __launch_bounds__(256) void k_state_scan(ScanJob j0, ScanJob j1, int Bz, int64_t nu,
                                                    int64_t ustride, int H, int PN, CbJob cb, int zcb)
{
    int z = (int)blockIdx.z;
    if constexpr (NCB > 0) {
        if (z < zcb) {
            const int64_t wi = ((int64_t)z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x;
            if (wi < cb_workgroups(cb, 4)) cb_tiles_wg<NCB, 4>(cb, wi, threadIdx.x >> 6, threadIdx.x & 63);
            return;
        }
        z -= zcb;
    }
    // z < Bz: job j0 for batch z; otherwise job j1 (a paired launch)
    const bool second = z >= Bz;
    const ScanJob j = second ? j1 : j0;
    const int h = blockIdx.y, b = second ? z - Bz : z;
    const int q = blockIdx.x * blockDim.x + threadIdx.x;  // float4 index
    if (q * 4 >= PN) return;
    const int64_t bh = (int64_t)b * H + h;
    float4 S = j.S0 ? reinterpret_cast<const float4*>(j.S0 + bh * PN)[q] : make_float4(0.f, 0.f, 0.f, 0.f);
    const float* lrow = j.lam + b * j.lam_bs + h * j.lam_hs;
    const int64_t ustep = (int64_t)H * PN;                       // floats between units
    const int64_t base = ((int64_t)b * ustride * H + h) * PN;    // unit 0 of (b, h)
    for (int64_t u0 = 0; u0 < nu; u0 += kScanWin) {
        float4 d[kScanWin];
        float l[kScanWin];
#pragma unroll
        for (int k = 0; k < kScanWin; ++k) {
            if (u0 + k < nu) {
                d[k] = reinterpret_cast<const float4*>(j.D + base + (u0 + k) * ustep)[q];
                l[k] = lrow[u0 + k];
            }
        }
#pragma unroll
        for (int k = 0; k < kScanWin; ++k) {
            const int64_t u = u0 + k;
            if (u < nu) {
                if (u >= j.u_write) reinterpret_cast<float4*>(j.Sout + base + u * ustep)[q] = S;
                const float e = expf(l[k]);
                S.x = e * S.x + d[k].x;
                S.y = e * S.y + d[k].y;
                S.z = e * S.z + d[k].z;
                S.w = e * S.w + d[k].w;
            }
        }
    }
    if (j.fin) reinterpret_cast<float4*>(j.fin + b * j.fin_bs + (int64_t)h * PN)[q] = S;
}

static hipError_t launch_scan_jobs(const FwdShape& s, int64_t nu, int64_t ustride, const ScanJob& j0,
                                   const ScanJob& j1, int njobs, const CbJob* cb, hipStream_t st)
{
    const int PN = (int)(s.P * s.N);
    const unsigned gx = (unsigned)((PN / 4 + 255) / 256), gy = (unsigned)s.H;
    const int64_t ncb = cb ? cb_workgroups(*cb, 4) : 0;
    const int zcb = (int)((ncb + (int64_t)gx * gy - 1) / ((int64_t)gx * gy));
    const CbJob none{nullptr, nullptr, nullptr, 0, 0, 0, 0, 0, 0};
    const dim3 grid(gx, gy, (unsigned)(njobs * s.Bz + zcb));
    if (!cb)
        hipLaunchKernelGGL(k_state_scan<0>, grid, dim3(256), 0, st, j0, j1, (int)s.Bz, nu, ustride, (int)s.H, PN,
                           none, 0);
    else if (cb->N == 128)
        hipLaunchKernelGGL(k_state_scan<128>, grid, dim3(256), 0, st, j0, j1, (int)s.Bz, nu, ustride, (int)s.H,
                           PN, *cb, zcb);
    else if (cb->N == 64)
        hipLaunchKernelGGL(k_state_scan<64>, grid, dim3(256), 0, st, j0, j1, (int)s.Bz, nu, ustride, (int)s.H,
                           PN, *cb, zcb);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_state_scan(const FwdShape& s, int64_t nu, int64_t ustride, const float* D,
                             const float* lam,
                             int64_t lam_bstride, int64_t lam_hstride, const float* S0,
                             float* Sout, int64_t u_write, float* final_, int64_t final_bstride,
                             hipStream_t st)
{
    const ScanJob j{D, lam, lam_bstride, lam_hstride, S0, Sout, u_write, final_, final_bstride};
    return launch_scan_jobs(s, nu, ustride, j, j, 1, nullptr, st);
}

hipError_t launch_state_scan_pair(const FwdShape& s, int64_t nu, int64_t ustride, const ScanJob& j0,
                                  const ScanJob& j1, const CbJob* cb, hipStream_t st)
{
    // grid.z within the 16-bit range: otherwise two launches and the tiles on their own
    const int64_t gxy = (int64_t)((s.P * s.N / 4 + 255) / 256) * s.H;
    const int64_t zcb = cb ? (cb_workgroups(*cb, 4) + gxy - 1) / gxy : 0;
    if (2 * s.Bz + zcb > 65535) {
        hipError_t e = launch_scan_jobs(s, nu, ustride, j0, j0, 1, nullptr, st);
        if (e == hipSuccess) e = launch_scan_jobs(s, nu, ustride, j1, j1, 1, nullptr, st);
        if (e == hipSuccess && cb) e = launch_cb_tiles(*cb, st);
        return e;
    }
    return launch_scan_jobs(s, nu, ustride, j0, j1, 2, cb, st);
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
