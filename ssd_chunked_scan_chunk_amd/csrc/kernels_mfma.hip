// kernels_mfma.hip -- bf16 MFMA kernels of the SSD layer for gfx950.
//
// The layer's sequence map is the 1-semiseparable matrix M = Lmask o (C B^T)
// applied to X (wiki review of "Transformers are SSMs", section "Core
// concepts"; CiteArk page, section "AI research summary": a block-decomposed
// matrix-multiplication algorithm over that matrix).  Blocking the sequence
// into chunks of Q steps gives four stages per chunk c:
//   1. in-chunk prefix sums cs of a (wavefront scans, fp32);
//   2. diagonal block:   Ydiag = (Lmask_cc o C_c B_c^T) X_c        (MFMA)
//   3. chunk state:      dS_c  = (w o X_c)^T B_c, w_j = exp(Lam_c - cs_j)  (MFMA)
//   4. state passing:    S_{c+1} = exp(Lam_c) S_c + dS_c            (in registers)
//   5. state to output:  Yoff = diag(exp(cs)) C_c S_c^T             (MFMA)
//
// One workgroup walks `seg_chunks` consecutive chunks of one (batch, head)
// and carries the fp32 P x N state in MFMA accumulator registers from chunk
// to chunk, so states never round-trip HBM inside a segment.  When a launch
// would leave CUs idle the sequence is split into segments: a state-only pass
// (stage 1 + 3 + 4) gives each segment's end state from zero, a short scan
// over segments (kernels_scan.hip) gives every segment's entering state, and
// the full pass runs all stages from that state.
//
// Workgroup: Q/32 wavefronts.  Row blocks of 16 steps are dealt to waves in
// pairs (w, Q/16-1-w) so every wave owns the same number of causal 16x16
// tiles.  The intra-chunk scores are formed transposed, S^T = B C^T, so that
// the v_mfma_f32_16x16x32_bf16 accumulator layout (lane = column i, registers
// = 4 consecutive rows j per 16-lane group) is already the A-operand layout
// of the next product with X: two adjacent 16-wide j tiles give the 8 k
// values of one lane group, and X is read from LDS in the same j order.
// Operand rounding: Lmask o S (after the fp32 mask), w o X and the entering
// state are rounded to bf16 for the MFMA; all accumulation is fp32.
#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {

template <int Q, int P, int N>
struct MfmaCfg {
    static constexpr int NW = Q / 32;       // wavefronts
    static constexpr int NT = NW * 64;      // threads
    static constexpr int RB = Q / 16;       // 16-step row blocks
    static constexpr int KN = N / 32;       // k steps over the state dim
    static constexpr int PT = P / 16;       // 16-wide head-dim tiles
    static constexpr int NTL = N / 16;      // 16-wide state-dim tiles
    static constexpr int TT = PT * NTL;     // state tiles
    static constexpr int TPW = TT / NW;     // state tiles per wave
    static constexpr int KJ = Q / 32;       // k steps over the chunk
    static constexpr int BLD = N + 8;       // LDS row strides (bf16 elements),
    static constexpr int XLD = Q + 8;       //   padded by 16 bytes against
    static constexpr int SLD = N + 8;       //   bank conflicts
    static_assert(Q % 64 == 0 && P % 16 == 0 && N % 32 == 0, "tile shape");
    static_assert(TT % NW == 0, "state tiles must split evenly over waves");
};

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));  // register-friendly 16-byte piece
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ __bf16 bits_to_bf(u16 v) { return __builtin_bit_cast(__bf16, v); }

template <int Q, int P, int N, bool FULL>
__global__ __launch_bounds__(Q * 2) void k_mfma_seg(
    const u16* __restrict__ X, const float* __restrict__ a, const u16* __restrict__ B,
    const u16* __restrict__ C, StateSrc src, u16* __restrict__ Y, float* __restrict__ S_fin,
    float* __restrict__ Sseg, float* __restrict__ lamseg, int64_t nseg_total, int64_t L,
    int H, int G, int64_t nc, int64_t seg_chunks)
{
    using Cfg = MfmaCfg<Q, P, N>;
    constexpr int NT = Cfg::NT, RB = Cfg::RB, KN = Cfg::KN, PT = Cfg::PT, TPW = Cfg::TPW;
    constexpr int KJ = Cfg::KJ, BLD = Cfg::BLD, XLD = Cfg::XLD, SLD = Cfg::SLD;

    __shared__ __attribute__((aligned(16))) u16 sB[Q * BLD];              // B_c  [j][n]
    __shared__ __attribute__((aligned(16))) u16 sWXt[P * XLD];            // (w o X_c)^T [p][j]
    __shared__ __attribute__((aligned(16))) u16 sXt[FULL ? P * XLD : 8];  // X_c^T [p][j]
    __shared__ __attribute__((aligned(16))) u16 sS[FULL ? P * SLD : 8];   // entering state [p][n]
    __shared__ __attribute__((aligned(16))) float sCs[Q];                 // cs * log2(e)
    __shared__ float sTot[8];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int h = blockIdx.x, b = blockIdx.z;
    const int64_t seg = blockIdx.y;
    const int grp = h * G / H;
    const int64_t PN = (int64_t)P * N;
    const int64_t c_begin = seg * seg_chunks;
    const int64_t c_end = (c_begin + seg_chunks < nc) ? c_begin + seg_chunks : nc;

    // this wave's state tiles (head-dim tile fastest)
    f32x4 Sacc[TPW];
    bool has_state = false;
#pragma unroll
    for (int s = 0; s < TPW; ++s) Sacc[s] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (FULL) {
        if (src.Sin) {
            const float* S0 = src.Sin + b * src.bstride + seg * src.sstride + (int64_t)h * PN;
#pragma unroll
            for (int s = 0; s < TPW; ++s) {
                const int tile = wave * TPW + s, pt = tile % PT, nt = tile / PT;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    Sacc[s][r] = S0[(pt * 16 + 4 * g4 + r) * N + nt * 16 + l16];
            }
            has_state = true;
        }
    }
    float lam2_total = 0.f;

    const int Ib = RB - 1 - wave, Is = wave;  // this wave's two row blocks

    for (int64_t c = c_begin; c < c_end; ++c) {
        const int64_t t0 = c * Q;
        lds_barrier();  // previous chunk's LDS reads are done

        // ---- issue every global load of the chunk before using any of it:
        // rows past the end of the sequence are clamped to a valid row and
        // zeroed afterwards (selects, no branches), so the loads overlap.
        constexpr int XPT = Q * P / 8 / NT, BPT = Q * N / 8 / NT;
        u32x4 xv[XPT], bv[BPT];
        bf16x8 Cf[2][KN];
        const int64_t last = L - 1 - t0;  // last valid in-chunk row
        float av = 0.f;
        if (tid < Q) av = a[((int64_t)b * L + t0 + (tid <= last ? tid : last)) * H + h];
#pragma unroll
        for (int k = 0; k < XPT; ++k) {
            const int q = tid + k * NT;
            const int j = q / (P / 8), p0 = (q % (P / 8)) * 8;
            const int64_t jr = j <= last ? j : last;
            xv[k] = *reinterpret_cast<const u32x4*>(X + (((int64_t)b * L + t0 + jr) * H + h) * P + p0);
        }
#pragma unroll
        for (int k = 0; k < BPT; ++k) {
            const int q = tid + k * NT;
            const int j = q / (N / 8), n0 = (q % (N / 8)) * 8;
            const int64_t jr = j <= last ? j : last;
            bv[k] = *reinterpret_cast<const u32x4*>(B + (((int64_t)b * L + t0 + jr) * G + grp) * N + n0);
        }
        if constexpr (FULL) {
#pragma unroll
            for (int rbi = 0; rbi < 2; ++rbi) {
                const int i = (rbi == 0 ? Ib : Is) * 16 + l16;
                const int64_t ir = i <= last ? i : last;
#pragma unroll
                for (int kk = 0; kk < KN; ++kk)
                    Cf[rbi][kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(
                        C + (((int64_t)b * L + t0 + ir) * G + grp) * N + 32 * kk + 8 * g4));
            }
        }

        // ---- stage 1: prefix sums of a over the chunk (log2 units) ----
        if (tid > last) av = 0.f;
        const float cs = block_inclusive_scan(av, sTot, Q / 64);
        if (tid < Q) sCs[tid] = cs * kLog2e;
        lds_barrier();
        const float lam2 = sCs[Q - 1];

        // ---- stage chunk tiles into LDS ----
        const u32x4 zero4 = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int k = 0; k < XPT; ++k) {
            const int q = tid + k * NT;
            const int j = q / (P / 8), p0 = (q % (P / 8)) * 8;
            const u32x4 v = j <= last ? xv[k] : zero4;
            const float w = fast_exp2(lam2 - sCs[j]);
            const uint32_t wds[4] = {v[0], v[1], v[2], v[3]};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const u16 xe = (u16)((wds[e >> 1] >> (16 * (e & 1))) & 0xffffu);
                if constexpr (FULL) sXt[(p0 + e) * XLD + j] = xe;
                sWXt[(p0 + e) * XLD + j] = f32_to_bf_bits(w * bf_bits_to_f32(xe));
            }
        }
#pragma unroll
        for (int k = 0; k < BPT; ++k) {
            const int q = tid + k * NT;
            const int j = q / (N / 8), n0 = (q % (N / 8)) * 8;
            *reinterpret_cast<u32x4*>(sB + j * BLD + n0) = j <= last ? bv[k] : zero4;
        }
        if constexpr (FULL) {
#pragma unroll
            for (int rbi = 0; rbi < 2; ++rbi) {
                const int i = (rbi == 0 ? Ib : Is) * 16 + l16;
                if (i > last) {
#pragma unroll
                    for (int kk = 0; kk < KN; ++kk) Cf[rbi][kk] = as_bf16x8(zero4);
                }
            }
            if (has_state) {
#pragma unroll
                for (int s = 0; s < TPW; ++s) {
                    const int tile = wave * TPW + s, pt = tile % PT, nt = tile / PT;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        sS[(pt * 16 + 4 * g4 + r) * SLD + nt * 16 + l16] = f32_to_bf_bits(Sacc[s][r]);
                }
            }
        }
        lds_barrier();

        if constexpr (FULL) {
            f32x4 Yacc[2][PT];
#pragma unroll
            for (int rbi = 0; rbi < 2; ++rbi)
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) Yacc[rbi][pt] = f32x4{0.f, 0.f, 0.f, 0.f};

            // ---- stage 2: diagonal block, (Lmask o S^T)^T X ----
            const float csi_b = sCs[Ib * 16 + l16], csi_s = sCs[Is * 16 + l16];
            const int npairs = (Ib + 2) / 2;
            for (int jp = 0; jp < npairs; ++jp) {
                const int J0 = 2 * jp, J1 = 2 * jp + 1;
                bf16x8 Xf[PT];
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) {
                    const u16* row = sXt + (pt * 16 + l16) * XLD;
                    const uint2 lo = *reinterpret_cast<const uint2*>(row + J0 * 16 + 4 * g4);
                    const uint2 hi = *reinterpret_cast<const uint2*>(row + J1 * 16 + 4 * g4);
                    Xf[pt] = as_bf16x8(u32x4{lo.x, lo.y, hi.x, hi.y});
                }
                bf16x8 Bf0[KN], Bf1[KN];
#pragma unroll
                for (int kk = 0; kk < KN; ++kk) {
                    Bf0[kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(sB + (J0 * 16 + l16) * BLD + 32 * kk + 8 * g4));
                    Bf1[kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(sB + (J1 * 16 + l16) * BLD + 32 * kk + 8 * g4));
                }
                const f32x4 csj0 = *reinterpret_cast<const f32x4*>(sCs + J0 * 16 + 4 * g4);
                const f32x4 csj1 = *reinterpret_cast<const f32x4*>(sCs + J1 * 16 + 4 * g4);
#pragma unroll
                for (int rbi = 0; rbi < 2; ++rbi) {
                    const int I = rbi == 0 ? Ib : Is;
                    if (J0 > I) continue;
                    const float csi = rbi == 0 ? csi_b : csi_s;
                    const int i = I * 16 + l16;
                    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < KN; ++kk) s0 = mfma16x16x32(Bf0[kk], Cf[rbi][kk], s0);
                    const bool has1 = J1 <= I;
                    if (has1) {
#pragma unroll
                        for (int kk = 0; kk < KN; ++kk) s1 = mfma16x16x32(Bf1[kk], Cf[rbi][kk], s1);
                    }
                    bf16x8 Pf;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int j0 = J0 * 16 + 4 * g4 + r, j1 = J1 * 16 + 4 * g4 + r;
                        // exponent is <= 0 on and below the diagonal; clamp so the
                        // masked (i < j) entries never evaluate exp of a large
                        // positive number, then select
                        const float e0 = fast_exp2(fminf(csi - csj0[r], 0.f));
                        const float e1 = fast_exp2(fminf(csi - csj1[r], 0.f));
                        const float v0 = (i >= j0) ? s0[r] * e0 : 0.f;
                        const float v1 = (has1 && i >= j1) ? s1[r] * e1 : 0.f;
                        Pf[r] = f32_to_bf(v0);
                        Pf[4 + r] = f32_to_bf(v1);
                    }
#pragma unroll
                    for (int pt = 0; pt < PT; ++pt) Yacc[rbi][pt] = mfma16x16x32(Pf, Xf[pt], Yacc[rbi][pt]);
                }
            }

            // ---- stage 5: state to output, diag(exp(cs)) C S^T ----
            if (has_state) {
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) {
                    bf16x8 Sf[KN];
#pragma unroll
                    for (int kk = 0; kk < KN; ++kk)
                        Sf[kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(sS + (pt * 16 + l16) * SLD + 32 * kk + 8 * g4));
#pragma unroll
                    for (int rbi = 0; rbi < 2; ++rbi) {
                        const int I = rbi == 0 ? Ib : Is;
                        f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int kk = 0; kk < KN; ++kk) o = mfma16x16x32(Cf[rbi][kk], Sf[kk], o);
                        const f32x4 csr = *reinterpret_cast<const f32x4*>(sCs + I * 16 + 4 * g4);
#pragma unroll
                        for (int r = 0; r < 4; ++r) Yacc[rbi][pt][r] += fast_exp2(csr[r]) * o[r];
                    }
                }
            }

            // ---- write Y (rows 4*g4+r of each row block, column p = lane) ----
#pragma unroll
            for (int rbi = 0; rbi < 2; ++rbi) {
                const int I = rbi == 0 ? Ib : Is;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int64_t t = t0 + I * 16 + 4 * g4 + r;
                    if (t < L) {
                        u16* yrow = Y + (((int64_t)b * L + t) * H + h) * P;
#pragma unroll
                        for (int pt = 0; pt < PT; ++pt) yrow[pt * 16 + l16] = f32_to_bf_bits(Yacc[rbi][pt][r]);
                    }
                }
            }
        }

        // ---- stages 3 + 4: S <- exp(Lam) S + (w o X)^T B ----
        const float dec = fast_exp2(lam2);
#pragma unroll
        for (int s = 0; s < TPW; ++s) Sacc[s] *= dec;
#pragma unroll
        for (int kk = 0; kk < KJ; ++kk) {
            bf16x8 Bg;
#pragma unroll
            for (int s = 0; s < TPW; ++s) {
                const int tile = wave * TPW + s, pt = tile % PT, nt = tile / PT;
                if (s == 0 || pt == 0) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) Bg[e] = bits_to_bf(sB[(32 * kk + 8 * g4 + e) * BLD + nt * 16 + l16]);
                }
                const bf16x8 Af = as_bf16x8(*reinterpret_cast<const u32x4*>(sWXt + (pt * 16 + l16) * XLD + 32 * kk + 8 * g4));
                Sacc[s] = mfma16x16x32(Af, Bg, Sacc[s]);
            }
        }
        has_state = true;
        lam2_total += lam2;
    }

    // ---- epilogue: final state (full pass, last segment) or segment summary ----
    float* Sdst = nullptr;
    if constexpr (FULL) {
        if (S_fin && seg == (int64_t)gridDim.y - 1) Sdst = S_fin + ((int64_t)b * H + h) * PN;
    } else {
        Sdst = Sseg + (((int64_t)b * nseg_total + seg) * H + h) * PN;
        if (lamseg && tid == 0) lamseg[((int64_t)b * H + h) * nseg_total + seg] = lam2_total * 0.69314718055994531f;
    }
    if (Sdst) {
#pragma unroll
        for (int s = 0; s < TPW; ++s) {
            const int tile = wave * TPW + s, pt = tile % PT, nt = tile / PT;
#pragma unroll
            for (int r = 0; r < 4; ++r) Sdst[(pt * 16 + 4 * g4 + r) * N + nt * 16 + l16] = Sacc[s][r];
        }
    }
}

bool mfma_supported(int64_t Q, int64_t P, int64_t N) {
    return (Q == 64 || Q == 128 || Q == 256) && (P == 32 || P == 64) && (N == 64 || N == 128);
}

#define SSD_MFMA_DISPATCH(MACRO)                                   \
    if (s.Q == 256 && s.P == 64 && s.N == 128) MACRO(256, 64, 128) \
    else if (s.Q == 256 && s.P == 64 && s.N == 64) MACRO(256, 64, 64) \
    else if (s.Q == 256 && s.P == 32 && s.N == 128) MACRO(256, 32, 128) \
    else if (s.Q == 256 && s.P == 32 && s.N == 64) MACRO(256, 32, 64) \
    else if (s.Q == 128 && s.P == 64 && s.N == 128) MACRO(128, 64, 128) \
    else if (s.Q == 128 && s.P == 64 && s.N == 64) MACRO(128, 64, 64) \
    else if (s.Q == 128 && s.P == 32 && s.N == 128) MACRO(128, 32, 128) \
    else if (s.Q == 128 && s.P == 32 && s.N == 64) MACRO(128, 32, 64) \
    else if (s.Q == 64 && s.P == 64 && s.N == 128) MACRO(64, 64, 128) \
    else if (s.Q == 64 && s.P == 64 && s.N == 64) MACRO(64, 64, 64) \
    else if (s.Q == 64 && s.P == 32 && s.N == 128) MACRO(64, 32, 128) \
    else if (s.Q == 64 && s.P == 32 && s.N == 64) MACRO(64, 32, 64) \
    else return hipErrorInvalidValue;

hipError_t launch_mfma_state(const FwdShape& s, int64_t seg_chunks, int64_t nseg_run,
                             int64_t nseg_total, const void* X, const float* a,
                             const void* B, float* Sseg, float* lamseg, hipStream_t st)
{
    if (nseg_run <= 0) return hipSuccess;
    const dim3 grid((unsigned)s.H, (unsigned)nseg_run, (unsigned)s.Bz);
    const StateSrc none{nullptr, 0, 0};
#define SSD_LAUNCH_STATE(QQ, PP, NN)                                                          \
    hipLaunchKernelGGL((k_mfma_seg<QQ, PP, NN, false>), grid, dim3(QQ * 2), 0, st,          \
                       (const u16*)X, a, (const u16*)B, (const u16*)nullptr, none,          \
                       (u16*)nullptr, (float*)nullptr, Sseg, lamseg, nseg_total, s.L,       \
                       (int)s.H, (int)s.G, s.nc, seg_chunks);
    SSD_MFMA_DISPATCH(SSD_LAUNCH_STATE)
#undef SSD_LAUNCH_STATE
    return hipGetLastError();
}

hipError_t launch_mfma_out(const FwdShape& s, int64_t seg_chunks, int64_t nseg,
                           const void* X, const float* a, const void* B, const void* C,
                           StateSrc src, void* Y, float* S_fin, hipStream_t st)
{
    const dim3 grid((unsigned)s.H, (unsigned)nseg, (unsigned)s.Bz);
#define SSD_LAUNCH_OUT(QQ, PP, NN)                                                            \
    hipLaunchKernelGGL((k_mfma_seg<QQ, PP, NN, true>), grid, dim3(QQ * 2), 0, st,           \
                       (const u16*)X, a, (const u16*)B, (const u16*)C, src, (u16*)Y, S_fin, \
                       (float*)nullptr, (float*)nullptr, (int64_t)0, s.L, (int)s.H,          \
                       (int)s.G, s.nc, seg_chunks);
    SSD_MFMA_DISPATCH(SSD_LAUNCH_OUT)
#undef SSD_LAUNCH_OUT
    return hipGetLastError();
}

}  // namespace ssd
