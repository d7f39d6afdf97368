// kernels_mfma.hip -- bf16 MFMA kernels of the SSD layer for gfx950.
//
// The layer's sequence map is the 1-semiseparable matrix M = Lmask o (C B^T)
// applied to X (wiki review of "Transformers are SSMs", section "Core
// concepts"; CiteArk page, section "AI research summary": a block-decomposed
// matrix-multiplication algorithm over that matrix).  Blocking the sequence
// into chunks of Q steps gives, per chunk c:
//   1. in-chunk prefix sums cs of a (wavefront scans, fp32);
//   2. diagonal block:   Ydiag = (Lmask_cc o C_c B_c^T) X_c               (MFMA)
//   3. chunk state:      dS_c  = X_c^T diag(w) B_c, w_j = exp(Lam_c - cs_j) (MFMA)
//   4. state passing:    S_{c+1} = exp(Lam_c) S_c + dS_c   (fp32, in registers)
//   5. state to output:  Yoff = diag(exp(cs)) C_c S_c^T                    (MFMA)
//
// One workgroup walks `seg_chunks` consecutive chunks of one (batch, head),
// carrying the fp32 P x N state in MFMA accumulators, so states never
// round-trip HBM inside a segment.  When a launch would leave CUs idle the
// sequence is split into segments: a state-only pass (stages 1, 3, 4) gives
// each segment's end state from zero, a scan over segments (kernels_scan.hip)
// gives every segment's entering state, and the full pass starts from it.
//
// Mapping onto gfx950.
//  * Workgroup = Q/64 wavefronts.  32-step row blocks are dealt to waves in
//    pairs (w, Q/32-1-w) so every wave owns the same number of causal 32x32
//    score tiles.  Every product is v_mfma_f32_32x32x16_bf16 (operand lane l
//    holds row/column l%32 and the 8 k values of group l/32; the accumulator
//    holds column l%32, rows 8(r/4) + 4(l/32) + r%4).
//  * Every input reaches LDS through asynchronous global_load_lds copies
//    (lane L of a wave-wide copy lands at LDS base + L * size), issued one
//    phase ahead of use, so HBM traffic overlaps the MFMA work and no register
//    holds prefetched data.  A chunk is consumed in two halves of Q/2 steps
//    (the contraction index j of stages 2 and 3); X and B halves are double
//    buffered, a and C single buffered (C in two row halves, moved into
//    operand registers as soon as they land).  Each buffer is guarded by an
//    explicit vmcnt wait (vector-memory operations complete in issue order)
//    followed by an LDS-only barrier.  The copies are written in inline
//    assembly: they have no register result, and keeping them out of the
//    compiler's view stops it from inserting full vmcnt waits before every
//    LDS access, which would serialise the prefetch.
//  * LDS tiles are unpadded row-major with the 16-byte pieces of row r stored
//    at piece ^ (r mod pieces-per-row), so the 16-byte row reads and the
//    transposing reads below touch distinct banks.
//  * Scores are formed transposed, S^T = B C^T, so lane = step i and the
//    registers hold steps j: after the decay mask they are directly the
//    B operand of Y^T = X^T (Lmask o S)^T.  Operands that need j along a
//    lane's registers (X^T for stage 2; B^T and X for stage 3) come from
//    ds_read_b64_tr_b16: in each 16-lane group, source lane m names row
//    R(m/4), columns 4(m%4)..+3, and output lane i receives column i of rows
//    R(0..3).  Outputs are Y^T tiles: a lane holds 4 consecutive head-dim
//    entries of one step, an 8-byte store.
//  * Workgroups are dealt to the 8 XCDs in contiguous ranges of (batch,
//    segment, head) items, so the heads that share a batch's B and C run on
//    one XCD and read them through one L2.
// Operand rounding: (Lmask o S), w o X, exp(cs) C and the entering state are
// rounded to bf16 for the MFMA; every accumulation is fp32.
#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));  // register-friendly 16-byte piece
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kXcds = 8;  // MI355X accelerator complex dies; workgroups alternate over them

template <int Q, int P, int N>
struct MfmaCfg {
    static constexpr int NW = Q / 64;        // wavefronts
    static constexpr int NT = Q;             // threads: one per step of the chunk
    static constexpr int RB = Q / 32;        // 32-step row blocks
    static constexpr int RBH = RB / 2;       // row blocks per half
    static constexpr int JH = Q / 2;         // steps per half
    static constexpr int KN = N / 16;        // k steps over the state dim
    static constexpr int KJH = JH / 16;      // k steps over one half of the chunk
    static constexpr int PT = P / 32;        // 32-wide head-dim tiles
    static constexpr int TT = PT * (N / 32); // state tiles
    static constexpr int TPW = TT / NW;      // state tiles per wave
    static constexpr int XPR = P / 8;        // 16-byte pieces per X row
    static constexpr int BPR = N / 8;        // 16-byte pieces per B, C and state row
    static constexpr int XPH = JH * XPR / NT;  // X copies per thread per half
    static constexpr int BPH = JH * BPR / NT;  // B (or C) copies per thread per half
    static constexpr int NH = XPH + BPH;       // copies of one X+B half
    static_assert(Q % 64 == 0 && P % 32 == 0 && N % 32 == 0, "tile shape");
    static_assert(TT % NW == 0, "state tiles must split evenly over waves");
    static_assert(XPH >= 1 && BPH >= 1, "half tiles must cover the workgroup");
};

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ u32x4 as_u32x4(bf16x8 v) { return __builtin_bit_cast(u32x4, v); }
__device__ __forceinline__ i16x4 lds_tr4(const u16* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}
__device__ __forceinline__ bf16x8 join8(i16x4 lo, i16x4 hi) {
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
}
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    return (uint32_t)f32_to_bf_bits(lo) | ((uint32_t)f32_to_bf_bits(hi) << 16);
}
__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int r = 0; r < 16; ++r) z[r] = 0.f;
    return z;
}
// bf16x8 scaled elementwise in fp32 and rounded back
__device__ __forceinline__ bf16x8 scale8(bf16x8 v, const float (&s)[8]) {
    const u32x4 u = as_u32x4(v);
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        o[e] = pack2(s[2 * e] * __uint_as_float(u[e] << 16), s[2 * e + 1] * __uint_as_float(u[e] & 0xffff0000u));
    return as_bf16x8(o);
}
__device__ __forceinline__ bf16x8 scale8(bf16x8 v, float s) {
    const u32x4 u = as_u32x4(v);
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        o[e] = pack2(s * __uint_as_float(u[e] << 16), s * __uint_as_float(u[e] & 0xffff0000u));
    return as_bf16x8(o);
}

// Element offset of (row, col) in a swizzled row-major tile of PR 16-byte
// pieces per row (col a multiple of 4 for 8-byte accesses, of 8 for 16-byte).
template <int PR>
__device__ __forceinline__ int swz(int row, int col) {
    return row * (PR * 8) + ((((col >> 3) ^ (row & (PR - 1))) << 3) | (col & 7));
}

// ---- asynchronous HBM -> LDS copies and their synchronisation -----------------
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) char*)p);
}
// 16 (or 4) bytes per lane from `g`; lane L writes LDS byte lds + 16 L (4 L).
// `lds` must be wave-uniform (it is moved into M0).
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(g), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* g, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
                 :: "v"(g), "s"(lds) : "memory", "m0");
}
// at most N of this wave's vector-memory operations outstanding
template <int N>
__device__ __forceinline__ void vm_wait() {
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}
// workgroup barrier ordering LDS only (no wait on HBM traffic)
__device__ __forceinline__ void sync_lds() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Copy rows [j0, j0 + ROWS) of a chunk tile (HBM row stride `stride`
// elements, PR pieces per row) into a swizzled LDS tile.  Wave w, step k
// fills LDS pieces (k*NT + 64w) .. +63.  Rows past the end of the sequence
// are clamped to the last valid row: their data never reaches an output
// (their scores are masked, their chunk-state weight and C rows are zero).
template <int NT, int PR, int ROWS>
__device__ __forceinline__ void dma_tile(const u16* lds, const u16* __restrict__ gbase, int stride, int j0,
                                         int lastc, int wave, int lane) {
    const uint32_t base = lds_addr(lds);
#pragma unroll
    for (int k = 0; k < ROWS * PR / NT; ++k) {
        const int slot = k * NT + wave * 64 + lane;
        const int r = slot / PR, pp = slot % PR;
        const int lp = pp ^ (r & (PR - 1));
        const int jr = j0 + r <= lastc ? j0 + r : lastc;
        dma16(gbase + (uint32_t)(jr * stride + lp * 8), base + (uint32_t)((k * NT + wave * 64) * 16));
    }
}

// Inclusive prefix sum over the workgroup (one value per thread).  s_tot may
// be reused only after a later barrier.
__device__ __forceinline__ float block_scan(float v, float* s_tot, int nwaves, int lane, int wave) {
    v = wave_inclusive_scan(v);
    if (lane == 63) s_tot[wave] = v;
    sync_lds();
    float add = 0.f;
    for (int w = 0; w < wave && w < nwaves; ++w) add += s_tot[w];
    return v + add;
}

template <int Q, int P, int N, bool FULL>
__global__ __launch_bounds__(Q) void k_mfma_seg(
    const u16* __restrict__ X, const float* __restrict__ a, const u16* __restrict__ B,
    const u16* __restrict__ C, StateSrc src, u16* __restrict__ Y, float* __restrict__ S_fin,
    float* __restrict__ Sseg, float* __restrict__ lamseg, int64_t nseg_total, int64_t L,
    int H, int G, int64_t nc, int64_t seg_chunks, int nseg_grid, int Bz)
{
    using Cfg = MfmaCfg<Q, P, N>;
    constexpr int NW = Cfg::NW, NT = Cfg::NT, RB = Cfg::RB, RBH = Cfg::RBH, JH = Cfg::JH;
    constexpr int KN = Cfg::KN, KJH = Cfg::KJH, PT = Cfg::PT, TPW = Cfg::TPW;
    constexpr int XPR = Cfg::XPR, BPR = Cfg::BPR, NHV = Cfg::NH;

    __shared__ __attribute__((aligned(16))) u16 sB0[JH * N];   // B rows of half 0 (swizzled)
    __shared__ __attribute__((aligned(16))) u16 sB1[JH * N];   // B rows of half 1
    __shared__ __attribute__((aligned(16))) u16 sX0[JH * P];   // X rows of half 0
    __shared__ __attribute__((aligned(16))) u16 sX1[JH * P];   // X rows of half 1
    __shared__ __attribute__((aligned(16))) u16 sC[FULL ? JH * N : 8];  // one row half of C
    __shared__ __attribute__((aligned(16))) u16 sS[FULL ? P * N : 8];   // entering state, bf16 [p][n]
    __shared__ __attribute__((aligned(16))) float sA[Q];       // a of the chunk
    __shared__ __attribute__((aligned(16))) float sCs[Q];      // cs * log2(e)
    __shared__ __attribute__((aligned(16))) float sW[Q];       // exp(Lam - cs_j), 0 past the end
    __shared__ float sTot[8];

    // ---- work item: contiguous item ranges per XCD (heads fastest) ----
    const int64_t items = (int64_t)Bz * nseg_grid * H;
    const int64_t per_xcd = gridDim.x / kXcds;
    const int64_t item = (int64_t)(blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
    if (item >= items) return;
    const int h = (int)(item % H);
    const int64_t seg = (item / H) % nseg_grid;
    const int b = (int)(item / H / nseg_grid);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, g2 = lane >> 5;
    const int trow = (lane & 15) >> 2, tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    const int grp = h * G / H;
    const int64_t PN = (int64_t)P * N;
    const int64_t c_begin = seg * seg_chunks;
    const int64_t c_end = (c_begin + seg_chunks < nc) ? c_begin + seg_chunks : nc;
    const int Ib = RB - 1 - wave, Is = wave;  // this wave's two row blocks
    const int GN = G * N, HP = H * P;

    auto chunk_last = [&](int64_t c) -> int {
        const int64_t last = L - 1 - c * Q;
        return (int)(last < Q - 1 ? last : Q - 1);
    };
    auto dma_a = [&](int64_t c) {
        const int lc = chunk_last(c);
        const float* ab = a + ((int64_t)b * L + c * Q) * H + h;
        dma4(ab + (uint32_t)((tid <= lc ? tid : lc) * H), lds_addr(sA) + (uint32_t)(wave * 256));
    };
    auto dma_c = [&](int64_t c, int half) {  // C rows [half*JH, half*JH + JH)
        dma_tile<NT, BPR, JH>(sC, C + (((int64_t)b * L + c * Q) * G + grp) * N, GN, half * JH,
                              chunk_last(c), wave, lane);
    };
    auto dma_half = [&](int64_t c, int half) {
        const int lc = chunk_last(c);
        dma_tile<NT, XPR, JH>(half ? sX1 : sX0, X + (((int64_t)b * L + c * Q) * H + h) * P, HP,
                              half * JH, lc, wave, lane);
        dma_tile<NT, BPR, JH>(half ? sB1 : sB0, B + (((int64_t)b * L + c * Q) * G + grp) * N, GN,
                              half * JH, lc, wave, lane);
    };

    // ---- carried state: this wave's 32x32 tiles of S^T (rows n, columns p) ----
    f32x16 Sacc[TPW];
    bool has_state = false;
#pragma unroll
    for (int s = 0; s < TPW; ++s) Sacc[s] = zero16();
    if constexpr (FULL) {
        if (src.Sin) {
            const float* S0 = src.Sin + b * src.bstride + seg * src.sstride + (int64_t)h * PN;
#pragma unroll
            for (int s = 0; s < TPW; ++s) {
                const int tile = wave * TPW + s, pt = tile % PT, nt = tile / PT;
                const float* row = S0 + (int64_t)(pt * 32 + l32) * N + nt * 32 + 4 * g2;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float4 v = *reinterpret_cast<const float4*>(row + 8 * q);
                    Sacc[s][4 * q + 0] = v.x;
                    Sacc[s][4 * q + 1] = v.y;
                    Sacc[s][4 * q + 2] = v.z;
                    Sacc[s][4 * q + 3] = v.w;
                }
            }
            has_state = true;
        }
    }
    float lam2_total = 0.f;

    // prologue copies, in the order the loop expects: a, C (upper rows), X+B half 0, half 1
    dma_a(c_begin);
    if constexpr (FULL) dma_c(c_begin, 1);
    dma_half(c_begin, 0);
    dma_half(c_begin, 1);

    for (int64_t c = c_begin; c < c_end; ++c) {
        const int64_t t0 = c * Q;
        const int last = chunk_last(c);
        const bool has_next = c + 1 < c_end;

        vm_wait<NHV>();  // a, upper C and half 0 of this chunk have landed (half 1 may fly)
        sync_lds();

        // ---- stage 1: prefix sums of a, chunk-state weights ----
        const float cs = block_scan(tid <= last ? sA[tid] : 0.f, sTot, NW, lane, wave);
        sCs[tid] = cs * kLog2e;
        sync_lds();
        const float lam2 = sCs[Q - 1];
        sW[tid] = tid <= last ? fast_exp2(lam2 - sCs[tid]) : 0.f;
        bf16x8 Cc[2][KN];
        float csi[2] = {0.f, 0.f};
        if constexpr (FULL) {
            csi[0] = sCs[Ib * 32 + l32];
            csi[1] = sCs[Is * 32 + l32];
            const bool ok = Ib * 32 + l32 <= last;
#pragma unroll
            for (int kk = 0; kk < KN; ++kk)
                Cc[0][kk] = ok ? as_bf16x8(*reinterpret_cast<const u32x4*>(
                                     sC + swz<BPR>((Ib - RBH) * 32 + l32, 16 * kk + 8 * g2)))
                               : as_bf16x8(u32x4{0u, 0u, 0u, 0u});
            if (has_state) {  // entering state, bf16, for stage 5
#pragma unroll
                for (int s = 0; s < TPW; ++s) {
                    const int tile = wave * TPW + s, pt = tile % PT, nt = tile / PT;
                    const int p = pt * 32 + l32;
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        *reinterpret_cast<uint2*>(sS + swz<BPR>(p, nt * 32 + 8 * q + 4 * g2)) =
                            make_uint2(pack2(Sacc[s][4 * q], Sacc[s][4 * q + 1]),
                                       pack2(Sacc[s][4 * q + 2], Sacc[s][4 * q + 3]));
                }
            }
        }
        sync_lds();  // sA and the upper C rows are consumed; sW, sS visible
        if constexpr (FULL) dma_c(c, 0);    // lower C rows
        else if (has_next) dma_a(c + 1);

        f32x16 Yt[2][PT];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) Yt[rb][pt] = zero16();
        const float dec = fast_exp2(lam2);
#pragma unroll
        for (int s = 0; s < TPW; ++s) Sacc[s] *= dec;

        // one causal 32x32 tile (I, J): Y^T[rb] += X_J^T (Lmask o S)^T
        auto tile = [&](const u16* sBh, const u16* sXh, int rb, int I, int J, int J0) {
            const int rJ = (J - J0) * 32;
            f32x16 St = zero16();
#pragma unroll
            for (int kk = 0; kk < KN; ++kk) {
                const bf16x8 Bf = as_bf16x8(*reinterpret_cast<const u32x4*>(
                    sBh + swz<BPR>(rJ + l32, 16 * kk + 8 * g2)));
                St = mfma32(Bf, Cc[rb][kk], St);
            }
            bf16x8 Xa[2][PT];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) {
                    const int r1 = rJ + 16 * ks + 4 * g2 + trow;
                    Xa[ks][pt] = join8(lds_tr4(sXh + swz<XPR>(r1, pt * 32 + tcol)),
                                       lds_tr4(sXh + swz<XPR>(r1 + 8, pt * 32 + tcol)));
                }
            float csj[16];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 v = *reinterpret_cast<const f32x4*>(sCs + J * 32 + 8 * q + 4 * g2);
                csj[4 * q] = v[0]; csj[4 * q + 1] = v[1]; csj[4 * q + 2] = v[2]; csj[4 * q + 3] = v[3];
            }
            const bool diag = (J == I);
            bf16x8 Pf[2];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                // row j = 8(r/4) + 4*g2 + r%4 of the tile, column i = l32;
                // masked entries (j > i) are replaced, never multiplied
                const int jl = 8 * (r >> 2) + 4 * g2 + (r & 3);
                float v = St[r] * fast_exp2(csi[rb] - csj[r]);
                if (diag && jl > l32) v = 0.f;
                Pf[r >> 3][r & 7] = f32_to_bf(v);
            }
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) Yt[rb][pt] = mfma32(Xa[ks][pt], Pf[ks], Yt[rb][pt]);
        };
        // stages 3 + 4 over one half: S^T += B^T diag(w) X
        auto chunk_state_half = [&](const u16* sBh, const u16* sXh, int half) {
#pragma unroll
            for (int kj = 0; kj < KJH; ++kj) {
                const int r0 = kj * 16 + 8 * g2 + trow;
                float w[8];
                const f32x4 w0 = *reinterpret_cast<const f32x4*>(sW + half * JH + kj * 16 + 8 * g2);
                const f32x4 w1 = *reinterpret_cast<const f32x4*>(sW + half * JH + kj * 16 + 8 * g2 + 4);
                w[0] = w0[0]; w[1] = w0[1]; w[2] = w0[2]; w[3] = w0[3];
                w[4] = w1[0]; w[5] = w1[1]; w[6] = w1[2]; w[7] = w1[3];
                bf16x8 Af, Bx;
                int cur_nt = -1, cur_pt = -1;
#pragma unroll
                for (int s = 0; s < TPW; ++s) {
                    const int tl = wave * TPW + s, pt = tl % PT, nt = tl / PT;
                    if (nt != cur_nt) {
                        Af = join8(lds_tr4(sBh + swz<BPR>(r0, nt * 32 + tcol)),
                                   lds_tr4(sBh + swz<BPR>(r0 + 4, nt * 32 + tcol)));
                        cur_nt = nt;
                    }
                    if (pt != cur_pt) {
                        Bx = scale8(join8(lds_tr4(sXh + swz<XPR>(r0, pt * 32 + tcol)),
                                          lds_tr4(sXh + swz<XPR>(r0 + 4, pt * 32 + tcol))), w);
                        cur_pt = pt;
                    }
                    Sacc[s] = mfma32(Af, Bx, Sacc[s]);
                }
            }
        };

        // ================= half 0: steps [0, Q/2) of the chunk =================
        if constexpr (FULL) {
            for (int J = 0; J < RBH; ++J) tile(sB0, sX0, 0, Ib, J, 0);  // upper row block
            vm_wait<0>();  // the lower C rows have landed (and half 1 with them)
            sync_lds();
            const bool ok = Is * 32 + l32 <= last;
#pragma unroll
            for (int kk = 0; kk < KN; ++kk)
                Cc[1][kk] = ok ? as_bf16x8(*reinterpret_cast<const u32x4*>(
                                     sC + swz<BPR>(Is * 32 + l32, 16 * kk + 8 * g2)))
                               : as_bf16x8(u32x4{0u, 0u, 0u, 0u});
            sync_lds();  // every wave has its C rows: sC and sA are free
            if (has_next) {
                dma_a(c + 1);
                dma_c(c + 1, 1);
            }
            for (int J = 0; J <= Is; ++J) tile(sB0, sX0, 1, Is, J, 0);  // lower row block
        }
        chunk_state_half(sB0, sX0, 0);

        sync_lds();  // every wave is done with buffer 0
        if (has_next) {
            dma_half(c + 1, 0);
            vm_wait<NHV>();  // half 1 of this chunk has landed (the copies just issued may fly)
        } else {
            vm_wait<0>();
        }
        sync_lds();

        // ================= half 1: steps [Q/2, Q) =================
        if constexpr (FULL) {
            for (int J = RBH; J <= Ib; ++J) tile(sB1, sX1, 0, Ib, J, RBH);
        }
        chunk_state_half(sB1, sX1, 1);
        if constexpr (FULL) {
            // ---- stage 5: Y^T += S (diag(exp(cs)) C)^T ----
            if (has_state) {
#pragma unroll
                for (int rb = 0; rb < 2; ++rb) {
                    const float sc = fast_exp2(csi[rb]);
#pragma unroll
                    for (int kk = 0; kk < KN; ++kk) Cc[rb][kk] = scale8(Cc[rb][kk], sc);
                }
#pragma unroll
                for (int pt = 0; pt < PT; ++pt)
#pragma unroll
                    for (int kk = 0; kk < KN; ++kk) {
                        const bf16x8 Sf = as_bf16x8(*reinterpret_cast<const u32x4*>(
                            sS + swz<BPR>(pt * 32 + l32, 16 * kk + 8 * g2)));
#pragma unroll
                        for (int rb = 0; rb < 2; ++rb) Yt[rb][pt] = mfma32(Sf, Cc[rb][kk], Yt[rb][pt]);
                    }
            }
            // ---- write Y: lane = step i, 4 consecutive head-dim entries per store ----
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                const int i = (rb == 0 ? Ib : Is) * 32 + l32;
                if (i <= last) {
                    u16* yrow = Y + (((int64_t)b * L + t0 + i) * H + h) * P + 4 * g2;
#pragma unroll
                    for (int pt = 0; pt < PT; ++pt)
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            *reinterpret_cast<uint2*>(yrow + pt * 32 + 8 * q) =
                                make_uint2(pack2(Yt[rb][pt][4 * q], Yt[rb][pt][4 * q + 1]),
                                           pack2(Yt[rb][pt][4 * q + 2], Yt[rb][pt][4 * q + 3]));
                }
            }
        }

        sync_lds();  // every wave is done with buffer 1, sCs, sW and sS
        if (has_next) dma_half(c + 1, 1);
        has_state = true;
        lam2_total += lam2;
    }

    // ---- epilogue: final state (full pass, last segment) or segment summary ----
    float* Sdst = nullptr;
    if constexpr (FULL) {
        if (S_fin && seg == nseg_grid - 1) Sdst = S_fin + ((int64_t)b * H + h) * PN;
    } else {
        Sdst = Sseg + (((int64_t)b * nseg_total + seg) * H + h) * PN;
        if (lamseg && tid == 0) lamseg[((int64_t)b * H + h) * nseg_total + seg] = lam2_total * 0.69314718055994531f;
    }
    if (Sdst) {
#pragma unroll
        for (int s = 0; s < TPW; ++s) {
            const int tl = wave * TPW + s, pt = tl % PT, nt = tl / PT;
            float* row = Sdst + (int64_t)(pt * 32 + l32) * N + nt * 32 + 4 * g2;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                *reinterpret_cast<float4*>(row + 8 * q) =
                    make_float4(Sacc[s][4 * q], Sacc[s][4 * q + 1], Sacc[s][4 * q + 2], Sacc[s][4 * q + 3]);
        }
    }
}

bool mfma_supported(int64_t Q, int64_t P, int64_t N) {
    if (!((Q == 64 || Q == 128 || Q == 256) && (P == 32 || P == 64) && (N == 64 || N == 128))) return false;
    return ((P / 32) * (N / 32)) % (Q / 64) == 0;
}

#define SSD_MFMA_DISPATCH(MACRO)                                        \
    if (s.Q == 256 && s.P == 64 && s.N == 128) MACRO(256, 64, 128)      \
    else if (s.Q == 256 && s.P == 64 && s.N == 64) MACRO(256, 64, 64)   \
    else if (s.Q == 256 && s.P == 32 && s.N == 128) MACRO(256, 32, 128) \
    else if (s.Q == 128 && s.P == 64 && s.N == 128) MACRO(128, 64, 128) \
    else if (s.Q == 128 && s.P == 64 && s.N == 64) MACRO(128, 64, 64)   \
    else if (s.Q == 128 && s.P == 32 && s.N == 128) MACRO(128, 32, 128) \
    else if (s.Q == 128 && s.P == 32 && s.N == 64) MACRO(128, 32, 64)   \
    else if (s.Q == 64 && s.P == 64 && s.N == 128) MACRO(64, 64, 128)   \
    else if (s.Q == 64 && s.P == 64 && s.N == 64) MACRO(64, 64, 64)     \
    else if (s.Q == 64 && s.P == 32 && s.N == 128) MACRO(64, 32, 128)   \
    else if (s.Q == 64 && s.P == 32 && s.N == 64) MACRO(64, 32, 64)     \
    else return hipErrorInvalidValue;

// one workgroup per (batch, segment, head) item, padded to a multiple of the XCD count
static unsigned grid_for(int64_t items) {
    return (unsigned)(((items + kXcds - 1) / kXcds) * kXcds);
}

hipError_t launch_mfma_state(const FwdShape& s, int64_t seg_chunks, int64_t nseg_run,
                             int64_t nseg_total, const void* X, const float* a,
                             const void* B, float* Sseg, float* lamseg, hipStream_t st)
{
    if (nseg_run <= 0) return hipSuccess;
    const dim3 grid(grid_for(s.Bz * nseg_run * s.H));
    const StateSrc none{nullptr, 0, 0};
#define SSD_LAUNCH_STATE(QQ, PP, NN)                                                          \
    hipLaunchKernelGGL((k_mfma_seg<QQ, PP, NN, false>), grid, dim3(QQ), 0, st,              \
                       (const u16*)X, a, (const u16*)B, (const u16*)nullptr, none,          \
                       (u16*)nullptr, (float*)nullptr, Sseg, lamseg, nseg_total, s.L,       \
                       (int)s.H, (int)s.G, s.nc, seg_chunks, (int)nseg_run, (int)s.Bz);
    SSD_MFMA_DISPATCH(SSD_LAUNCH_STATE)
#undef SSD_LAUNCH_STATE
    return hipGetLastError();
}

hipError_t launch_mfma_out(const FwdShape& s, int64_t seg_chunks, int64_t nseg,
                           const void* X, const float* a, const void* B, const void* C,
                           StateSrc src, void* Y, float* S_fin, hipStream_t st)
{
    const dim3 grid(grid_for(s.Bz * nseg * s.H));
#define SSD_LAUNCH_OUT(QQ, PP, NN)                                                            \
    hipLaunchKernelGGL((k_mfma_seg<QQ, PP, NN, true>), grid, dim3(QQ), 0, st,               \
                       (const u16*)X, a, (const u16*)B, (const u16*)C, src, (u16*)Y, S_fin, \
                       (float*)nullptr, (float*)nullptr, (int64_t)0, s.L, (int)s.H,          \
                       (int)s.G, s.nc, seg_chunks, (int)nseg, (int)s.Bz);
    SSD_MFMA_DISPATCH(SSD_LAUNCH_OUT)
#undef SSD_LAUNCH_OUT
    return hipGetLastError();
}

}  // namespace ssd
