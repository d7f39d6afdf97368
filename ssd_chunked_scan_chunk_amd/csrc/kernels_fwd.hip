// kernels_fwd.hip -- the fused forward pass of the SSD layer (bf16 MFMA,
// gfx950), one barrier per block.
//
// The layer's sequence map is the 1-semiseparable matrix M = Lmask o (C B^T)
// applied to X (wiki review of "Transformers are SSMs", section "Core
// concepts"; CiteArk page, section "AI research summary": a block-decomposed
// matrix-multiplication algorithm over that matrix).  Per 64-step block c:
//   1. prefix sums cs of a (wavefront scans, fp32) and the decay scales;
//   2. diagonal block   Ydiag = (Lmask_cc o C_c B_c^T) X_c             (MFMA)
//   3. block state      dS_c  = X_c^T diag(w) B_c                       (MFMA)
//   4. state passing    S_{c+1} = exp(Lam_c) S_c + dS_c  (fp32, in the MFMA
//                       accumulators, the decay kept as a power-of-two scale)
//   5. state to output  Yoff  = diag(exp(cs)) C_c S_c^T                  (MFMA)
// with the same factorisation of the decay as the segmented kernel
// (kernels_mfma.hip): the masked scores C_i . B_j are the same for every head
// of a group, X is weighted per step and the output scaled per step.
//
// Work split.  A unit is one 32-wide head-dim slice of one head; its slice of
// the fp32 state (32 x N) lives in one wavefront's MFMA accumulators for the
// whole segment.  A workgroup holds SW such state waves over consecutive units
// of one group (so they share B and C) plus two helper waves:
//  * the X wave streams X two blocks ahead into three LDS buffers with
//    asynchronous global_load_lds copies (it issues no stores, so its vmcnt
//    waits are exact), copies a two blocks ahead, and runs stage 1 (the scans
//    and the scale decisions of every head the units touch) one block ahead;
//  * the score wave copies B and C of the next block into LDS as soon as
//    their buffers are free (right after the block's barrier), and forms the
//    next block's three causal 32x32 score tiles from them.
// Everything a block needs is therefore ready when it starts, and a block has
// exactly one barrier: it publishes the block's X, B, C, scores and stage-1
// results and frees the buffers of the block before.  With SW a template
// parameter the host picks the split that fills the 256 CUs (the 2.7B-shaped
// layer has 8 x 80 x 2 = 1280 units: 256 workgroups of five).
//
// Operand rounding as in the segmented kernel: masked scores, X weighted by
// the state weights and the carried state are bf16 MFMA operands; every
// accumulation and the per-step output factor are fp32.
#include <type_traits>

#include "mfma_util.hpp"
#include "ssd_launch.hpp"

namespace ssd {

// Most heads that sw consecutive units starting at a multiple of sw can
// touch, with ps units per head.
constexpr int heads_touched(int sw, int ps) {
    int m = 0;
    for (int q = 0; q < ps; ++q) {
        const int u0 = q * sw;
        const int n = (u0 + sw - 1) / ps - u0 / ps + 1;
        m = n > m ? n : m;
    }
    return m;
}

template <int P, int N, int SW>
struct FwdCfg {
    static constexpr int PS = P / 32;              // units per head
    static constexpr int NTL = N / 32;             // 32-wide state-dim tiles
    static constexpr int BPR = N / 8;              // 16-byte pieces per B / C row
    static constexpr int XPU = 4;                  // 16-byte pieces per row of a unit's X tile (32 p)
    static constexpr int HWX = heads_touched(SW, PS);   // heads one workgroup's units touch, at most
    static constexpr int NXB = 3;                  // X buffers: two blocks in flight
    static constexpr int NW = SW + 2;              // wavefronts per workgroup
    static constexpr int XOPS = SW * kT * XPU / 64;   // X copies (64 lanes x 16 bytes) per block
    static_assert(P % 32 == 0 && N % 32 == 0 && SW >= 2 && NW <= 8, "shape");
};

template <int P, int N, int SW, bool REV = false>
__global__ __launch_bounds__(64 * (SW + 2)) __attribute__((amdgpu_waves_per_eu(2))) void k_fwd(
    const u16* __restrict__ X, const float* __restrict__ a, const u16* __restrict__ B,
    const u16* __restrict__ C, StateSrc src, u16* __restrict__ Y, float* __restrict__ S_fin,
    const float* __restrict__ fin_a, int64_t fin_a_bstride, int64_t L, int H, int G,
    int64_t blocks_per_seg, int nseg_grid, int Bz)
{
    using Cfg = FwdCfg<P, N, SW>;
    constexpr int PS = Cfg::PS, NTL = Cfg::NTL, XPU = Cfg::XPU, HWX = Cfg::HWX;
    constexpr int SUB = kT * 32;                   // elements of one 32-column sub-tile
    constexpr int NXB = Cfg::NXB, XOPS = Cfg::XOPS;

    __shared__ __attribute__((aligned(16))) u16 sX[NXB][SW][kT * 32];   // [buf][unit][step][32 p]
    // B and C as 32-column sub-tiles [buf][n / 32][step][32], each swizzled
    // like a unit's X tile: the sub-tile and row-block parts of every operand
    // address are then instruction immediates
    __shared__ __attribute__((aligned(16))) u16 sB[2][kT * N];
    __shared__ __attribute__((aligned(16))) u16 sC[2][kT * N];
    __shared__ __attribute__((aligned(16))) u16 sP[2][3][32 * kPRow];   // masked scores [i][j]
    __shared__ __attribute__((aligned(16))) float sA[2][HWX][kT];       // a [buf][head][step]
    // stage 1's results per head, two buffers: output exponents, state
    // weights per step, and the block's scale decisions
    __shared__ __attribute__((aligned(16))) float sCs[2][HWX][kT];
    __shared__ __attribute__((aligned(16))) float sW[2][HWX][kT];
    __shared__ __attribute__((aligned(16))) float sPar[2][HWX][8];
    __shared__ __attribute__((aligned(16))) float sTouch[64];          // landing area of cache touches

    // ---- work item: contiguous item ranges per XCD (unit sets fastest) ----
    const int HPG = H / G;
    const int UPG = HPG * PS;                      // units per group
    const int UQ = (UPG + SW - 1) / SW;            // workgroups per (batch, segment, group)
    const int64_t items = (int64_t)Bz * nseg_grid * G * UQ;
    const int64_t per_xcd = gridDim.x / kXcds;
    const int64_t item = (int64_t)(blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
    if (item >= items) return;
    const int uq = (int)(item % UQ);
    const int grp = (int)((item / UQ) % G);
    const int64_t seg = (item / UQ / G) % nseg_grid;
    const int b = (int)(item / UQ / G / nseg_grid);
    const int u0 = uq * SW;                        // first unit of the workgroup within the group
    const int ulast = (u0 + SW < UPG ? u0 + SW : UPG) - 1;
    const int hl0 = u0 / PS;                       // first head touched (within the group)
    const int nh = ulast / PS - hl0 + 1;           // heads touched (<= HWX)

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, g2 = lane >> 5;
    const int64_t PN = (int64_t)P * N;
    const int64_t nblk = (L + kT - 1) / kT;
    const int64_t c_begin = seg * blocks_per_seg;
    const int64_t c_end = (c_begin + blocks_per_seg < nblk) ? c_begin + blocks_per_seg : nblk;
    auto block_last = [&](int64_t c) -> int {
        const int64_t last = L - 1 - c * kT;
        return (int)(last < kT - 1 ? last : kT - 1);
    };
    // Time order of the sequence arrays.  REV: step t of the problem is step
    // L - 1 - t of X, B, C and Y, and its decay is a at step L - t (none at
    // t = 0), the time-reversed problem of the backward read in place (L a
    // multiple of the block: block c is the memory block L/kT - 1 - c, rows
    // reversed).  row_base: first memory row of block c; row_loc: memory row
    // of the block's step r relative to it.
    constexpr bool rev = REV;
    auto row_base = [&](int64_t c) -> int64_t { return rev ? L - kT * (c + 1) : c * kT; };
    auto row_loc = [&](unsigned r) -> unsigned { return rev ? (unsigned)(kT - 1) - r : r; };

    // Decay scales (as in the segmented kernel).  The true state is 2^ld *
    // Sacc.  In a block whose log2-decays stay within range of the state
    // scale the decay is never applied to the accumulators: with
    // X~_j = 2^(-ld - cs2_j) X_j,
    //   Y_i   = 2^(cs2_i + ld) * (C_i Sacc + sum_{j<=i} (C_i . B_j) X~_j)
    //   Sacc' = Sacc + B^T X~,   ld' = ld + Lam2.
    // Each 16-step quarter (one MFMA k step) is checked on its own and the
    // scale re-based to the quarter's centre when needed; a block with a
    // quarter too wide for any scale takes the direct form (per-element decay
    // of the shared scores, then Sacc' = 2^(ld + Lam2) Sacc + B^T (w o X)).
    // kRange bounds every weight and output exponent: |log2| <= 96 keeps X~
    // (bf16 shares fp32's exponent range), the scaled state and every fp32
    // accumulation (sums of 64 products of scores below 2^9 with X~ below
    // 2^98) at least 2^10 away from overflow, while re-basing far less often
    // than a tighter range would.
    constexpr int kQ = 4;
    constexpr float kRange = 96.f;
    constexpr float kSpan = 2.f * kRange - 8.f;
    auto fits = [](float l, float absh, float lamh_) {
        return l >= 0.5f * (absh - lamh_) - kRange && l <= kRange - 0.5f * (absh + lamh_);
    };

    if (wave == SW) {
        // ======== X wave: copies of X and a two blocks ahead, stage 1 one block ahead ========
        // (issue priority over the state wave sharing its SIMD: its copies and
        // stage 1 gate the next block)
        __builtin_amdgcn_s_setprio(2);
        // Copy k of unit j fills the 16-byte LDS slots 64k + lane of the unit's
        // tile: row (64k + lane) / 4, stored piece lane % 4, which holds the
        // row's logical piece (lane % 4) ^ swzbits<4>(row).
        auto copy_x = [&](int64_t c, int xs) {
            const unsigned lc = (unsigned)block_last(c);
            const u16* Xg = X + ((int64_t)b * L + row_base(c)) * H * P;
#pragma unroll
            for (int k = 0; k < XOPS; ++k) {
                const int j = k / (kT * XPU / 64);             // unit (uniform)
                const int kk = k % (kT * XPU / 64);            // copy within the unit
                const int uj = u0 + j <= ulast ? u0 + j : ulast;
                const int hj = grp * HPG + uj / PS, pj = (uj % PS) * 32;
                const unsigned r = (unsigned)(kk * 64 + lane) / XPU;
                const unsigned q = ((unsigned)lane % XPU) ^ (unsigned)swzbits<XPU>((int)r);
                const unsigned tr = r <= lc ? r : lc;
                dma16(Xg, ((row_loc(tr) * (unsigned)H + (unsigned)hj) * P + pj + q * 8) * 2u,
                      lds_addr(&sX[xs][j][0]) + (uint32_t)(kk * 64 * 16));
            }
        };
        // a of every head the units touch (lane = step); HWX copies always, so
        // that the wait counts below are constants
        auto copy_a = [&](int64_t c, int as) {
            const unsigned lc = (unsigned)block_last(c);
            const float* ag = a + ((int64_t)b * L + row_base(c)) * H + grp * HPG;
            // rev: the decay of step t is a at memory step L - t, one row past
            // step t's own; for t = 0 (c = 0, lane 0) that is past the end, so
            // the lane reads a row inside and stage 1 takes zero instead
            const unsigned tr0 = (unsigned)lane <= lc ? (unsigned)lane : lc;
            const unsigned tr = !rev ? tr0 : (c == 0 && tr0 == 0) ? (unsigned)(kT - 1) : (unsigned)kT - tr0;
#pragma unroll
            for (int hh = 0; hh < HWX; ++hh) {
                const unsigned hx = (unsigned)(hl0 + (hh < nh ? hh : nh - 1));
                dma4(ag, (tr * (unsigned)H + hx) * 4u, lds_addr(&sA[as][hh][0]));   // (row tr already in memory order)
            }
        };
        // Stage 1, vectorised over heads: one 16-lane row per head, lane li of
        // row r holding steps 4li .. 4li+3 of head slot 4*pass + r, so four
        // heads take one pass.  The rows' prefix sums are DPP row scans; a
        // quarter (16 steps) is a quad of lanes.  The scale reference is
        // carried across quarters by a four-step scan of row shifts: quarter
        // q takes the reference left by quarter q - 1 (the state's scale ld
        // for quarter 0), keeps it if the quarter fits, else re-bases to the
        // quarter's centre -Lam_q / 2 (at quarter 0 that re-bases the carried
        // state before stage 5; later it folds the accumulators between the
        // quarters' products).
        constexpr int NPASS = (HWX + 3) / 4;
        const int rw = lane >> 4, li = lane & 15, qq = li >> 2;   // row, lane in row, quarter
        auto dpp_ctl = [](float v, auto ctrl_const) {
            return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), decltype(ctrl_const)::value,
                                                              0xf, 0xf, true));
        };
        using C_shr1 = std::integral_constant<int, 0x111>;
        using C_shr2 = std::integral_constant<int, 0x112>;
        using C_shr4 = std::integral_constant<int, 0x114>;
        using C_shr8 = std::integral_constant<int, 0x118>;
        using C_q3 = std::integral_constant<int, 0xff>;        // quad_perm [3,3,3,3]
        using C_qx1 = std::integral_constant<int, 0xb1>;       // quad_perm [1,0,3,2]
        using C_qx2 = std::integral_constant<int, 0x4e>;       // quad_perm [2,3,0,1]
        float ldv[NPASS];   // scale of each row's head after the latest block
#pragma unroll
        for (int ps = 0; ps < NPASS; ++ps) ldv[ps] = 0.f;
        auto decide = [&](int64_t cn) {
            const int io = (int)((cn - c_begin) & 1);
            const int lastn = block_last(cn);
#pragma unroll
            for (int ps = 0; ps < NPASS; ++ps) {
                const int hh = 4 * ps + rw < HWX ? 4 * ps + rw : HWX - 1;   // head slot of this row
                const bool row_ok = 4 * ps + rw < HWX;
                const float4 a4 = *reinterpret_cast<const float4*>(&sA[io][hh][4 * li]);
                const bool first = rev && cn == 0 && li == 0;   // reversed step 0 has no decay
                const float av[4] = {4 * li + 0 <= lastn && !first ? a4.x : 0.f, 4 * li + 1 <= lastn ? a4.y : 0.f,
                                     4 * li + 2 <= lastn ? a4.z : 0.f, 4 * li + 3 <= lastn ? a4.w : 0.f};
                // in-lane prefix sums, then the row scan of the lanes' totals
                float pin[4];
                pin[0] = av[0];
#pragma unroll
                for (int e = 1; e < 4; ++e) pin[e] = pin[e - 1] + av[e];
                const float ab = fabsf(av[0]) + fabsf(av[1]) + fabsf(av[2]) + fabsf(av[3]);
                float t = pin[3];
                t += dpp_ctl(t, C_shr1{});
                t += dpp_ctl(t, C_shr2{});
                t += dpp_ctl(t, C_shr4{});
                t += dpp_ctl(t, C_shr8{});
                const float excl = t - pin[3];                 // sum of a before this lane's steps
                // per quarter (quad): cumulative sum at its end, at the end of
                // the quarter before, and the sum of |a| over it (log2 units)
                const float qend = dpp_ctl(t, C_q3{});
                const float qprev = dpp_ctl(qend, C_shr4{});  // zero for quarter 0
                float aq = ab + dpp_ctl(ab, C_qx1{});
                aq += dpp_ctl(aq, C_qx2{});
                const float lamq = (qend - qprev) * kLog2e;
                const float absq = aq * kLog2e;
                const float base = qprev * kLog2e;             // cs2 before this quarter
                // row-wide: total log2-decay (lane 15 of the row) and whether
                // every quarter fits some scale
                auto row_last = [&](float v) {   // v at lane 15 of this lane's row
                    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 15));
                    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 31));
                    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 47));
                    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
                    return rw == 0 ? r0 : rw == 1 ? r1 : rw == 2 ? r2 : r3;
                };
                const float lam2 = row_last(t) * kLog2e;
                const unsigned long long wide = __builtin_amdgcn_ballot_w64(!(absq <= kSpan));
                const bool fast = ((wide >> (16 * rw)) & 0xffffull) == 0;
                // the reference of each quarter, carried across the quarters
                float lin = ldv[ps], ref = 0.f, rqm = 0.f;
#pragma unroll
                for (int q = 0; q < kQ; ++q) {
                    // a re-base moves the reference by a whole number k of
                    // octaves to within half of one of the quarter's centre
                    // (well inside the margin kSpan leaves), so that the
                    // state is moved by an exact ldexp: 2^k itself can fall
                    // below fp32's normal range when the product does not
                    const bool fold = fast & !fits(lin, absq, lamq);
                    const float k = rintf(lin + 0.5f * lamq);
                    const float r = fold ? lin - k : lin;
                    if (qq == q) {
                        ref = r;
                        rqm = fold ? k : 0.f;
                    }
                    const float nxt = dpp_ctl(r + lamq, C_shr4{});   // quarter q's output, one quarter on
                    if (qq == q + 1) lin = nxt;
                }
                // per step: output exponent and state weight
                float cs2[4], ocs[4], wgt[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    cs2[e] = (excl + pin[e]) * kLog2e;
                    ocs[e] = fast ? cs2[e] - base + ref : cs2[e];
                    const float wsh = fast ? base - ref : lam2;
                    wgt[e] = 4 * li + e <= lastn ? fast_exp2(wsh - cs2[e]) : 0.f;
                }
                // the scale after the block (quarter 3's output), for the row
                const float ld_out = fast ? row_last(ref + lamq) : 0.f;
                ldv[ps] = ld_out;
                if (row_ok) {
                    *reinterpret_cast<float4*>(&sCs[io][hh][4 * li]) = make_float4(ocs[0], ocs[1], ocs[2], ocs[3]);
                    *reinterpret_cast<float4*>(&sW[io][hh][4 * li]) = make_float4(wgt[0], wgt[1], wgt[2], wgt[3]);
                    // decisions: (fast, re-base k, ld_in, lam2) from quarter 0, the
                    // folds of quarters 1..3, and the scale after the block
                    if (li == 0)
                        *reinterpret_cast<float4*>(&sPar[io][hh][0]) =
                            make_float4(fast ? 1.f : 0.f, rqm, ref, lam2);
                    if (li == 4 || li == 8 || li == 12) sPar[io][hh][4 + qq - 1] = rqm;
                    if (li == 15) sPar[io][hh][7] = ld_out;
                }
            }
        };
        // Per block c: wait for X and a of block c + 1 (issued a block ago),
        // stage 1 of block c + 1, then the copies of block c + 2 -- after the
        // score wave's burst of B and C copies at the top of the block.
        if (c_begin < c_end) {
            copy_x(c_begin, 0);
            copy_a(c_begin, 0);
            if (c_begin + 1 < c_end) {
                copy_x(c_begin + 1, 1);
                copy_a(c_begin + 1, 1);
                vm_wait_le<XOPS + HWX>();   // block c_begin's copies have landed
            } else {
                vm_wait_all();
            }
            decide(c_begin);
        }
        for (int64_t c = c_begin; c < c_end; ++c) {
            sync_lds();   // top of block c
            if (c + 1 < c_end) {
                vm_wait_all();   // X and a of block c + 1 have landed
                decide(c + 1);
                if (c + 2 < c_end) {
                    copy_x(c + 2, (int)((c + 2 - c_begin) % NXB));
                    copy_a(c + 2, (int)((c + 2 - c_begin) & 1));
                }
            }
        }
        return;
    }

    if (wave == SW + 1) {
        __builtin_amdgcn_s_setprio(2);
        // ======== score wave: B and C of the next block, and its scores ========
        // Copy k of sub-tile nt fills the 16-byte slots 64k + lane: row
        // 16k + lane/4, stored piece lane % 4, which holds logical piece
        // (lane % 4) ^ swzbits<4>(row) = (lane % 4) ^ ((lane / 16) % 4).
        const unsigned qb = ((unsigned)lane & 3u) ^ (((unsigned)lane >> 4) & 3u);
        auto copy_bc = [&](int64_t c, int bs) {
            const unsigned lc = (unsigned)block_last(c);
            const int64_t row0 = (((int64_t)b * L + row_base(c)) * G + grp) * N;
#pragma unroll
            for (int k = 0; k < kT * XPU / 64; ++k) {
                const unsigned r = 16u * (unsigned)k + (unsigned)lane / 4u;
                const unsigned tr = r <= lc ? r : lc;
#pragma unroll
                for (int nt = 0; nt < NTL; ++nt) {
                    const uint32_t go = (row_loc(tr) * (unsigned)(G * N) + (unsigned)(nt * 32) + qb * 8u) * 2u;
                    dma16(B + row0, go, lds_addr(&sB[bs][nt * SUB]) + (uint32_t)(k * 64 * 16));
                    dma16(C + row0, go, lds_addr(&sC[bs][nt * SUB]) + (uint32_t)(k * 64 * 16));
                }
            }
        };
        // B and C of block c two blocks ahead into L2: one 4-byte copy per
        // 128-byte line, landing in a scratch LDS area nobody reads, so that
        // the real copies a block later hit L2 instead of waiting on HBM
        // (the workgroups of a batch all ask for the same rows at once)
        constexpr int kTouch = 2 * kT * N * 2 / 128 / 64;   // touch copies per block
        auto touch_bc = [&](int64_t c) {
            const unsigned lc = (unsigned)block_last(c);
            const int64_t row0 = (((int64_t)b * L + row_base(c)) * G + grp) * N;
#pragma unroll
            for (int k = 0; k < kTouch; ++k) {
                const unsigned li = (unsigned)(k * 64 + lane);     // line index over B then C
                const unsigned half = li / (unsigned)(kT * N * 2 / 128);
                const unsigned ln = li % (unsigned)(kT * N * 2 / 128);
                const unsigned r = ln / (unsigned)(N * 2 / 128), piece = ln % (unsigned)(N * 2 / 128);
                const unsigned tr = r <= lc ? r : lc;
                dma4(half ? C + row0 : B + row0, (row_loc(tr) * (unsigned)(G * N) + piece * 64u) * 2u,
                     lds_addr(&sTouch[0]));
            }
        };
        // row operand of rows 32R + l32, the k values 16hf + 8g2 + 0..7 of
        // sub-tile nt (the v_mfma_f32_32x32x16_bf16 operand layout)
        const uint32_t ro[2] = {(uint32_t)swz<XPU>(l32, 8 * g2), (uint32_t)swz<XPU>(l32, 16 + 8 * g2)};
        // the three causal score tiles t = (I, J) in {(0,0), (1,0), (1,1)} as
        // S^T = B_J C_I^T (lane = i), stored [i][j] in bf16; masked entries
        // (j > i on the diagonal) are replaced by zero, never multiplied.
        // Every operand is read first; the three tiles' chains then interleave.
        auto scores = [&](int bs) {
            const u16* bT = &sB[bs][0];
            const u16* cT = &sC[bs][0];
            u32x4 fb[2][NTL][2], fc[2][NTL][2];
#pragma unroll
            for (int R = 0; R < 2; ++R)
#pragma unroll
                for (int nt = 0; nt < NTL; ++nt)
#pragma unroll
                    for (int hf = 0; hf < 2; ++hf) {
                        fb[R][nt][hf] = *reinterpret_cast<const u32x4*>(bT + nt * SUB + 32 * R * 32 + ro[hf]);
                        fc[R][nt][hf] = *reinterpret_cast<const u32x4*>(cT + nt * SUB + 32 * R * 32 + ro[hf]);
                    }
            f32x16 St[3] = {zero16(), zero16(), zero16()};
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                    for (int t = 0; t < 3; ++t) {
                        const int I = t > 0 ? 1 : 0, J = t == 2 ? 1 : 0;
                        St[t] = mfma32(as_bf16x8(fb[J][nt][hf]), as_bf16x8(fc[I][nt][hf]), St[t]);
                    }
#pragma unroll
            for (int t = 0; t < 3; ++t) {
                const bool diag = t != 1;
                u16* prow = &sP[bs][t][l32 * kPRow];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int j0 = 8 * q + 4 * g2;
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = (!diag || j0 + e <= l32) ? St[t][4 * q + e] : 0.f;
                    *reinterpret_cast<uint2*>(prow + j0) = make_uint2(pack2(v[0], v[1]), pack2(v[2], v[3]));
                }
            }
        };
        // issue order per block: B and C of block c + 1, then the touches of
        // block c + 2; "at most kTouch outstanding" is then the copies landed
        if (c_begin < c_end) {
            copy_bc(c_begin, 0);
            if (c_begin + 1 < c_end) touch_bc(c_begin + 1);
            vm_wait_all();
            scores(0);
        }
        for (int64_t c = c_begin; c < c_end; ++c) {
            sync_lds();   // top of block c: buffers (c + 1) & 1 are free
            if (c + 1 < c_end) {
                const int nb = (int)((c + 1 - c_begin) & 1);
                copy_bc(c + 1, nb);
                if (c + 2 < c_end) {
                    touch_bc(c + 2);
                    vm_wait_le<kTouch>();
                } else {
                    vm_wait_all();
                }
                scores(nb);
            }
        }
        vm_wait_all();   // no copy may land in LDS after the workgroup ends
        return;
    }

    // ======================= state waves =======================
    const int sw = wave;
    const int uw = u0 + sw;                        // this wave's unit
    const bool uvalid = uw <= ulast;
    const int uc = uvalid ? uw : ulast;
    const int hlw = uc / PS;                       // head within the group
    const int hw = hlw - hl0;                      // head slot in the stage-1 buffers
    const int h = grp * HPG + hlw;
    const int pc = (uc % PS) * 32;                 // first head-dim column

    // carried state: S^T tiles (rows n, columns p of this unit); register r of
    // tile nt holds n = 32nt + 16(r/8) + 8g2 + r%8 of column p = pc + l32
    f32x16 Sacc[NTL];
#pragma unroll
    for (int nt = 0; nt < NTL; ++nt) Sacc[nt] = zero16();
    {
        const float* S0 = seg == 0 ? (src.first ? src.first + b * src.first_bstride : nullptr)
                                   : (src.Sin ? src.Sin + b * src.bstride + seg * src.sstride : nullptr);
        if (S0) {
            S0 += (int64_t)h * PN;
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt) {
                const float* row = S0 + (int64_t)(pc + l32) * N + nt * 32 + 8 * g2;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float4 v = *reinterpret_cast<const float4*>(row + 16 * (q >> 1) + 4 * (q & 1));
                    Sacc[nt][4 * q + 0] = v.x;
                    Sacc[nt][4 * q + 1] = v.y;
                    Sacc[nt][4 * q + 2] = v.z;
                    Sacc[nt][4 * q + 3] = v.w;
                }
            }
        }
    }
    // Lane-dependent offsets (loop invariant).  B's transposing reads take
    // the column quads of each 16 in the order 0, 2, 1, 3, so that stage 3
    // leaves the 8 state rows a lane holds in registers 8hf .. 8hf+7 of tile
    // nt as the consecutive n = 32nt + 16hf + 8g2 + 0..7: the stage-5 operand
    // order of a plain 16-byte row read of C.  Element offsets into the
    // swizzled 32-column tiles (the swizzle of a row depends only on the row
    // modulo 16, so row blocks of 16 and sub-tiles are added per use as
    // immediates):
    //  roff: row reads of C (row l32, the 16 bytes at column 16hf + 8g2);
    //  toff: transposing reads of B (source row 8g2 + 4s + trow, column tcolb);
    //  xoff: those of this unit's X tile (column tcol).
    const int trow = (lane & 15) >> 2, tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    const int tcolb = 16 * ((lane >> 4) & 1) + 4 * ((lane & 3) == 1 ? 2 : (lane & 3) == 2 ? 1 : (lane & 3));
    uint32_t roff[2], toff[2], xoff[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) roff[hf] = (uint32_t)swz<XPU>(l32, 16 * hf + 8 * g2);
#pragma unroll
    for (int sh = 0; sh < 2; ++sh) {
        const int r = 8 * g2 + 4 * sh + trow;
        toff[sh] = (uint32_t)swz<XPU>(r, tcolb);
        xoff[sh] = (uint32_t)swz<XPU>(r, tcol);
    }

    float ld = 0.f;   // the scale of Sacc (log2) after the latest block
    // The state lives in one fixed register range across the loop: without
    // the pin the compiler kept the loop-carried state in one range and the
    // fast form's products in another, copying 64 registers out and back in
    // every block.
    auto pin_state = [&]() {
        if constexpr (NTL == 4)
            asm volatile("" : "+{v[2:17]}"(Sacc[0]), "+{v[18:33]}"(Sacc[1]), "+{v[34:49]}"(Sacc[2]),
                              "+{v[50:65]}"(Sacc[3]));
        else
            asm volatile("" : "+{v[2:17]}"(Sacc[0]), "+{v[18:33]}"(Sacc[1]));
    };
    for (int64_t c = c_begin; c < c_end; ++c) {
        pin_state();
        const int bs = (int)((c - c_begin) & 1);          // B, C, scores, stage-1 buffers
        const int xs = (int)((c - c_begin) % NXB);        // X buffer
        const int last = block_last(c);
        sync_lds();   // top of block c: its X, B, C, scores and stage-1 results are visible

        const u16* bT = &sB[bs][0];
        const u16* cT = &sC[bs][0];
        const u16* xT = &sX[xs][sw][0];
        u16* xTm = &sX[xs][sw][0];
        // ---- the block's stage-1 results for this unit's head ----
        const float4 pa = *reinterpret_cast<const float4*>(&sPar[bs][hw][0]);
        const float4 pb = *reinterpret_cast<const float4*>(&sPar[bs][hw][4]);
        auto uni = [](float v) { return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v))); };
        const bool fast = uni(pa.x) != 0.f;
        const float ld_in = uni(pa.z), lam2 = uni(pa.w);
        // whole-octave re-bases: quarter 0's (before stage 5), then quarters 1..3
        const int rq[kQ] = {(int)uni(pa.y), (int)uni(pb.x), (int)uni(pb.y), (int)uni(pb.z)};
        const bool fold[kQ] = {rq[0] != 0, rq[1] != 0, rq[2] != 0, rq[3] != 0};
        ld = uni(pb.w);

        auto load_c = [&](int nt, u32x4 (&dst)[2][2]) {
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int I = 0; I < 2; ++I)
                    dst[hf][I] = *reinterpret_cast<const u32x4*>(cT + nt * SUB + 32 * I * 32 + roff[hf]);
        };
        // B^T fragments of quarter q = (J, ks), one per state tile (the two
        // transposing reads land directly in the halves of the operand)
        auto load_bt = [&](int q, bf16x8 (&dst)[NTL]) {
            const u16* t = bT + (32 * (q >> 1) + 16 * (q & 1)) * 32;
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt)
                dst[nt] = join8(lds_tr4(t + nt * SUB + toff[0]), lds_tr4(t + nt * SUB + toff[1]));
        };
        // X^T fragment i = (J, ks) of this unit (lane = p, k = step) and its steps' weights
        auto load_x = [&](int i, i16x4 (&dst)[2]) {
            const u16* t = xT + (32 * (i >> 1) + 16 * (i & 1)) * 32;
            dst[0] = lds_tr4(t + xoff[0]);
            dst[1] = lds_tr4(t + xoff[1]);
        };
        auto load_w = [&](int i, float4 (&dst)[2]) {
            const float* wp = &sW[bs][hw][32 * (i >> 1) + 16 * (i & 1) + 8 * g2];
            dst[0] = *reinterpret_cast<const float4*>(wp);
            dst[1] = *reinterpret_cast<const float4*>(wp + 4);
        };
        // X~ = w o X in registers, rounded once to bf16
        auto weigh = [](const i16x4 (&x)[2], const float4 (&w)[2]) {
            const float w8[8] = {w[0].x, w[0].y, w[0].z, w[0].w, w[1].x, w[1].y, w[1].z, w[1].w};
            return scale8(join8(x[0], x[1]), w8);
        };
        // score tile i as stage 2's B operand: (tile, ks) = (0,0) (1,0) (0,1) (1,1) (2,0) (2,1)
        auto load_p = [&](int i) {
            return *reinterpret_cast<const u32x4*>(
                &sP[bs][i < 4 ? (i & 1) : 2][l32 * kPRow + 16 * (i < 4 ? (i >> 1) : (i & 1)) + 8 * g2]);
        };
        auto fence = []() { __builtin_amdgcn_sched_barrier(0); };

        f32x16 Yt[2] = {zero16(), zero16()};
        uint2 Yb[2][4];
        auto pack_y = [&]() {
#pragma unroll
            for (int I = 0; I < 2; ++I)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    Yb[I][q] = make_uint2(pack2(Yt[I][4 * q], Yt[I][4 * q + 1]),
                                          pack2(Yt[I][4 * q + 2], Yt[I][4 * q + 3]));
        };
        // ---- Y^T through this unit's own X tile (dead after stage 3), so that
        // copy k of a lane holds 16 contiguous bytes of step 16k + lane/4 and a
        // store covers 16 steps x 64 bytes.  Called at the end of each form,
        // so that nothing after the branch needs registers while the state is
        // live (a shared tail made the compiler move the state out and back) ----
        auto store_y = [&]() {
#pragma unroll
            for (int I = 0; I < 2; ++I)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    *reinterpret_cast<uint2*>(xTm + swz<XPU>(32 * I + l32, 8 * q + 4 * g2)) = Yb[I][q];
            u32x4 Yr[4];
#pragma unroll
            for (int k = 0; k < 4; ++k)
                Yr[k] = *reinterpret_cast<const u32x4*>(xTm + swz<XPU>(16 * k + (lane >> 2), 8 * (lane & 3)));
            if (uvalid) {
                u16* yblk = Y + ((int64_t)b * L + row_base(c)) * H * P;
                const int yoff = (int)((row_loc((unsigned)(lane >> 2)) * H + h) * P + pc + 8 * (lane & 3));
                const int ystep = rev ? -16 * H * P : 16 * H * P;   // step 16k + lane/4 of the block
                if (last == kT - 1) {
                    // a whole block: no per-lane conditions, so that the four
                    // reads above stay ahead of the stores (under per-store
                    // conditions the compiler moved them into the branches,
                    // one read, wait and store after another).  The backward's
                    // dX (REV) is not read again: non-temporal stores
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        if constexpr (REV)
                            __builtin_nontemporal_store(Yr[k], reinterpret_cast<u32x4*>(yblk + (yoff + k * ystep)));
                        else
                            *reinterpret_cast<u32x4*>(yblk + (yoff + k * ystep)) = Yr[k];
                    }
                } else {
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        if (16 * k + (lane >> 2) <= last)
                            *reinterpret_cast<u32x4*>(yblk + (yoff + k * ystep)) = Yr[k];
                }
            }
        };
        // ================= one instruction stream for both forms =================
        // Operand reads are issued a group ahead of the MFMAs that consume
        // them, with scheduling fences so that the compiler keeps them there:
        // one state tile of C ahead in stage 5, stage 2's operands during
        // stage 5's last tiles, one quarter of B^T ahead in stage 3.  A block
        // in the direct form (a quarter's log2-decay spread too wide for any
        // power-of-two scale) runs the same products on other operands and
        // scales: stage 5's output and the state are scaled after stage 5
        // (Sacc' = 2^(ld + Lam2) Sacc + B^T (w o X)), and stage 2 multiplies
        // the unweighted X by the per-element decayed scores.  Keeping one
        // stream (the form only picks operands and in-place scalings) keeps
        // the state in one register range; two separate forms made the
        // compiler move all 64 state registers out and back every block.
        u32x4 cf[2][2][2];          // C fragments, two state tiles
        load_c(0, cf[0]);
        if (fold[0]) {              // the block's re-based scale, before stage 5 (fast form)
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt) scale_pow2(Sacc[nt], rq[0]);
        }
        i16x4 xr[4][2];             // X^T fragments (J, ks) = (0,0), (0,1), (1,0), (1,1)
        float4 wv[4][2];            // their steps' state weights
        u32x4 pt[6];                // score tiles as stage 2's B operands
        float csr[2];               // output exponents of rows l32 and 32 + l32
        bf16x8 xk[4];               // X~ fragments
        // ---- stage 5: Y^T = Sacc C^T ----
#pragma unroll
        for (int nt = 0; nt < NTL; ++nt) {
            if (nt + 1 < NTL) load_c(nt + 1, cf[(nt + 1) & 1]);
            if (nt == NTL - 2 || NTL == 1) {
#pragma unroll
                for (int i = 0; i < 4; ++i) load_x(i, xr[i]);
                load_w(0, wv[0]);
                load_w(1, wv[1]);
            }
            if (nt == NTL - 1) {
                load_w(2, wv[2]);
                load_w(3, wv[3]);
                pt[0] = load_p(0);
                pt[1] = load_p(1);
                csr[0] = sCs[bs][hw][l32];
                csr[1] = sCs[bs][hw][32 + l32];
            }
            fence();
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const bf16x8 Sf = acc_half(Sacc[nt], hf);
#pragma unroll
                for (int I = 0; I < 2; ++I) Yt[I] = mfma32(Sf, as_bf16x8(cf[nt & 1][hf][I]), Yt[I]);
            }
            if (nt == NTL - 1) {
                xk[0] = weigh(xr[0], wv[0]);
                xk[1] = weigh(xr[1], wv[1]);
            }
            fence();
        }
#pragma unroll
        for (int i = 2; i < 6; ++i) pt[i] = load_p(i);
        xk[2] = weigh(xr[2], wv[2]);
        xk[3] = weigh(xr[3], wv[3]);
        bf16x8 bt[2][NTL];          // B^T fragments, two quarters
        load_bt(0, bt[0]);
        if (!fast) {
            // direct form: stage 5's output at the block's entering scale,
            // the state moved to the block's end, and the scores decayed per
            // element by 2^(cs2_i - cs2_j) (masked entries stay zero: their
            // exponent may overflow).  Score tile i is (t, ks) = (0,0) (1,0)
            // (0,1) (1,1) (2,0) (2,1); tile t covers rows 32 (t > 0) .. and
            // columns 32 (t == 2) ..
            Yt[0] *= fast_exp2(csr[0] + ld_in);
            Yt[1] *= fast_exp2(csr[1] + ld_in);
            const float f = fast_exp2(ld_in + lam2);
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt) Sacc[nt] *= f;
#pragma unroll
            for (int i = 0; i < 6; ++i) {
                const int t = i < 4 ? (i & 1) : 2, ks = i < 4 ? (i >> 1) : (i & 1);
                const float csi = t == 0 ? csr[0] : csr[1];
                const int jl = 32 * (t == 2) + 16 * ks + 8 * g2;
                const f32x4 c0 = *reinterpret_cast<const f32x4*>(&sCs[bs][hw][jl]);
                const f32x4 c1 = *reinterpret_cast<const f32x4*>(&sCs[bs][hw][jl + 4]);
                const float cj[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
                const bool diag = t != 1;
                float v[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int j = 16 * ks + 8 * g2 + e;
                    const float x = __uint_as_float(e & 1 ? (pt[i][e >> 1] & 0xffff0000u) : (pt[i][e >> 1] << 16));
                    v[e] = (!diag || j <= l32) ? x * fast_exp2(csi - cj[e]) : 0.f;
                }
                pt[i] = u32x4{pack2(v[0], v[1]), pack2(v[2], v[3]), pack2(v[4], v[5]), pack2(v[6], v[7])};
            }
        }
        // ---- stages 2, 3 and 4, quarter by quarter, interleaved (the two
        // stages are independent: stage 3 updates the state, stage 2 the
        // output).  Stage 3: Sacc' = Sacc + B^T X~, with the state moved to
        // a re-based quarter's reference before its products.  Stage 2:
        // Y^T += X~^T P (direct form: X^T P~); at a re-based quarter the rows
        // from that quarter on move to its reference after the products
        // before it. ----
        const bool upper = l32 >= 16;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (q + 1 < 4) load_bt(q + 1, bt[(q + 1) & 1]);
            fence();
            if (q > 0 && fold[q]) {
#pragma unroll
                for (int nt = 0; nt < NTL; ++nt) scale_pow2(Sacc[nt], rq[q]);
            }
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt)
                Sacc[nt] = mfma32(bt[q & 1][nt], xk[q], Sacc[nt]);
            bf16x8 xa = xk[q];      // stage 2's X operand (direct form: X itself, read again)
            if (!fast) {
                i16x4 xu[2];
                load_x(q, xu);
                xa = join8(xu[0], xu[1]);
            }
            if (q < 2) {
                Yt[0] = mfma32(xa, as_bf16x8(pt[2 * q]), Yt[0]);
                Yt[1] = mfma32(xa, as_bf16x8(pt[2 * q + 1]), Yt[1]);
            } else {
                Yt[1] = mfma32(xa, as_bf16x8(pt[2 + q]), Yt[1]);
            }
            if (q == 0 && fold[1]) {
                scale_pow2(Yt[0], upper ? rq[1] : 0);
                scale_pow2(Yt[1], rq[1]);
            }
            if (q == 1 && fold[2]) scale_pow2(Yt[1], rq[2]);
            if (q == 2 && fold[3]) scale_pow2(Yt[1], upper ? rq[3] : 0);
            fence();
        }
        if (fast) {
            Yt[0] *= fast_exp2(csr[0]);
            Yt[1] *= fast_exp2(csr[1]);
        }
        pack_y();
        store_y();
        pin_state();
    }

    // ---- epilogue: final state (last segment) ----
    if (!uvalid || !S_fin || seg != nseg_grid - 1) return;
    float* Sdst = S_fin + ((int64_t)b * H + h) * PN;
    const float f = fast_exp2(ld);
    const float e = fin_a ? expf(fin_a[b * fin_a_bstride + h]) : 1.f;   // the state, then this factor
#pragma unroll
    for (int nt = 0; nt < NTL; ++nt) {
        float* row = Sdst + (int64_t)(pc + l32) * N + nt * 32 + 8 * g2;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            *reinterpret_cast<float4*>(row + 16 * (q >> 1) + 4 * (q & 1)) =
                make_float4(e * (f * Sacc[nt][4 * q]), e * (f * Sacc[nt][4 * q + 1]),
                            e * (f * Sacc[nt][4 * q + 2]), e * (f * Sacc[nt][4 * q + 3]));
    }
}

// one workgroup per (batch, segment, group, unit set), padded to a multiple of the XCD count
static int64_t fwd_items(const FwdShape& s, int64_t nseg, int sw) {
    const int64_t upg = (s.H / s.G) * (s.P / 32);
    return s.Bz * nseg * s.G * ((upg + sw - 1) / sw);
}

int64_t fwd_workgroups(const FwdShape& s, int64_t nseg, int sw) {
    return ((fwd_items(s, nseg, sw) + kXcds - 1) / kXcds) * kXcds;
}

hipError_t launch_fwd(const FwdShape& s, int sw, int64_t seg_chunks, int64_t nseg, const void* X,
                      const float* a, const void* B, const void* C, StateSrc src, void* Y,
                      float* S_fin, hipStream_t st, bool rev, const float* fin_a, int64_t fin_a_bstride)
{
    if (rev && s.L % kT != 0) return hipErrorInvalidValue;
    const dim3 grid((unsigned)fwd_workgroups(s, nseg, sw));
    const int64_t bps = seg_chunks * (s.Q / kT);
#define SSD_LAUNCH_FWD(PP, NN, SWW, RR)                                                         \
    hipLaunchKernelGGL((k_fwd<PP, NN, SWW, RR>), grid, dim3(64 * (SWW + 2)), 0, st, (const u16*)X, \
                       a, (const u16*)B, (const u16*)C, src, (u16*)Y, S_fin, fin_a, fin_a_bstride, \
                       s.L, (int)s.H,                                                          \
                       (int)s.G, bps, (int)nseg, (int)s.Bz)
#define SSD_FWD_SW(PP, NN)                                 \
    if (sw == 4) SSD_LAUNCH_FWD(PP, NN, 4, false);         \
    else if (sw == 5) SSD_LAUNCH_FWD(PP, NN, 5, false);    \
    else if (sw == 6 && PP == 64) SSD_LAUNCH_FWD(64, NN, 6, false); \
    else return hipErrorInvalidValue;
#define SSD_FWD_SW_REV(NN)                                 \
    if (sw == 4) SSD_LAUNCH_FWD(64, NN, 4, true);          \
    else if (sw == 5) SSD_LAUNCH_FWD(64, NN, 5, true);     \
    else if (sw == 6) SSD_LAUNCH_FWD(64, NN, 6, true);     \
    else return hipErrorInvalidValue;
    if (!fwd_units_supported(s.P, sw)) return hipErrorInvalidValue;
    // the time-reversed instantiations exist for headdim 64 (the backward's dX pass)
    if (rev) {
        if (s.P == 64 && s.N == 128) { SSD_FWD_SW_REV(128) }
        else if (s.P == 64 && s.N == 64) { SSD_FWD_SW_REV(64) }
        else return hipErrorInvalidValue;
        return hipGetLastError();
    }
    if (s.P == 64 && s.N == 128) { SSD_FWD_SW(64, 128) }
    else if (s.P == 64 && s.N == 64) { SSD_FWD_SW(64, 64) }
    else if (s.P == 32 && s.N == 128) { SSD_FWD_SW(32, 128) }
    else if (s.P == 32 && s.N == 64) { SSD_FWD_SW(32, 64) }
    else return hipErrorInvalidValue;
#undef SSD_FWD_SW_REV
#undef SSD_FWD_SW
#undef SSD_LAUNCH_FWD
    return hipGetLastError();
}

}  // namespace ssd
