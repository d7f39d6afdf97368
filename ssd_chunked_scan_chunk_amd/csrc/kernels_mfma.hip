// kernels_mfma.hip -- bf16 MFMA kernels of the SSD layer for gfx950: the
// state-only pass of the segmented forward plan (stages 1, 3, 4) and the
// backward's exchanged-dimension products (the output pass, in the direct
// form).  The forward's full pass is the fused kernel of kernels_fwd.hip; the
// design below is shared by both files.
//
// The layer's sequence map is the 1-semiseparable matrix M = Lmask o (C B^T)
// applied to X (wiki review of "Transformers are SSMs", section "Core
// concepts"; CiteArk page, section "AI research summary": a block-decomposed
// matrix-multiplication algorithm over that matrix).  Blocking the sequence
// into blocks of T steps gives, per block c:
//   1. in-block prefix sums cs of a (wavefront scan, fp32);
//   2. diagonal block:   Ydiag = (Lmask_cc o C_c B_c^T) X_c               (MFMA)
//   3. block state:      dS_c  = X_c^T diag(w) B_c, w_j = exp(Lam_c - cs_j) (MFMA)
//   4. state passing:    S_{c+1} = exp(Lam_c) S_c + dS_c   (fp32, in registers,
//                        the decay kept as a separate power-of-two scale)
//   5. state to output:  Yoff = diag(exp(cs)) C_c S_c^T                    (MFMA)
// Y and the final state do not depend on the block length (every blocking is
// the same sum, only rounded differently), so the fused kernels block at
// T = 64 whatever chunk length the caller names: on gfx950 the causal
// quadratic work of longer blocks costs more MFMA and VALU work than the
// extra state passes it saves.  A caller's chunk still sets segment
// boundaries (segments are whole chunks).
//
// Decomposition on gfx950.
//  * A workgroup is eight wavefronts, two per SIMD, over the heads of one
//    group that share B and C.  Six are state waves: each owns one 32-wide
//    head-dim tile of one head (P/32 waves per head, 192/P heads per
//    workgroup) and carries that slice of the head's fp32 state in MFMA
//    accumulators, so states never round-trip HBM inside a segment.  The
//    other two are copy waves: they issue every copy into LDS, form the
//    shared score tiles and run stage 1 (the scans of a, the scale decisions
//    and the per-step weights) one block ahead.  A wave whose memory
//    instruction finds the CU's queue full stalls until it drains; keeping
//    the copies on waves with no state work lets those stalls overlap the
//    state waves' MFMA and VALU work instead of delaying them.  Copy and
//    state waves run separate loops with the same two barriers per block, so
//    neither keeps the other's values in registers.  When a launch would
//    leave CUs idle the
//    sequence is split into segments: a state-only pass (stages 1, 3, 4)
//    gives each segment's end state from zero, a scan over segments
//    (kernels_scan.hip) gives every segment's entering state, and the full
//    pass (kernels_fwd.hip) starts from it.
//  * The masked scores of a block do not depend on the head (the decay is
//    moved onto X and the output, below), so the copy waves form the three
//    causal 32x32 score tiles once per workgroup and share them in LDS as
//    bf16.
//  * Inputs reach LDS through asynchronous global_load_lds copies (lane L of a
//    wave-wide copy lands at LDS base + L * size), double buffered one block
//    ahead (a: triple buffered two blocks ahead, for stage 1), so HBM traffic
//    overlaps the MFMA work and no register holds
//    prefetched data.  The copies are written in inline assembly: they have no
//    register result, and keeping them out of the compiler's view stops it
//    from inserting full vmcnt waits before every LDS access, which would
//    serialise the prefetch.  Only the copy waves wait for copies (vmcnt(0)
//    once per block); state waves store their outputs at the end of each
//    block and never wait on memory.  Two barriers per block: one publishes the
//    block's copies and stage-1 results (and frees the other buffers), one
//    publishes the shared scores.
//  * Every product is v_mfma_f32_32x32x16_bf16 (operand lane l holds row or
//    column l%32 and 8 k values of group l/32; the accumulator holds column
//    l%32, rows 8(r/4) + 4(l/32) + r%4 in register r).  Contractions take k
//    in natural order (group g holds k = 8g..8g+7 of each 16-wide step).
//    The fp32 state becomes the stage-5 operand in place (rounded to bf16):
//    the accumulator rows a lane holds in registers 8h..8h+7 are the k values
//    8g..8g+7 of step h, and stage 3 writes the state rows in an order that
//    makes those the consecutive n = 16h + 8g + 0..7, so the C operand is a
//    plain 16-byte row read.  16-byte row reads keep every LDS read of a row
//    tile conflict-free; 8-byte reads of 32 rows cannot be (two rows share
//    each 16-byte bank slot).  Operands with the contraction along memory
//    rows (X^T, B^T) come from ds_read_b64_tr_b16: in each 16-lane group,
//    source lane m names row R(m/4) and a 4-column quad Q(m%4), and output
//    lanes 4j..4j+3 receive the columns of quad Q(j) of rows R(0..3).
//  * Scores are formed transposed, S^T = B C^T, so lane = step i; outputs are
//    Y^T tiles, a lane holding 4 consecutive head-dim entries of one step.
//  * LDS tiles are row-major with their 16-byte pieces permuted per row
//    (swzbits below) so that row reads and transposing reads spread over the
//    banks.
//  * Workgroups are dealt to the 8 XCDs in contiguous ranges of (batch,
//    segment, group, head-set) items, so the workgroups sharing B and C run
//    on one XCD and read them through one L2.
// Operand rounding: masked scores, X weighted by the state weights, and the
// entering state are rounded to bf16 for the MFMA; every accumulation and the
// per-step output factor are fp32.
#include <type_traits>

#include "cb_tiles.hpp"
#include "mfma_util.hpp"
#include "ssd_launch.hpp"

namespace ssd {

constexpr int kWaves = 8;    // wavefronts per workgroup (two per SIMD)
constexpr int kStateWaves = kMfmaStateWaves;     // waves that carry head states
constexpr int kAuxThreads = 64 * (kWaves - kStateWaves);   // copy and score waves
constexpr int kThreads = 64 * kWaves;

template <int P, int N, int SW = kStateWaves>
struct MfmaCfg {
    static constexpr int PS = P / 32;                    // state waves per head (one head-dim tile each)
    static constexpr int HW = SW / PS;                   // heads per workgroup
    static constexpr int NTL = N / 32;                   // 32-wide state-dim tiles
    static constexpr int XPR = P / 8;                    // 16-byte pieces per X row
    static constexpr int BPR = N / 8;                    // 16-byte pieces per B / C row
    static constexpr int XOPS = HW * kT * XPR / kAuxThreads;   // X copies per aux thread per block
    static constexpr int BOPS = kT * BPR / kAuxThreads;        // B (or C) copies per aux thread
    static_assert(P % 32 == 0 && N % 32 == 0 && SW % PS == 0, "tile shape");
    static_assert((HW * kT * XPR) % kAuxThreads == 0 && (kT * BPR) % kAuxThreads == 0, "copy shape");
    static_assert(kAuxThreads % XPR == 0 && kAuxThreads % BPR == 0 && (kT * XPR) % kAuxThreads == 0,
                  "a copy covers whole rows of one head");
};


// XG (the backward's exchanged-dimension products): X is a B or C array of
// x_groups groups whose rows hold the HPG heads of a group side by side (head
// hl of group grp reads columns hl*P .. of group grp / (G / x_groups)); every
// head of a group reads the a of head grp of an [L][G] array; and the entering
// states are read transposed, head hl of group grp taking columns hl*P .. of
// the [N][HPG*P] state of head grp; Y is written in fp32.  These outputs are
// summed over the original group's heads afterwards, and those sums can
// cancel (at a single step, dB and dC are a sum over heads of x.dy times one
// row), so the output path keeps about 16 bits: every block takes the direct
// form, the copy waves store the decayed masked scores (the same for all the
// workgroup's heads, which share one decay) as bf16 high and low parts, and
// stage 5 multiplies the state's high and low parts.  SW is the number of
// state waves (the workgroup has SW + 2 wavefronts).
// The body of one workgroup; wg is its index among the nwg workgroups of
// its launch (or of its half of a paired launch).
template <int P, int N, bool FULL, bool XG, int SW>
__device__ __forceinline__ void mfma_seg_body(
    const u16* __restrict__ X, const float* __restrict__ a, const u16* __restrict__ B,
    const u16* __restrict__ C, StateSrc src, u16* __restrict__ Y, float* __restrict__ S_fin,
    float* __restrict__ Sseg, float* __restrict__ lamseg, int64_t nseg_total, int64_t L,
    int H, int G, int64_t blocks_per_seg, int nseg_grid, int Bz, int x_groups, unsigned wg,
    unsigned nwg, int rev)
{
    static_assert(!FULL || XG, "the output pass runs only as the backward's exchanged-dimension products");
    using Cfg = MfmaCfg<P, N, SW>;
    constexpr int HW = Cfg::HW, NTL = Cfg::NTL, XPR = Cfg::XPR, BPR = Cfg::BPR;
    constexpr int XOPS = Cfg::XOPS, BOPS = Cfg::BOPS;

    __shared__ __attribute__((aligned(16))) u16 sX[2][HW * kT * P];    // [buf][head][step][p]
    __shared__ __attribute__((aligned(16))) u16 sB[2][kT * N];         // [buf][step][n]
    __shared__ __attribute__((aligned(16))) u16 sC[FULL ? 2 : 1][FULL ? kT * N : 8];
    // output pass: the decayed masked scores [i][j], high part then low part,
    // unpadded rows with the 16-byte pieces XOR-swizzled by (i / 4) % 4
    __shared__ __attribute__((aligned(16))) u16 sP[FULL ? 3 : 1][FULL ? 2 * 32 * 32 : 8];
    __shared__ __attribute__((aligned(16))) float sA[3][HW * kT];     // [buf][head][step]
    // stage 1's results per head, two buffers: output exponents, state weights
    // per step, and the block's scale decisions
    __shared__ __attribute__((aligned(16))) float sCs[2][HW][kT];
    __shared__ __attribute__((aligned(16))) float sW[2][HW][kT];
    __shared__ __attribute__((aligned(16))) float sPar[2][HW][8];

    // ---- work item: contiguous item ranges per XCD (head sets fastest) ----
    const int HPG = H / G;
    const int HQ = (HPG + HW - 1) / HW;
    const int64_t items = (int64_t)Bz * nseg_grid * G * HQ;
    const int64_t per_xcd = nwg / kXcds;
    const int64_t item = (int64_t)(wg % kXcds) * per_xcd + wg / kXcds;
    if (item >= items) return;
    const int hq = (int)(item % HQ);
    const int grp = (int)((item / HQ) % G);
    const int64_t seg = (item / HQ / G) % nseg_grid;
    const int b = (int)(item / HQ / G / nseg_grid);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool aux = wave >= SW;                 // copy / score wave
    const int sw = aux ? 0 : wave;               // state wave index (aux waves: unused)
    const int l32 = lane & 31, g2 = lane >> 5;
    const int trow = (lane & 15) >> 2, tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    // B's transposing reads take the column quads of each 16 in the order
    // 0, 2, 1, 3: the state rows then come out of stage 3 in an order in which
    // the 8 rows that lane (l32, g2) holds in registers 8hf .. 8hf+7 of tile nt
    // are the consecutive n = 32nt + 16hf + 8g2 + 0..7 (the stage-5 operand
    // order of a plain 16-byte row read of C, and 32 contiguous bytes of a
    // state row in memory).
    const int tcolb = 16 * ((lane >> 4) & 1) + 4 * ((lane & 3) == 1 ? 2 : (lane & 3) == 2 ? 1 : (lane & 3));
    const int hl0 = hq * HW;                     // first head of the set within the group
    const int hw = sw % HW;                      // this state wave's head within the set
    const int hlw = hl0 + hw;
    const bool hvalid = !aux && hlw < HPG;
    const int h = grp * HPG + (hlw < HPG ? hlw : HPG - 1);  // this wave's head (clamped)
    const int pc = (sw / HW) * 32;               // this wave's first head-dim column
    const int64_t PN = (int64_t)P * N;
    const int64_t nblk = (L + kT - 1) / kT;
    const int64_t c_begin = seg * blocks_per_seg;
    const int64_t c_end = (c_begin + blocks_per_seg < nblk) ? c_begin + blocks_per_seg : nblk;
    const int GN = G * N;

    auto block_last = [&](int64_t c) -> int {
        const int64_t last = L - 1 - c * kT;
        return (int)(last < kT - 1 ? last : kT - 1);
    };
    // Time order of the sequence arrays.  rev: step t of the problem is step
    // L - 1 - t of X, B, C and Y, and its decay is a at step L - t (none at
    // t = 0), the time-reversed problem of the backward read in place (L a
    // multiple of the block: block c is the memory block L/kT - 1 - c, rows
    // reversed).  row_base: first memory row of block c; row_loc: memory row
    // of the block's step r relative to it.
    auto row_base = [&](int64_t c) -> int64_t { return rev ? L - kT * (c + 1) : c * kT; };
    auto row_loc = [&](unsigned r) -> unsigned { return rev ? (unsigned)(kT - 1) - r : r; };
    // Per-lane element offsets into the swizzled LDS tiles, loop invariant.
    // Tile row bases that are multiples of 16 rows (and so of the swizzle
    // period) are added per use as immediates.
    //  roff: row reads of B / C (lane = row l32, the 16 bytes at column
    //        nt*32 + 16hf + 8*g2);
    //  toff: transposing reads of B (source row 8*g2 + 4s + trow, columns
    //        nt*32 + tcolb);  xoff: those of this wave's X head-dim tile
    //        (columns pc + tcol).
    uint32_t roff[NTL][2], toff[NTL][2], xoff[2];
#pragma unroll
    for (int nt = 0; nt < NTL; ++nt)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) roff[nt][hf] = (uint32_t)swz<BPR>(l32, nt * 32 + 16 * hf + 8 * g2);
#pragma unroll
    for (int sh = 0; sh < 2; ++sh) {
        const int r = 8 * g2 + 4 * sh + trow;
#pragma unroll
        for (int nt = 0; nt < NTL; ++nt) toff[nt][sh] = (uint32_t)swz<BPR>(r, nt * 32 + tcolb);
        xoff[sh] = (uint32_t)swz<XPR>(r, pc + tcol);
    }
    // Row fragment of B or C: row 32I + l32, columns nt*32 + 16hf + 8*g2 .. +7
    // (k in natural order within the 16-wide step hf).
    auto rowfrag = [&](const u16* tile, int I, int nt, int hf) {
        return as_bf16x8(*reinterpret_cast<const u32x4*>(tile + 32 * I * N + roff[nt][hf]));
    };

    // ---- copies (aux waves only).  Copy k of X, B or C by aux thread at
    // fills the 16-byte LDS slot k * kAuxThreads + at (a is copied per head,
    // lane = step).  A thread's piece within a row is fixed, and so is the
    // row's swizzle; per copy only a uniform row or head base changes.  Rows past the end of the sequence are clamped to
    // the last valid row (their scores are masked, their state weight is zero
    // and their outputs are not stored). ----
    const unsigned at = (unsigned)(tid - SW * 64);           // aux thread (valid for aux waves)
    const unsigned aw = (unsigned)(wave - SW);
    constexpr unsigned XHT = kT * XPR;                          // slots per head tile
    constexpr unsigned BRS = kAuxThreads / BPR;                 // B / C rows per copy
    const unsigned br0 = at / BPR, bq = at % BPR;
    // X copies of aux wave vw's slots (either aux wave may issue them)
    auto copy_x = [&](int64_t c, int bf, unsigned vw) {
        const unsigned atv = vw * 64 + (unsigned)lane;
        const unsigned xr0 = atv / XPR, xlp = (atv % XPR) ^ (unsigned)swzbits<XPR>((int)(atv / XPR));
        const unsigned lc = (unsigned)block_last(c);
        const u16* Xg;
        if constexpr (XG) Xg = X + (((int64_t)b * L + row_base(c)) * x_groups + grp / (G / x_groups)) * (HPG * P);
        else Xg = X + (((int64_t)b * L + row_base(c)) * H + grp * HPG) * P;
#pragma unroll
        for (int k = 0; k < XOPS; ++k) {
            const unsigned s0 = (unsigned)k * kAuxThreads;      // first slot of the copy
            const unsigned hh = s0 / XHT;                       // uniform: a copy stays in one head
            const unsigned r = (s0 % XHT) / XPR + xr0;
            const unsigned tr = row_loc(r <= lc ? r : lc);
            const unsigned hx = hl0 + hh < (unsigned)HPG ? hl0 + hh : HPG - 1;
            if constexpr (XG)
                dma16(Xg, (tr * (unsigned)(x_groups * HPG * P) + hx * P + xlp * 8) * 2u,
                      lds_addr(&sX[bf][0]) + (uint32_t)((s0 + vw * 64) * 16));
            else
                dma16(Xg, ((tr * (unsigned)H + hx) * P + xlp * 8) * 2u,
                      lds_addr(&sX[bf][0]) + (uint32_t)((s0 + vw * 64) * 16));
        }
    };
    auto copy_bc = [&](int64_t c, int bf, bool isB) {
        const unsigned lc = (unsigned)block_last(c);
        const u16* Tg = (isB ? B : C) + (((int64_t)b * L + row_base(c)) * G + grp) * N;
        const u16* tile = isB ? &sB[bf][0] : &sC[FULL ? bf : 0][0];
#pragma unroll
        for (int k = 0; k < BOPS; ++k) {
            const unsigned r = (unsigned)k * BRS + br0;
            const unsigned tr = row_loc(r <= lc ? r : lc);
            const unsigned q = bq ^ (unsigned)swzbits<BPR>((int)r);
            dma16(Tg, (tr * (unsigned)GN + q * 8) * 2u,
                  lds_addr(tile) + (uint32_t)((k * kAuxThreads + aw * 64) * 16));
        }
    };
    // a of the heads this copy wave scans (hh % 2 == aw), lane = step: the
    // wave that scans a head also copies it, so its own wait suffices
    auto copy_a = [&](int64_t c, int ia) {
        const unsigned lc = (unsigned)block_last(c);
        const float* ag;
        if constexpr (XG) ag = a + ((int64_t)b * L + row_base(c)) * G + grp;
        else ag = a + ((int64_t)b * L + row_base(c)) * H + grp * HPG;
        // rev: the decay of step t is a at memory step L - t, one row past
        // step t's own; for t = 0 (c = 0, lane 0) that is past the end, so
        // the lane reads a row inside and stage 1 takes zero instead
        const unsigned tr0 = (unsigned)lane <= lc ? (unsigned)lane : lc;
        const unsigned tr = !rev ? tr0 : (c == 0 && tr0 == 0) ? (unsigned)(kT - 1) : (unsigned)kT - tr0;
#pragma unroll
        for (int hh = 0; hh < HW; ++hh) {
            if ((hh & 1) != (int)aw) continue;
            const unsigned hx = hl0 + hh < (unsigned)HPG ? hl0 + hh : HPG - 1;
            if constexpr (XG) dma4(ag, tr * (unsigned)G * 4u, lds_addr(&sA[ia][hh * kT]));
            else dma4(ag, (tr * (unsigned)H + hx) * 4u, lds_addr(&sA[ia][hh * kT]));
        }
    };

    // The true state is 2^ld * Sacc.  In a block whose log2-decays stay within
    // range of the state scale (the common case) the decay is never applied to
    // the accumulators: with X~_j = 2^(-ld - cs2_j) X_j
    //   Y_i     = 2^(cs2_i + ld) * (C_i Sacc + sum_{j<=i} (C_i . B_j) X~_j)
    //   Sacc'   = Sacc + B^T X~,   ld' = ld + Lam2,
    // so stages 2 and 5 share one accumulator, the scores need only the causal
    // mask (and so are the same for every head), and one per-step factor
    // scales the output.  Each 16-step quarter of the block (one MFMA k step)
    // is checked on its own: a quarter whose prefix sums (relative to its
    // start) lie in [-neg, pos] keeps every weight exponent -ld - cs2_j and
    // output exponent cs2_i + ld within +-kRange exactly when ld lies in
    // [neg - kRange, kRange - pos] (neg and pos follow from the quarter's
    // total and its sum of |a|).  When the scale reached at a quarter's start
    // falls outside that interval it is re-based to the interval's centre,
    // -Lam_q / 2: at the block start by multiplying Sacc, inside the block by
    // multiplying Sacc between the quarters' stage-3 products and the output
    // accumulators of the rows from that quarter on between the quarters'
    // stage-2 products; that quarter's X~ and output factors then use its own
    // prefix sums.  Such a scale exists when the quarter's spread neg + pos is
    // at most 2 kRange (kSpan keeps a margin so the factor between two
    // quarters' references stays below 2^127).  Only a block with a wider
    // quarter takes the direct form: per-element decay of the shared scores,
    // then Sacc' = 2^(ld + Lam2) Sacc + B^T (w o X), ld' = 0.
    //
    // Stage 1 (the scans of a and these decisions) runs on the copy waves one
    // block ahead; the state waves read the decisions, the output exponents
    // and the weights of their head from LDS.
    constexpr int kQ = 4;          // 16-step quarters of a block (one MFMA k step each)
    constexpr float kRange = 64.f;
    constexpr float kSpan = 2.f * kRange - 8.f;
    auto fits = [](float l, float absh, float lamh_) {
        return l >= 0.5f * (absh - lamh_) - kRange && l <= kRange - 0.5f * (absh + lamh_);
    };
    if (aux) {
        // ================= copy waves: copies, scores and stage 1 =================
        // (copy and state waves run separate loops with the same two barriers
        // per block, so neither keeps the other's values in registers)
        // Stage 1 of block c+1 runs here, after the copies of block c, while
        // the state waves work on block c: a is copied two blocks ahead (three
        // buffers), so a[c+1] has landed by the top of block c.  Copy wave aw
        // handles the heads hh with hh % 2 == aw (it copied their a itself)
        // and tracks their scale ld across blocks.
        float ldh[HW];
#pragma unroll
        for (int hh = 0; hh < HW; ++hh) ldh[hh] = 0.f;
        auto decide = [&](int64_t cn) {
            const int ia = (int)((cn - c_begin) % 3), io = (int)((cn - c_begin) & 1);
            const int lastn = block_last(cn);
#pragma unroll
            for (int hh = 0; hh < HW; ++hh) {
                if ((hh & 1) != (int)aw) continue;
                // prefix sums of a (lane = step) and the sums of |a| over each
                // quarter, which bound the spread of cs2 within it (log2 units)
                const bool first = rev && cn == 0 && lane == 0;   // reversed step 0 has no decay
                const float av = lane <= lastn && !first ? sA[ia][hh * kT + lane] : 0.f;
                float absa = fabsf(av);
                const float cs2 = wave_scan64_rowsum(av, absa, lane) * kLog2e;
                float base[kQ + 1], lamq[kQ], absq[kQ];   // base[q]: cs2 before quarter q
                base[0] = 0.f;
                bool fast = !XG;
#pragma unroll
                for (int q = 0; q < kQ; ++q) {
                    base[q + 1] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cs2), 16 * q + 15));
                    absq[q] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(absa), 16 * q + 15)) * kLog2e;
                    lamq[q] = base[q + 1] - base[q];
                    fast = fast & (absq[q] <= kSpan);                 // wave-uniform
                }
                const float lam2 = base[kQ];
                const float ld = ldh[hh];
                const bool rebase = fast & !fits(ld, absq[0], lamq[0]);   // re-base the state scale
                const float target = -0.5f * lamq[0];
                const float pre = rebase ? fast_exp2(ld - target) : 1.f;
                const float ld_in = rebase ? target : ld;
                // reference of each quarter; rq[q] != 0: re-based at the start of
                // quarter q (the accumulators then take the factor 2^(rq[q]))
                float ldq[kQ], rq[kQ];
                ldq[0] = ld_in;
                rq[0] = 0.f;
#pragma unroll
                for (int q = 1; q < kQ; ++q) {
                    const float raw = ldq[q - 1] + lamq[q - 1];
                    const bool fold = fast & !fits(raw, absq[q], lamq[q]);
                    ldq[q] = fold ? -0.5f * lamq[q] : raw;
                    rq[q] = raw - ldq[q];
                }
                const float ld_out = fast ? ldq[kQ - 1] + lamq[kQ - 1] : 0.f;
                ldh[hh] = ld_out;
                // this lane's step j: quarter qj; state weight 2^(wsh - cs2_j), and
                // (fast form) output exponent cs2_j - base + reference
                const int qj = lane >> 4;
                const float bj = qj == 0 ? base[0] : qj == 1 ? base[1] : qj == 2 ? base[2] : base[3];
                const float lj = qj == 0 ? ldq[0] : qj == 1 ? ldq[1] : qj == 2 ? ldq[2] : ldq[3];
                const float wsh = fast ? bj - lj : lam2;
                sCs[io][hh][lane] = fast ? cs2 - bj + lj : cs2;
                sW[io][hh][lane] = lane <= lastn ? fast_exp2(wsh - cs2) : 0.f;
                if (lane == 0) {
                    *reinterpret_cast<float4*>(&sPar[io][hh][0]) = make_float4(fast ? 1.f : 0.f, pre, ld_in, lam2);
                    *reinterpret_cast<float4*>(&sPar[io][hh][4]) = make_float4(rq[1], rq[2], rq[3], ld_out);
                }
            }
        };
        if (c_begin < c_end) {
            // a of the first block first; its stage 1 runs as soon as that copy
            // has landed, while the larger copies are still in flight (the
            // second a copy repeats the first block's when there is no second)
            copy_a(c_begin, 0);
            copy_a(c_begin + 1 < c_end ? c_begin + 1 : c_begin, 1);
            copy_x(c_begin, 0, aw);
            copy_bc(c_begin, 0, true);
            if constexpr (FULL) copy_bc(c_begin, 0, false);
            constexpr int kRest = XOPS + BOPS + (FULL ? BOPS : 0);
            if (aw == 0) vm_wait_le<(HW + 1) / 2 + kRest>();
            else vm_wait_le<HW / 2 + kRest>();
            decide(c_begin);
        }
        for (int64_t c = c_begin; c < c_end; ++c) {
            const int bf = (int)((c - c_begin) & 1);
            const bool has_next = c + 1 < c_end;
            vm_wait_all();   // the copies of block c (and a of block c+1) are done
            sync_lds();      // ... and visible; buffer bf^1 and the score tiles are free
            const u16* bT = &sB[bf][0];
            (void)bT;
            if constexpr (FULL) {
                // ---- shared masked scores: aux wave 0 forms tiles 0 and 1, aux
                // wave 1 tile 2, tile t = (I, J) in {(0,0), (1,0), (1,1)} as
                // S^T = B_J C_I^T, stored [i][j] in bf16 ----
                const u16* cT = &sC[bf][0];
#pragma unroll
                for (int t = 0; t < 3; ++t) {
                    if ((t < 2) != (aw == 0)) continue;
                    const int I = t > 0 ? 1 : 0, J = t == 2 ? 1 : 0;
                    f32x16 St = zero16();
#pragma unroll
                    for (int nt = 0; nt < NTL; ++nt)
#pragma unroll
                        for (int hf = 0; hf < 2; ++hf) St = mfma32(rowfrag(bT, J, nt, hf), rowfrag(cT, I, nt, hf), St);
                    // row j of accumulator register r: 8(r/4) + 4*g2 + r%4; lane = i.
                    // Masked entries (j > i on the diagonal) are replaced, never multiplied.
                    // decayed by 2^(cs2_i - cs2_j) (the direct form's exponents,
                    // shared by every head here), split into high and low parts
                    const bool diag = I == J;
                    const float csi = sCs[bf][0][32 * I + l32];
                    u16* prow = &sP[t][l32 * 32];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int j0 = 8 * q + 4 * g2;
                        const float4 cj = *reinterpret_cast<const float4*>(&sCs[bf][0][32 * J + j0]);
                        const float cjv[4] = {cj.x, cj.y, cj.z, cj.w};
                        float v[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            v[e] = (!diag || j0 + e <= l32) ? St[4 * q + e] * fast_exp2(csi - cjv[e]) : 0.f;
                        const uint32_t h01 = pack2(v[0], v[1]), h23 = pack2(v[2], v[3]);
                        const uint32_t l01 = pack2(v[0] - __uint_as_float(h01 << 16), v[1] - __uint_as_float(h01 & 0xffff0000u));
                        const uint32_t l23 = pack2(v[2] - __uint_as_float(h23 << 16), v[3] - __uint_as_float(h23 & 0xffff0000u));
                        const int off = 8 * (q ^ ((l32 >> 2) & 3)) + 4 * g2;
                        *reinterpret_cast<uint2*>(prow + off) = make_uint2(h01, h23);
                        *reinterpret_cast<uint2*>(prow + 32 * 32 + off) = make_uint2(l01, l23);
                    }
                }
            }
            if constexpr (FULL) sync_lds();  // the shared score tiles are complete
            // ---- copies of block c+1 (each copy wave fills its own half of X) ----
            if (has_next) {
                copy_x(c + 1, bf ^ 1, aw);
                if (c + 2 < c_end) copy_a(c + 2, (int)((c + 2 - c_begin) % 3));
                copy_bc(c + 1, bf ^ 1, true);
                if constexpr (FULL) copy_bc(c + 1, bf ^ 1, false);
                decide(c + 1);   // after the copies are on their way
            }
        }
        return;
    }

    // ================= state waves =================
    // ---- carried state (state waves): S^T tiles (rows n, columns p of this
    // wave's tile); register r of tile nt holds n = 32nt + 16(r/8) + 8g2 + r%8
    // of column p = pc + l32 ----
    f32x16 Sacc[NTL];
#pragma unroll
    for (int nt = 0; nt < NTL; ++nt) Sacc[nt] = zero16();
    if constexpr (FULL) {
        const float* S0 = seg == 0 ? (src.first ? src.first + b * src.first_bstride : nullptr)
                                   : (src.Sin ? src.Sin + b * src.bstride + seg * src.sstride : nullptr);
        if (S0) {
            // transposed: Sacc(p, n) = S[grp][n][hl*P + p] of an [N][HPG*P] state
            const int hlc = hlw < HPG ? hlw : HPG - 1;
            const float* St = S0 + (int64_t)grp * HPG * PN + hlc * P + pc + l32;
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    Sacc[nt][r] = St[(int64_t)(nt * 32 + 16 * (r >> 3) + 8 * g2 + (r & 7)) * (HPG * P)];
        }
    }
    float lam2_total = 0.f;   // the segment's log2-decay
    float ld = 0.f;           // the scale of Sacc (log2) after the latest block
    for (int64_t c = c_begin; c < c_end; ++c) {
        const int bf = (int)((c - c_begin) & 1);
        const int last = block_last(c);
        sync_lds();   // the block's copies are visible

        const u16* bT = &sB[bf][0];
        const u16* xT = &sX[bf][hw * kT * P];
        // X^T fragments of this wave's head-dim tile (lane = p, k = step)
        auto xfrag = [&](int J, int ks) {
            const u16* t = xT + (32 * J + 16 * ks) * P;
            return join8(lds_tr4(t + xoff[0]), lds_tr4(t + xoff[1]));
        };
        // ... weighted in registers, X~ = w o X: the fragment's k values are
        // the steps 32J + 16ks + 8g2 + 0..7, whose state weights stage 1 left
        // in LDS (X itself stays unweighted in LDS for the direct form)
        auto xwfrag = [&](int J, int ks) {
            const float* wp = &sW[bf][hw][32 * J + 16 * ks + 8 * g2];
            const float4 w0 = *reinterpret_cast<const float4*>(wp);
            const float4 w1 = *reinterpret_cast<const float4*>(wp + 4);
            const float w8[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
            return scale8(xfrag(J, ks), w8);
        };

        // ---- the block's stage-1 results for this wave's head ----
        const float4 pa = *reinterpret_cast<const float4*>(&sPar[bf][hw][0]);
        const float4 pb = *reinterpret_cast<const float4*>(&sPar[bf][hw][4]);
        auto uni = [](float v) { return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v))); };
        const bool fast = !XG && uni(pa.x) != 0.f;   // (XG: always the direct form)
        const float pre = uni(pa.y), ld_in = uni(pa.z), lam2 = uni(pa.w);
        const float rq[kQ] = {0.f, uni(pb.x), uni(pb.y), uni(pb.z)};
        const bool fold[kQ] = {false, rq[1] != 0.f, rq[2] != 0.f, rq[3] != 0.f};
        ld = uni(pb.w);
        lam2_total += lam2;
        if (pre != 1.f) {   // the block's re-based scale (fast form only), before stage 5
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt) Sacc[nt] *= pre;
        }

        f32x16 Yt[2] = {zero16(), zero16()};
        if constexpr (FULL) {
            // ---- stage 5 (at the block's re-based scale): Y^T = Sacc C^T ----
            const u16* cT = &sC[bf][0];
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const bf16x8 Sf = acc_half(Sacc[nt], hf);
#pragma unroll
                    for (int I = 0; I < 2; ++I) Yt[I] = mfma32(Sf, rowfrag(cT, I, nt, hf), Yt[I]);
                    if constexpr (XG) {   // the state's low part
                        const bf16x8 Sl = acc_half_lo(Sacc[nt], hf, Sf);
#pragma unroll
                        for (int I = 0; I < 2; ++I) Yt[I] = mfma32(Sl, rowfrag(cT, I, nt, hf), Yt[I]);
                    }
                }
        }

        if constexpr (FULL) sync_lds();  // the shared score tiles are complete

        bf16x8 xk[4];   // X~ fragments (J, ks) = (0,0), (0,1), (1,0), (1,1)
        if constexpr (FULL) {
            // stage 5's part at the block's entering scale, then stage 2 in the
            // direct form: the copy waves' decayed scores, high and low parts,
            // on unweighted X
            Yt[0] *= fast_exp2(sCs[bf][hw][l32] + ld_in);
            Yt[1] *= fast_exp2(sCs[bf][hw][32 + l32] + ld_in);
            auto pt = [&](int t, int ks, int part) {
                return as_bf16x8(*reinterpret_cast<const u32x4*>(
                    &sP[t][part * 32 * 32 + l32 * 32 + 8 * ((2 * ks + g2) ^ ((l32 >> 2) & 3))]));
            };
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const bf16x8 xa0 = xfrag(0, ks);
                const bf16x8 xa1 = xfrag(1, ks);
#pragma unroll
                for (int part = 0; part < 2; ++part) {
                    Yt[0] = mfma32(xa0, pt(0, ks, part), Yt[0]);
                    Yt[1] = mfma32(xa0, pt(1, ks, part), Yt[1]);
                    Yt[1] = mfma32(xa1, pt(2, ks, part), Yt[1]);
                }
            }
            // fp32 out, straight from the accumulators (lane = step, four
            // consecutive head-dim entries per register quad): the backward
            // sums these over a group's heads before rounding, reading them
            // once (non-temporal stores: they do not stay in the caches)
            if (hvalid) {
                typedef float f32x4_nt __attribute__((ext_vector_type(4)));
                float* yrow = reinterpret_cast<float*>(Y) + (((int64_t)b * L + row_base(c)) * H + h) * P + pc + 4 * g2;
#pragma unroll
                for (int I = 0; I < 2; ++I)
                    if (32 * I + l32 <= last)
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            __builtin_nontemporal_store(
                                f32x4_nt{Yt[I][4 * q], Yt[I][4 * q + 1], Yt[I][4 * q + 2], Yt[I][4 * q + 3]},
                                reinterpret_cast<f32x4_nt*>(yrow + (int64_t)row_loc((unsigned)(32 * I + l32)) * H * P + 8 * q));
            }
        }

        // ---- stages 3 + 4: Sacc' = (direct form: 2^(ld + Lam2)) Sacc + B^T X~ ----
        if (!fast) {
            const float f = fast_exp2(ld_in + lam2);
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt) Sacc[nt] *= f;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) xk[i] = xwfrag(i >> 1, i & 1);
#pragma unroll
        for (int J = 0; J < 2; ++J) {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                if (fold[2 * J + ks]) {   // the state so far at this quarter's reference
                    const float f = fast_exp2(rq[2 * J + ks]);
#pragma unroll
                    for (int nt = 0; nt < NTL; ++nt) Sacc[nt] *= f;
                }
                const bf16x8 xw = xk[2 * J + ks];
#pragma unroll
                for (int nt = 0; nt < NTL; ++nt) {
                    const u16* t = bT + (32 * J + 16 * ks) * N;
                    const bf16x8 Af = join8(lds_tr4(t + toff[nt][0]), lds_tr4(t + toff[nt][1]));
                    Sacc[nt] = mfma32(Af, xw, Sacc[nt]);
                }
            }
        }
    }

    // ---- epilogue: final state (full pass, last segment) or segment summary ----
    if (!hvalid) return;
    float* Sdst = nullptr;
    if constexpr (FULL) {
        if (S_fin && seg == nseg_grid - 1) Sdst = S_fin + ((int64_t)b * H + h) * PN;
    } else {
        Sdst = Sseg + (((int64_t)b * nseg_total + seg) * H + h) * PN;
        if (lamseg && lane == 0 && pc == 0)
            lamseg[((int64_t)b * H + h) * nseg_total + seg] = lam2_total * 0.69314718055994531f;
    }
    if (Sdst) {
        const float f = fast_exp2(ld);
#pragma unroll
        for (int nt = 0; nt < NTL; ++nt) {
            float* row = Sdst + (int64_t)(pc + l32) * N + nt * 32 + 8 * g2;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                *reinterpret_cast<float4*>(row + 16 * (q >> 1) + 4 * (q & 1)) =
                    make_float4(f * Sacc[nt][4 * q], f * Sacc[nt][4 * q + 1], f * Sacc[nt][4 * q + 2],
                                f * Sacc[nt][4 * q + 3]);
        }
    }
}

template <int P, int N, bool FULL, bool XG = false, int SW = kStateWaves>
__global__ __launch_bounds__(64 * (SW + 2)) __attribute__((amdgpu_waves_per_eu(SW == kStateWaves ? 2 : 3))) void k_mfma_seg(
    const u16* __restrict__ X, const float* __restrict__ a, const u16* __restrict__ B,
    const u16* __restrict__ C, StateSrc src, u16* __restrict__ Y, float* __restrict__ S_fin,
    float* __restrict__ Sseg, float* __restrict__ lamseg, int64_t nseg_total, int64_t L,
    int H, int G, int64_t blocks_per_seg, int nseg_grid, int Bz, int x_groups, int rev)
{
    mfma_seg_body<P, N, FULL, XG, SW>(X, a, B, C, src, Y, S_fin, Sseg, lamseg, nseg_total, L, H, G,
                                      blocks_per_seg, nseg_grid, Bz, x_groups, blockIdx.x, gridDim.x, rev);
}

// Two exchanged-dimension products in one launch (the backward's dC and dB
// passes): workgroups [0, grid0) run the first, the rest the second.  Both
// share every size but the sequence length; grid0 is a multiple of the XCD
// count, so a workgroup's XCD is the same in either numbering.
template <int SW>
__global__ __launch_bounds__(64 * (SW + 2)) __attribute__((amdgpu_waves_per_eu(3))) void k_mfma_xg_pair(
    XgPass p0, XgPass p1, unsigned grid0, int H, int G, int64_t blocks_per_seg, int nseg_grid, int Bz,
    int x_groups)
{
    const bool second = blockIdx.x >= grid0;
    const XgPass& p = second ? p1 : p0;
    const unsigned wg = second ? blockIdx.x - grid0 : blockIdx.x;
    const unsigned nwg = second ? gridDim.x - grid0 : grid0;
    mfma_seg_body<64, 64, true, true, SW>(static_cast<const u16*>(p.X), p.a, static_cast<const u16*>(p.B),
                                          static_cast<const u16*>(p.C), p.src, reinterpret_cast<u16*>(p.Y),
                                          nullptr, nullptr, nullptr, 0, p.L, H, G, blocks_per_seg, nseg_grid,
                                          Bz, x_groups, wg, nwg, p.rev);
}

constexpr int kCbWaves = 4;

template <int N>
__global__ __launch_bounds__(64 * kCbWaves) void k_cb_tiles(CbJob j)
{
    cb_tiles_wg<N, kCbWaves>(j, blockIdx.x, threadIdx.x >> 6, threadIdx.x & 63);
}

// Two state-only passes in one launch (the backward's forward-time and
// reversed-time chunk states): workgroups [0, grid0) run the first, the rest
// the second.  Both share every size; grid0 is a multiple of the XCD count.
template <int P, int N>
__global__ __launch_bounds__(64 * (kStateWaves + 2)) __attribute__((amdgpu_waves_per_eu(2))) void k_mfma_state_pair(
    StatePass p0, StatePass p1, unsigned grid0, int64_t nseg_total, int64_t L, int H, int G,
    int64_t blocks_per_seg, int nseg_grid, int Bz)
{
    const bool second = blockIdx.x >= grid0;
    const StatePass& p = second ? p1 : p0;
    const unsigned wg = second ? blockIdx.x - grid0 : blockIdx.x;
    const unsigned nwg = grid0;
    const StateSrc none{nullptr, 0, nullptr, 0, 0};
    mfma_seg_body<P, N, false, false, kStateWaves>(static_cast<const u16*>(p.X), p.a, static_cast<const u16*>(p.B),
                                                   nullptr, none, nullptr, nullptr, p.Sseg, p.lamseg, nseg_total, L,
                                                   H, G, blocks_per_seg, nseg_grid, Bz, 0, wg, nwg, p.rev);
}

#define SSD_MFMA_DISPATCH(MACRO)                     \
    if (s.P == 64 && s.N == 128) MACRO(64, 128)      \
    else if (s.P == 64 && s.N == 64) MACRO(64, 64)   \
    else if (s.P == 32 && s.N == 128) MACRO(32, 128) \
    else if (s.P == 32 && s.N == 64) MACRO(32, 64)   \
    else return hipErrorInvalidValue;

// one workgroup per (batch, segment, group, head set) item, padded to a multiple of the XCD count
static unsigned grid_for(const FwdShape& s, int64_t nseg) {
    const int64_t hw = mfma_heads_per_workgroup(s.P, s.N);
    const int64_t hq = (s.H / s.G + hw - 1) / hw;
    const int64_t items = s.Bz * nseg * s.G * hq;
    return (unsigned)(((items + kXcds - 1) / kXcds) * kXcds);
}

hipError_t launch_mfma_state(const FwdShape& s, int64_t seg_chunks, int64_t nseg_run,
                             int64_t nseg_total, const void* X, const float* a,
                             const void* B, float* Sseg, float* lamseg, hipStream_t st, bool rev)
{
    if (nseg_run <= 0) return hipSuccess;
    if (rev && s.L % kT != 0) return hipErrorInvalidValue;
    const dim3 grid(grid_for(s, nseg_run));
    const StateSrc none{nullptr, 0, nullptr, 0, 0};
    const int64_t bps = seg_chunks * (s.Q / kT);
#define SSD_LAUNCH_STATE(PP, NN)                                                              \
    hipLaunchKernelGGL((k_mfma_seg<PP, NN, false>), grid, dim3(kThreads), 0, st,             \
                       (const u16*)X, a, (const u16*)B, (const u16*)nullptr, none,          \
                       (u16*)nullptr, (float*)nullptr, Sseg, lamseg, nseg_total, s.L,       \
                       (int)s.H, (int)s.G, bps, (int)nseg_run, (int)s.Bz, 0, rev ? 1 : 0);
    SSD_MFMA_DISPATCH(SSD_LAUNCH_STATE)
#undef SSD_LAUNCH_STATE
    return hipGetLastError();
}

hipError_t launch_cb_tiles(const CbJob& j, hipStream_t st)
{
    const int64_t nwg = cb_workgroups(j, kCbWaves);
    if (nwg <= 0) return hipSuccess;
    if (j.N == 128) hipLaunchKernelGGL((k_cb_tiles<128>), dim3((unsigned)nwg), dim3(64 * kCbWaves), 0, st, j);
    else if (j.N == 64) hipLaunchKernelGGL((k_cb_tiles<64>), dim3((unsigned)nwg), dim3(64 * kCbWaves), 0, st, j);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_mfma_state_pair(const FwdShape& s, int64_t seg_chunks, int64_t nseg_run, int64_t nseg_total,
                                  const StatePass& p0, const StatePass& p1, hipStream_t st)
{
    if (nseg_run <= 0) return hipSuccess;
    if ((p0.rev || p1.rev) && s.L % kT != 0) return hipErrorInvalidValue;
    const unsigned grid0 = grid_for(s, nseg_run);
    const int64_t bps = seg_chunks * (s.Q / kT);
#define SSD_LAUNCH_STATE_PAIR(PP, NN)                                                         \
    hipLaunchKernelGGL((k_mfma_state_pair<PP, NN>), dim3(2 * grid0), dim3(kThreads), 0, st, p0, p1, \
                       grid0, nseg_total, s.L, (int)s.H, (int)s.G, bps, (int)nseg_run, (int)s.Bz);
    SSD_MFMA_DISPATCH(SSD_LAUNCH_STATE_PAIR)
#undef SSD_LAUNCH_STATE_PAIR
    return hipGetLastError();
}

hipError_t launch_mfma_out_xg_pair(const FwdShape& s, int64_t x_groups, const XgPass& p0, const XgPass& p1,
                                   hipStream_t st)
{
    if (!(s.P == 64 && s.N == 64) || x_groups < 1 || s.G % x_groups != 0) return hipErrorInvalidValue;
    if ((p0.L + s.Q - 1) / s.Q != s.nc || (p1.L + s.Q - 1) / s.Q != s.nc) return hipErrorInvalidValue;
    if ((p0.rev && p0.L % kT != 0) || (p1.rev && p1.L % kT != 0)) return hipErrorInvalidValue;
    // four state waves: two sub-heads of 64 per workgroup (a group has H/G of them)
    constexpr int kSW = 4;
    const int64_t hq = (s.H / s.G + kSW / 2 - 1) / (kSW / 2);
    const int64_t items = s.Bz * s.nc * s.G * hq;
    const unsigned grid0 = (unsigned)(((items + kXcds - 1) / kXcds) * kXcds);
    const int64_t bps = s.Q / kT;
    hipLaunchKernelGGL((k_mfma_xg_pair<kSW>), dim3(2 * grid0), dim3(64 * (kSW + 2)), 0, st, p0, p1, grid0,
                       (int)s.H, (int)s.G, bps, (int)s.nc, (int)s.Bz, (int)x_groups);
    return hipGetLastError();
}

}  // namespace ssd
