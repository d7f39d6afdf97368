// api.cpp -- the C ABI of libssd.so (declared in include/ssd.h).
//
// Every entry point validates all of its arguments on the host before the
// first HIP call; a rejected call enqueues nothing and writes no output.
// Accepted calls only enqueue work on the caller's stream.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "ssd.h"
#include "ssd_launch.hpp"

namespace {

thread_local char g_err[512] = "";

ssd_status fail(ssd_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

ssd_status ok() {
    g_err[0] = '\0';
    return SSD_OK;
}

ssd_status hip_fail(hipError_t e, const char* what) {
    return fail(SSD_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

struct Range {
    const char* name;
    uintptr_t lo, hi;  // [lo, hi)
};
Range rng(const char* name, const void* p, int64_t bytes) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{name, lo, p ? lo + (uintptr_t)(bytes > 0 ? bytes : 0) : lo};
}
bool overlap(const Range& a, const Range& b) {
    if (a.lo == a.hi || b.lo == b.hi) return false;
    return a.lo < b.hi && b.lo < a.hi;
}

constexpr int64_t kNumCU = 256;          // MI355X compute units
constexpr int64_t kLdsPerCU = 160 * 1024;
constexpr int64_t kMfmaThreads = 512;    // the largest workgroup of the MFMA kernels

// LDS of the MFMA kernel's full pass for (P, N): double-buffered 64-step
// blocks of X for the workgroup's heads, B and C, the shared score tiles and
// the per-step vectors --
// used to estimate how many workgroups share a CU when planning segments.
int64_t mfma_lds_bytes(int64_t P, int64_t N) {
    const int64_t T = 64, HW = ssd::mfma_heads_per_workgroup(P, N);
    // X, B, C double buffered; a triple buffered; scans, quarter sums, score
    // tiles and the per-wave output exponents
    return 2 * (HW * T * P * 2 + 2 * T * N * 2) + 3 * HW * T * 4 + 2 * HW * T * 4 + 2 * HW * 16 +
           3 * 32 * 40 * 2 + 6 * T * 4;
}

struct Plan {
    int32_t algo;
    int64_t seg_chunks, nseg;
    int sw;          // units per workgroup of the fused pass (MFMA path)
    size_t ws;
    ssd::FwdShape s;
    bool bf16;
};

ssd_status check_desc(const ssd_fwd_desc* d, bool need_chunk_le_256) {
    if (!d) return fail(SSD_ERR_NULL, "desc is NULL");
    if (d->batch < 0 || d->seqlen < 0 || d->nheads < 1 || d->headdim < 1 || d->dstate < 1 ||
        d->ngroups < 1)
        return fail(SSD_ERR_SHAPE,
                    "sizes must be batch>=0, seqlen>=0, nheads,headdim,dstate,ngroups>=1 "
                    "(got %lld,%lld,%lld,%lld,%lld,%lld)",
                    (long long)d->batch, (long long)d->seqlen, (long long)d->nheads,
                    (long long)d->headdim, (long long)d->dstate, (long long)d->ngroups);
    if (d->nheads % d->ngroups != 0)
        return fail(SSD_ERR_SHAPE, "nheads (%lld) must be a multiple of ngroups (%lld)",
                    (long long)d->nheads, (long long)d->ngroups);
    if (d->chunk < 1) return fail(SSD_ERR_SHAPE, "chunk must be >= 1 (got %lld)", (long long)d->chunk);
    if (d->seg_chunks < 0) return fail(SSD_ERR_SHAPE, "seg_chunks must be >= 0");
    if (d->dtype != SSD_F32 && d->dtype != SSD_BF16)
        return fail(SSD_ERR_DTYPE, "dtype %d is not SSD_F32 or SSD_BF16", (int)d->dtype);
    if (d->algo < SSD_ALGO_AUTO || d->algo > SSD_ALGO_MFMA)
        return fail(SSD_ERR_UNSUPPORTED, "unknown algo %d", (int)d->algo);
    if (d->wg_units != 0 && (d->wg_units < 4 || d->wg_units > 6))
        return fail(SSD_ERR_UNSUPPORTED, "wg_units must be 0 (automatic), 4, 5 or 6 (got %d)", (int)d->wg_units);
    if (d->reserved != 0) return fail(SSD_ERR_SHAPE, "reserved must be 0");
    if (need_chunk_le_256 && d->chunk > 256)
        return fail(SSD_ERR_UNSUPPORTED, "chunk %lld > 256", (long long)d->chunk);
    // grid limits (dims are launched as unsigned grid sizes) and 32-bit in-slice indexing
    if (d->nheads > 65535 || d->batch > 65535 || d->headdim * d->dstate > (1 << 24) ||
        d->seqlen > ((int64_t)1 << 40))
        return fail(SSD_ERR_UNSUPPORTED, "sizes beyond the supported range");
    if ((d->headdim * d->dstate) % 4 != 0)
        return fail(SSD_ERR_UNSUPPORTED, "headdim*dstate must be a multiple of 4");
    return SSD_OK;
}

ssd::FwdShape shape_of(const ssd_fwd_desc* d) {
    ssd::FwdShape s;
    s.Bz = d->batch; s.L = d->seqlen; s.H = d->nheads; s.P = d->headdim; s.N = d->dstate;
    s.G = d->ngroups; s.Q = d->chunk;
    s.nc = (s.L + s.Q - 1) / s.Q;
    return s;
}

// Plan of the MFMA path: the segment length k (chunks one workgroup walks
// while carrying the state in registers) and the fused pass's units per
// workgroup sw.  The estimate (microseconds) is a model fitted to timings of
// 49 plans over eight shapes on MI355X at running clocks (most within 7%):
//  - fused pass: one workgroup per CU, so ceil(workgroups / 256) rounds of
//    k * Q / 64 blocks each; a block takes kFusedUs[N][sw] when few
//    workgroups run, plus kOccUs[N] * sw / 5 scaled by the fraction of the
//    CUs in use (HBM and L2 contention);
//  - more than one segment adds the state-only pass (rounds of its
//    workgroups, kStateUs[N] per block), the segment scan's sequential
//    latency per segment, the states' HBM round trip (written by the state
//    pass, read and written by the scan, read by the fused pass) and the two
//    extra launches.
// For each segment count only the most balanced k is tried; the cheapest
// (k, sw) wins, ties going to fewer segments and fewer units.  Segments are
// at most kMaxSegSteps long when that leaves them few enough: longer ones
// measured slower than the model predicts (the 512K-step sweep point: 90-chunk
// segments 1.63 ms against 1.51 ms at 45 chunks).
constexpr int64_t kMaxSegSteps = 16384;
double plan_cost_us(const ssd::FwdShape& s, int64_t k, int sw) {
    constexpr double kFusedUs[2][3] = {{1.88, 1.94, 2.25}, {1.97, 2.70, 2.83}};   // [N > 64][sw - 4]
    constexpr double kOccUs[2] = {0.48, 0.55}, kStateUs[2] = {1.22, 1.30};
    constexpr double kLaunchUs = 6.1, kSegExtraUs = 8.2, kSegLatencyUs = 0.25, kUsPerStateMB = 0.1166;
    const int wide = s.N > 64 ? 1 : 0;
    const int64_t nseg = (s.nc + k - 1) / k;
    const double blocks = (double)k * (double)((s.Q + 63) / 64);
    const int64_t upg = (s.H / s.G) * (s.P / 32);
    const int64_t wg_full = s.Bz * s.G * ((upg + sw - 1) / sw) * nseg;
    const double busy = (double)(wg_full < kNumCU ? wg_full : kNumCU) / (double)kNumCU;
    double cost = kLaunchUs + (double)((wg_full + kNumCU - 1) / kNumCU) * blocks *
                                  (kFusedUs[wide][sw - 4] + kOccUs[wide] * busy * sw / 5.0);
    if (nseg > 1) {
        const int64_t hw = ssd::mfma_heads_per_workgroup(s.P, s.N);
        const int64_t per_cu = kLdsPerCU / mfma_lds_bytes(s.P, s.N);
        const int64_t slots = kNumCU * (per_cu > 0 ? per_cu : 1);
        const int64_t wg_state = s.Bz * s.G * ((s.H / s.G + hw - 1) / hw) * (nseg - 1);
        const double state_mb = 4.0 * (double)(s.Bz * s.H * s.P * s.N) * 4.0 * 1e-6;
        cost += (double)((wg_state + slots - 1) / slots) * blocks * kStateUs[wide];
        cost += kSegExtraUs + kSegLatencyUs * (double)nseg + kUsPerStateMB * state_mb * (double)nseg;
    }
    return cost;
}

// Workspace of the segmented plan: the fp32 states of segments 1 .. nseg-1
// (slot 0 is never used) and the segments' log-decays, each region rounded
// up to 256 bytes; none for a single segment.
size_t fwd_ws_bytes(const ssd::FwdShape& s, int64_t nseg) {
    if (nseg <= 1) return 0;
    const size_t states = (size_t)s.Bz * nseg * s.H * s.P * s.N * sizeof(float);
    const size_t lams = (size_t)s.Bz * s.H * nseg * sizeof(float);
    return ((states + 255) / 256) * 256 + ((lams + 255) / 256) * 256;
}

// Cheapest plan whose workspace fits ws_cap (a single segment always does).
void auto_plan(const ssd::FwdShape& s, int64_t k_fixed, int sw_fixed, size_t ws_cap, int64_t* k_out,
               int* sw_out) {
    const int64_t max_seg = s.nc < 65535 ? s.nc : 65535;
    double best = 1e300;
    int64_t best_k = k_fixed > 0 ? k_fixed : s.nc;
    int best_sw = sw_fixed > 0 ? sw_fixed : 4;
    for (int sw = 4; sw <= 6; ++sw) {
        if ((sw_fixed > 0 && sw != sw_fixed) || !ssd::fwd_units_supported(s.P, sw)) continue;
        int64_t prev_k = -1;
        for (int64_t want = 1; want <= max_seg; ++want) {
            const int64_t k = k_fixed > 0 ? k_fixed : (s.nc + want - 1) / want;   // longest segment
            if (k == prev_k) continue;
            prev_k = k;
            if (k_fixed <= 0 && k * s.Q > kMaxSegSteps && (s.nc + kMaxSegSteps / s.Q - 1) / (kMaxSegSteps / s.Q) <= max_seg)
                continue;
            if (k_fixed <= 0 && fwd_ws_bytes(s, (s.nc + k - 1) / k) > ws_cap) continue;
            const double cost = plan_cost_us(s, k, sw);
            if (cost < best - 1e-9) {
                best = cost;
                best_k = k;
                best_sw = sw;
            }
            if (k_fixed > 0) break;
        }
    }
    *k_out = best_k;
    *sw_out = best_sw;
}

ssd_status make_plan(const ssd_fwd_desc* d, Plan* p, size_t ws_cap = SIZE_MAX) {
    ssd_status st = check_desc(d, false);
    if (st != SSD_OK) return st;
    p->s = shape_of(d);
    p->bf16 = d->dtype == SSD_BF16;
    const ssd::FwdShape& s = p->s;
    const bool mfma_ok = p->bf16 && ssd::mfma_supported(s.Q, s.P, s.N) && s.Q <= 256;
    const bool valu_ok = ssd::valu_fwd_supported(s);
    if (d->algo == SSD_ALGO_MFMA) {
        if (!mfma_ok)
            return fail(SSD_ERR_UNSUPPORTED,
                        "no MFMA kernel for dtype=%d chunk=%lld headdim=%lld dstate=%lld "
                        "(bf16, chunk in {64,128,256}, headdim in {32,64}, dstate in {64,128})",
                        (int)d->dtype, (long long)s.Q, (long long)s.P, (long long)s.N);
        p->algo = SSD_ALGO_MFMA;
    } else if (d->algo == SSD_ALGO_VALU) {
        if (!valu_ok)
            return fail(SSD_ERR_UNSUPPORTED, "VALU kernel needs chunk<=256 and headdim*dstate<=16384");
        p->algo = SSD_ALGO_VALU;
    } else {
        if (mfma_ok) p->algo = SSD_ALGO_MFMA;
        else if (valu_ok) p->algo = SSD_ALGO_VALU;
        else
            return fail(SSD_ERR_UNSUPPORTED, "no kernel for chunk=%lld headdim=%lld dstate=%lld",
                        (long long)s.Q, (long long)s.P, (long long)s.N);
    }
    p->seg_chunks = 0;
    p->nseg = 1;
    p->sw = 0;
    p->ws = 0;
    if (p->algo == SSD_ALGO_MFMA && s.nc > 0 && s.Bz > 0) {
        if (d->wg_units != 0 && !ssd::fwd_units_supported(s.P, d->wg_units))
            return fail(SSD_ERR_UNSUPPORTED, "wg_units %d is not compiled for headdim %lld", (int)d->wg_units,
                        (long long)s.P);
        int64_t k = 0;
        int sw = 0;
        auto_plan(s, d->seg_chunks, d->wg_units, ws_cap, &k, &sw);
        if (k > s.nc) k = s.nc;
        p->sw = sw;
        p->seg_chunks = k;
        p->nseg = (s.nc + k - 1) / k;
        if (p->nseg > 65535) return fail(SSD_ERR_UNSUPPORTED, "too many segments (%lld)", (long long)p->nseg);
        // one-dimensional grid of at most batch*segments*heads workgroups (plus
        // padding to the XCD count) of kMfmaThreads threads each
        if ((s.Bz * p->nseg * s.H + 8) * kMfmaThreads >= ((int64_t)1 << 32))
            return fail(SSD_ERR_UNSUPPORTED, "batch*segments*heads (%lld) too large for one launch",
                        (long long)(s.Bz * p->nseg * s.H));
        p->ws = fwd_ws_bytes(s, p->nseg);
        if (p->ws > ws_cap)
            return fail(SSD_ERR_WORKSPACE,
                        "the requested plan (%lld chunks per segment, %lld segments) needs %zu bytes of "
                        "workspace; the fixed workspace holds %zu",
                        (long long)p->seg_chunks, (long long)p->nseg, p->ws, ws_cap);
    }
    return SSD_OK;
}

ssd_status check_fwd_io(const Plan& p, const void* X, const float* a, const void* B,
                        const void* C, const float* S0, const void* Y, const float* Sfin) {
    const ssd::FwdShape& s = p.s;
    if (s.Bz > 0 && s.L > 0 && (!X || !a || !B || !C || !Y))
        return fail(SSD_ERR_NULL, "X, a, B, C and Y are required");
    const void* v[] = {X, B, C, Y, S0, Sfin};
    const char* nm[] = {"X", "B", "C", "Y", "initial_state", "final_state"};
    for (int i = 0; i < 6; ++i)
        if (v[i] && !aligned(v[i], 16)) return fail(SSD_ERR_ALIGN, "%s is not 16-byte aligned", nm[i]);
    if (a && !aligned(a, 4)) return fail(SSD_ERR_ALIGN, "a is not 4-byte aligned");
    const int64_t es = p.bf16 ? 2 : 4;
    const int64_t nX = s.Bz * s.L * s.H * s.P, nBC = s.Bz * s.L * s.G * s.N;
    const int64_t nS = s.Bz * s.H * s.P * s.N;
    const Range in[] = {rng("X", X, nX * es), rng("a", a, s.Bz * s.L * s.H * 4), rng("B", B, nBC * es),
                        rng("C", C, nBC * es), rng("initial_state", S0, S0 ? nS * 4 : 0)};
    const Range outs[] = {rng("Y", Y, nX * es), rng("final_state", Sfin, Sfin ? nS * 4 : 0)};
    for (const Range& o : outs)
        for (const Range& i : in)
            if (overlap(o, i)) return fail(SSD_ERR_ALIAS, "%s overlaps input %s", o.name, i.name);
    if (overlap(outs[0], outs[1])) return fail(SSD_ERR_ALIAS, "Y overlaps final_state");
    return SSD_OK;
}

// Enqueue the planned forward; every argument has been validated.
ssd_status run_fwd(const Plan& p, const void* X, const float* a, const void* B, const void* C,
                   const float* initial_state, void* Y, float* final_state, void* workspace,
                   hipStream_t hs, bool y_f32 = false) {
    const ssd::FwdShape& s = p.s;
    const int64_t PN = s.P * s.N;
    hipError_t e = hipSuccess;
    if (s.Bz == 0) return ok();
    if (s.L == 0) {
        if (final_state) {
            e = initial_state ? ssd::launch_copy_f32(final_state, initial_state, s.Bz * s.H * PN, hs)
                              : ssd::launch_fill_zero(final_state, s.Bz * s.H * PN, hs);
            if (e != hipSuccess) return hip_fail(e, "empty-sequence final state");
        }
        return ok();
    }
    if (y_f32 && p.algo != SSD_ALGO_VALU)
        return fail(SSD_ERR_UNSUPPORTED, "fp32 output from bf16 inputs needs the VALU kernel");
    if (p.algo == SSD_ALGO_VALU) {
        e = ssd::launch_valu_fwd(s, p.bf16, X, a, B, C, initial_state, Y, final_state, hs, nullptr, y_f32);
        if (e != hipSuccess) return hip_fail(e, "VALU forward launch");
        return ok();
    }
    if (p.nseg == 1) {
        ssd::StateSrc src{initial_state, s.H * PN, nullptr, 0, 0};
        e = ssd::launch_fwd(s, p.sw, p.seg_chunks, 1, X, a, B, C, src, Y, final_state, hs);
        if (e != hipSuccess) return hip_fail(e, "MFMA forward launch");
        return ok();
    }
    float* Sbuf = static_cast<float*>(workspace);
    const size_t states = (size_t)s.Bz * p.nseg * s.H * PN * sizeof(float);
    float* lamseg = reinterpret_cast<float*>(static_cast<char*>(workspace) + ((states + 255) / 256) * 256);
    e = ssd::launch_mfma_state(s, p.seg_chunks, p.nseg - 1, p.nseg, X, a, B, Sbuf, lamseg, hs);
    if (e != hipSuccess) return hip_fail(e, "MFMA segment-state launch");
    // segment 0 starts from initial_state itself, so slot 0 is never written
    e = ssd::launch_state_scan(s, p.nseg - 1, p.nseg, Sbuf, lamseg, s.H * p.nseg, p.nseg,
                               initial_state, Sbuf, 1, Sbuf + (p.nseg - 1) * s.H * PN,
                               p.nseg * s.H * PN, hs);
    if (e != hipSuccess) return hip_fail(e, "segment scan launch");
    ssd::StateSrc src{initial_state, s.H * PN, Sbuf, p.nseg * s.H * PN, s.H * PN};
    e = ssd::launch_fwd(s, p.sw, p.seg_chunks, p.nseg, X, a, B, C, src, Y, final_state, hs);
    if (e != hipSuccess) return hip_fail(e, "MFMA forward launch");
    return ok();
}


// ---- backward plan ------------------------------------------------------------
// Workspace regions of the backward, in order.
enum BwdBuf {
    W_SFW, W_LAMFW,       // forward chunk-entering states and chunk log-decays
    W_SREV, W_LAMREV,     // the same for the time-reversed adjoint problem
    W_DYR, W_CR, W_BR, W_AR, W_DXR,   // reversed dY, C, B, shifted a; reversed dX
    W_BEXP, W_AEXP, W_S0T, W_DCH,     // dC pass: B per head, a per sub-head, S0^T, output
    W_CREXP, W_XR, W_AREXP, W_DSFT, W_DBH,   // dB pass (reversed)
    W_INNER,              // workspace of the dC / dB passes
    W_CBT,                // C B^T tiles of every chunk for the da kernel
    kBwdBufs
};

struct BwdPlan {
    ssd::FwdShape s;   // the layer
    ssd::FwdShape sr;  // the reversed problem: seqlen padded to whole chunks
    int64_t ns;        // the dB / dC passes split the state dimension into ns head-dims of 64
    bool xg;           // bf16, headdim 64: dB / dC read B, C, a and the chunk states in place
    bool f32;          // fp32 inputs: VALU kernels throughout
    int64_t es;        // element bytes of X, B, C and the gradients
    Plan pc, pb;       // plans of the dC and dB passes (otherwise)
    size_t off[kBwdBufs + 1];
};

ssd_status make_bwd_plan(const ssd_fwd_desc* d, BwdPlan* bp) {
    ssd_status st = check_desc(d, true);
    if (st != SSD_OK) return st;
    const ssd::FwdShape s = shape_of(d);
    bp->f32 = d->dtype == SSD_F32;
    bp->es = bp->f32 ? 4 : 2;
    if (bp->f32) {
        // fp32: the VALU forward for every pass and the VALU da
        if (!ssd::valu_fwd_supported(s) || (s.H * s.P) % 4 != 0 || s.N % 8 != 0)
            return fail(SSD_ERR_UNSUPPORTED,
                        "no fp32 backward for chunk=%lld headdim=%lld dstate=%lld (chunk <= 256, "
                        "headdim*dstate <= 16384, nheads*headdim a multiple of 4, dstate of 8)",
                        (long long)s.Q, (long long)s.P, (long long)s.N);
        if (d->algo == SSD_ALGO_MFMA)
            return fail(SSD_ERR_UNSUPPORTED, "the MFMA backward needs bf16 inputs");
    } else {
        if (d->algo == SSD_ALGO_VALU)
            return fail(SSD_ERR_UNSUPPORTED, "the bf16 backward has no VALU variant");
        if (!ssd::mfma_supported(s.Q, s.P, s.N) || !ssd::bwd_da_supported(s.Q, s.P, s.N))
            return fail(SSD_ERR_UNSUPPORTED,
                        "no backward kernels for chunk=%lld headdim=%lld dstate=%lld "
                        "(chunk in {64,128,256}, headdim in {32,64}, dstate in {64,128})",
                        (long long)s.Q, (long long)s.P, (long long)s.N);
    }
    // the chunk-state and dX passes launch up to batch*chunks*heads workgroups,
    // the exchanged-dimension passes up to batch*chunks*(heads+groups), the
    // paired chunk-state passes with the C B^T tiles up to
    // batch*chunks*(2/3 heads + 7 groups) (plus XCD padding), each of at most
    // kMfmaThreads threads
    if ((s.Bz * s.nc * (s.H + 8 * s.G) + 24) * kMfmaThreads >= ((int64_t)1 << 32) || s.nc > 0x7fffffff)
        return fail(SSD_ERR_UNSUPPORTED, "batch*chunks*heads too large for one launch");
    // the C B^T tile kernel launches batch * chunks * groups * ceil(T(T+1)/8)
    // workgroups of 256 threads (T = chunk / 32, at most 8)
    if (!bp->f32 && s.Bz * s.nc * s.G * 9 * 256 >= ((int64_t)1 << 32))
        return fail(SSD_ERR_UNSUPPORTED, "batch*chunks*groups too large for the C B^T tile kernel");
    // the copy kernels launch (row blocks of up to 256 threads) x steps blocks
    const int64_t row_items = s.H * (s.N > s.P ? s.N : s.P) * bp->es / 16;
    if (s.nc * s.Q * (((row_items + 255) / 256) * 256) >= ((int64_t)1 << 31))
        return fail(SSD_ERR_UNSUPPORTED, "seqlen*nheads too large for the backward's copy kernels");
    bp->s = s;
    bp->sr = s;
    bp->sr.L = s.nc * s.Q;
    bp->ns = bp->f32 ? 1 : s.N / 64;
    bp->xg = !bp->f32 && s.P == 64;
    // dC: the forward-time product with x in the role of B, dy in that of C and
    // B (split into 64-wide pieces, one per sub-head) in that of X; dB: the same
    // on reversed time with dy as B, x as C and C as X
    ssd_fwd_desc dc{s.Bz, s.L, s.H * bp->ns, s.N / bp->ns, s.P, s.H, s.Q, d->dtype,
                    SSD_ALGO_AUTO, 0};
    ssd_fwd_desc db = dc;
    db.seqlen = bp->sr.L;
    if (!bp->xg) {   // (the in-place exchanged-dimension passes need no plan of their own)
        st = make_plan(&dc, &bp->pc);
        if (st != SSD_OK) return st;
        st = make_plan(&db, &bp->pb);
        if (st != SSD_OK) return st;
    }
    const int64_t Bz = s.Bz, L = s.L, Lp = bp->sr.L, H = s.H, G = s.G, P = s.P, N = s.N;
    const int64_t nc = s.nc, PN = P * N, ns = bp->ns, es = bp->es;
    int64_t bytes[kBwdBufs] = {};
    if (Bz > 0 && L > 0) {
        bytes[W_SFW] = Bz * nc * H * PN * 4;
        bytes[W_LAMFW] = Bz * H * nc * 4;
        bytes[W_SREV] = bytes[W_SFW];
        bytes[W_LAMREV] = bytes[W_LAMFW];
        bytes[W_DYR] = Bz * Lp * H * P * es;
        bytes[W_CR] = Bz * Lp * G * N * es;
        bytes[W_BR] = bytes[W_CR];
        bytes[W_AR] = Bz * Lp * H * 4;
        bytes[W_DXR] = bytes[W_DYR];
        // per-head dC / dB contributions in fp32, summed over the group's heads
        // before the one rounding
        const int64_t eh = 4;
        bytes[W_DCH] = Bz * L * H * N * eh;
        bytes[W_XR] = bytes[W_DYR];
        bytes[W_DBH] = Bz * Lp * H * N * eh;
        if (!bp->xg) {
            bytes[W_BEXP] = Bz * L * H * N * es;
            bytes[W_AEXP] = Bz * L * H * ns * 4;
            bytes[W_S0T] = Bz * H * PN * 4;
            bytes[W_CREXP] = Bz * Lp * H * N * es;
            bytes[W_AREXP] = Bz * Lp * H * ns * 4;
            bytes[W_DSFT] = bytes[W_S0T];
            bytes[W_INNER] = (int64_t)(bp->pc.ws > bp->pb.ws ? bp->pc.ws : bp->pb.ws);
        }
        if (!bp->f32) bytes[W_CBT] = ssd::cb_tiles_bytes(s);
    }
    size_t o = 0;
    for (int i = 0; i < kBwdBufs; ++i) {
        bp->off[i] = o;
        o += (size_t)(((bytes[i] + 255) / 256) * 256);
    }
    bp->off[kBwdBufs] = o;
    return SSD_OK;
}

}  // namespace

namespace ssd {

ssd_status fwd_with_fixed_workspace(const ssd_fwd_desc* desc, const void* X, const float* a,
                                    const void* B, const void* C, const float* initial_state,
                                    void* Y, float* final_state, size_t ws_cap,
                                    hipError_t (*get_ws)(void**), void* stream) {
    Plan p;
    ssd_status st = make_plan(desc, &p, ws_cap);
    if (st != SSD_OK) return st;
    st = check_fwd_io(p, X, a, B, C, initial_state, Y, final_state);
    if (st != SSD_OK) return st;
    void* ws = nullptr;
    if (p.ws > 0) {
        const hipError_t e = get_ws(&ws);
        if (e != hipSuccess) return hip_fail(e, "fixed workspace address");
    }
    return run_fwd(p, X, a, B, C, initial_state, Y, final_state, ws, reinterpret_cast<hipStream_t>(stream));
}

}  // namespace ssd

extern "C" {

const char* ssd_status_str(ssd_status s) {
    switch (s) {
    case SSD_OK: return "SSD_OK: success";
    case SSD_ERR_NULL: return "SSD_ERR_NULL: a required pointer is NULL";
    case SSD_ERR_SHAPE: return "SSD_ERR_SHAPE: invalid sizes";
    case SSD_ERR_DTYPE: return "SSD_ERR_DTYPE: unknown dtype";
    case SSD_ERR_ALIGN: return "SSD_ERR_ALIGN: misaligned buffer";
    case SSD_ERR_UNSUPPORTED: return "SSD_ERR_UNSUPPORTED: no kernel compiled for this shape";
    case SSD_ERR_WORKSPACE: return "SSD_ERR_WORKSPACE: workspace missing or too small";
    case SSD_ERR_HIP: return "SSD_ERR_HIP: HIP runtime error";
    case SSD_ERR_ALIAS: return "SSD_ERR_ALIAS: an output overlaps an input";
    }
    return "unknown ssd_status";
}

const char* ssd_last_error(void) { return g_err; }

int32_t ssd_version(void) { return 100; }

ssd_status ssd_fwd_workspace_bytes(const ssd_fwd_desc* desc, size_t* bytes) {
    if (!bytes) return fail(SSD_ERR_NULL, "bytes is NULL");
    Plan p;
    ssd_status st = make_plan(desc, &p);
    if (st != SSD_OK) return st;
    *bytes = p.ws;
    return ok();
}

ssd_status ssd_fwd_plan(const ssd_fwd_desc* desc, int32_t* algo, int64_t* seg_chunks, int64_t* nseg,
                        int32_t* wg_units) {
    Plan p;
    ssd_status st = make_plan(desc, &p);
    if (st != SSD_OK) return st;
    if (algo) *algo = p.algo;
    if (seg_chunks) *seg_chunks = p.seg_chunks;
    if (nseg) *nseg = p.nseg;
    if (wg_units) *wg_units = p.sw;
    return ok();
}

ssd_status ssd_chunk_scan_fwd(const ssd_fwd_desc* desc, const void* X, const float* a,
                              const void* B, const void* C, const float* initial_state,
                              void* Y, float* final_state, void* workspace,
                              size_t workspace_bytes, void* stream) {
    Plan p;
    ssd_status st = make_plan(desc, &p);
    if (st != SSD_OK) return st;
    st = check_fwd_io(p, X, a, B, C, initial_state, Y, final_state);
    if (st != SSD_OK) return st;
    if (p.ws > 0) {
        if (!workspace || workspace_bytes < p.ws)
            return fail(SSD_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu%s)", p.ws,
                        workspace_bytes, workspace ? "" : ", NULL");
        if (!aligned(workspace, 16)) return fail(SSD_ERR_ALIGN, "workspace is not 16-byte aligned");
        const int64_t es = p.bf16 ? 2 : 4;
        const ssd::FwdShape& s = p.s;
        const Range w = rng("workspace", workspace, (int64_t)p.ws);
        const Range others[] = {
            rng("X", X, s.Bz * s.L * s.H * s.P * es), rng("a", a, s.Bz * s.L * s.H * 4),
            rng("B", B, s.Bz * s.L * s.G * s.N * es), rng("C", C, s.Bz * s.L * s.G * s.N * es),
            rng("Y", Y, s.Bz * s.L * s.H * s.P * es),
            rng("initial_state", initial_state, initial_state ? s.Bz * s.H * s.P * s.N * 4 : 0),
            rng("final_state", final_state, final_state ? s.Bz * s.H * s.P * s.N * 4 : 0)};
        for (const Range& o : others)
            if (overlap(w, o)) return fail(SSD_ERR_ALIAS, "workspace overlaps %s", o.name);
    }
    return run_fwd(p, X, a, B, C, initial_state, Y, final_state, workspace,
                   reinterpret_cast<hipStream_t>(stream));
}

ssd_status ssd_step(const ssd_step_desc* d, float* state, const void* x, const float* a,
                    const void* B, const void* C, void* y, void* stream) {
    if (!d) return fail(SSD_ERR_NULL, "desc is NULL");
    if (d->batch < 0 || d->nheads < 1 || d->headdim < 1 || d->dstate < 1 || d->ngroups < 1)
        return fail(SSD_ERR_SHAPE, "sizes must be batch>=0 and nheads,headdim,dstate,ngroups>=1");
    if (d->nheads % d->ngroups != 0)
        return fail(SSD_ERR_SHAPE, "nheads (%lld) must be a multiple of ngroups (%lld)",
                    (long long)d->nheads, (long long)d->ngroups);
    if (d->dtype != SSD_F32 && d->dtype != SSD_BF16)
        return fail(SSD_ERR_DTYPE, "dtype %d is not SSD_F32 or SSD_BF16", (int)d->dtype);
    if (d->reserved != 0) return fail(SSD_ERR_SHAPE, "reserved must be 0");
    if (d->batch * d->nheads > ((int64_t)1 << 31) - 1 || d->headdim * d->dstate > (1 << 24))
        return fail(SSD_ERR_UNSUPPORTED, "sizes beyond the supported range");
    // every launch shape of the step kernels is at most one thread per 4 state
    // elements (at least one per row), and a launch holds < 2^32 threads
    if (d->batch * d->nheads * d->headdim * (d->dstate >= 4 ? d->dstate / 4 : 1) >= ((int64_t)1 << 32))
        return fail(SSD_ERR_UNSUPPORTED, "batch*nheads*headdim*dstate too large for one launch");
    if (d->batch == 0) return ok();
    if (!state || !x || !a || !B || !C || !y) return fail(SSD_ERR_NULL, "state, x, a, B, C and y are required");
    const int64_t es = d->dtype == SSD_BF16 ? 2 : 4;
    if (!aligned(state, 16) || !aligned(B, 8) || !aligned(C, 8))
        return fail(SSD_ERR_ALIGN, "state must be 16-byte and B, C 8-byte aligned");
    if (!aligned(x, es) || !aligned(y, es) || !aligned(a, 4))
        return fail(SSD_ERR_ALIGN, "x, y, a must be element aligned");
    const int64_t BH = d->batch * d->nheads;
    const Range ins[] = {rng("state", state, BH * d->headdim * d->dstate * 4),
                         rng("x", x, BH * d->headdim * es), rng("a", a, BH * 4),
                         rng("B", B, d->batch * d->ngroups * d->dstate * es),
                         rng("C", C, d->batch * d->ngroups * d->dstate * es)};
    const Range yo = rng("y", y, BH * d->headdim * es);
    for (const Range& i : ins)
        if (overlap(yo, i)) return fail(SSD_ERR_ALIAS, "y overlaps %s", i.name);
    for (int i = 1; i < 5; ++i)
        if (overlap(ins[0], ins[i])) return fail(SSD_ERR_ALIAS, "state overlaps %s", ins[i].name);
    hipError_t e = ssd::launch_step(d->batch, d->nheads, d->headdim, d->dstate, d->ngroups,
                                    d->dtype == SSD_BF16, state, x, a, B, C, y,
                                    reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "decode step launch");
    return ok();
}

ssd_status ssd_stream_rmw(float* data, int64_t n, float scale, int32_t per_thread, int32_t nontemporal,
                          void* stream) {
    if (n < 0 || n % 4 != 0) return fail(SSD_ERR_SHAPE, "n (%lld) must be a non-negative multiple of 4", (long long)n);
    if (per_thread != 1 && per_thread != 2 && per_thread != 4 && per_thread != 8)
        return fail(SSD_ERR_UNSUPPORTED, "per_thread must be 1, 2, 4 or 8");
    if (nontemporal != 0 && nontemporal != 1) return fail(SSD_ERR_SHAPE, "nontemporal must be 0 or 1");
    // one thread per float4 at most, and a launch holds < 2^32 threads
    if (n / 4 >= ((int64_t)1 << 32)) return fail(SSD_ERR_UNSUPPORTED, "n beyond the supported range");
    if (n == 0) return ok();
    if (!data) return fail(SSD_ERR_NULL, "data is NULL");
    if (!aligned(data, 16)) return fail(SSD_ERR_ALIGN, "data must be 16-byte aligned");
    const hipError_t e = ssd::launch_stream_rmw(data, n / 4, scale, per_thread, nontemporal != 0,
                                                reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "stream launch");
    return ok();
}

ssd_status ssd_chunk_cumsum(const ssd_fwd_desc* desc, const float* a, float* cs, float* lam,
                            void* stream) {
    ssd_status st = check_desc(desc, true);
    if (st != SSD_OK) return st;
    const ssd::FwdShape s = shape_of(desc);
    if (s.Bz == 0 || s.L == 0) return ok();
    if (!a || !cs || !lam) return fail(SSD_ERR_NULL, "a, cs and lam are required");
    if (!aligned(a, 4) || !aligned(cs, 4) || !aligned(lam, 4)) return fail(SSD_ERR_ALIGN, "misaligned");
    const Range ra = rng("a", a, s.Bz * s.L * s.H * 4);
    const Range rc = rng("cs", cs, s.Bz * s.H * s.nc * s.Q * 4), rl = rng("lam", lam, s.Bz * s.H * s.nc * 4);
    if (overlap(ra, rc) || overlap(ra, rl) || overlap(rc, rl)) return fail(SSD_ERR_ALIAS, "outputs overlap");
    hipError_t e = ssd::launch_chunk_cumsum(s, a, cs, lam, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "cumsum launch");
    return ok();
}

ssd_status ssd_chunk_state(const ssd_fwd_desc* desc, const void* X, const float* a, const void* B,
                           float* dstates, void* stream) {
    ssd_fwd_desc d1;
    if (!desc) return fail(SSD_ERR_NULL, "desc is NULL");
    d1 = *desc;
    d1.algo = SSD_ALGO_MFMA;
    if (d1.seg_chunks < 1) d1.seg_chunks = 1;
    Plan p;
    ssd_status st = make_plan(&d1, &p);
    if (st != SSD_OK) return st;
    const ssd::FwdShape& s = p.s;
    if (s.Bz == 0 || s.L == 0) return ok();
    if (!X || !a || !B || !dstates) return fail(SSD_ERR_NULL, "X, a, B and dstates are required");
    if (!aligned(X, 16) || !aligned(B, 16) || !aligned(dstates, 16) || !aligned(a, 4))
        return fail(SSD_ERR_ALIGN, "misaligned buffer");
    const Range out = rng("dstates", dstates, s.Bz * p.nseg * s.H * s.P * s.N * 4);
    const Range ins[] = {rng("X", X, s.Bz * s.L * s.H * s.P * 2), rng("a", a, s.Bz * s.L * s.H * 4),
                         rng("B", B, s.Bz * s.L * s.G * s.N * 2)};
    for (const Range& i : ins)
        if (overlap(out, i)) return fail(SSD_ERR_ALIAS, "dstates overlaps %s", i.name);
    hipError_t e = ssd::launch_mfma_state(s, p.seg_chunks, p.nseg, p.nseg, X, a, B, dstates, nullptr,
                                          reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "chunk state launch");
    return ok();
}

ssd_status ssd_state_passing(const ssd_fwd_desc* desc, const float* dstates, const float* lam,
                             const float* initial_state, float* states_in, float* final_state,
                             void* stream) {
    ssd_status st = check_desc(desc, false);
    if (st != SSD_OK) return st;
    const ssd::FwdShape s = shape_of(desc);
    if (s.Bz == 0) return ok();
    const int64_t PN = s.P * s.N;
    const int64_t k = desc->seg_chunks > 1 ? desc->seg_chunks : 1;
    const int64_t nu = (s.nc + k - 1) / k;   // units of k chunks
    if (s.L == 0) {
        if (final_state) {
            if (!aligned(final_state, 16)) return fail(SSD_ERR_ALIGN, "final_state misaligned");
            hipError_t e = initial_state
                ? ssd::launch_copy_f32(final_state, initial_state, s.Bz * s.H * PN, reinterpret_cast<hipStream_t>(stream))
                : ssd::launch_fill_zero(final_state, s.Bz * s.H * PN, reinterpret_cast<hipStream_t>(stream));
            if (e != hipSuccess) return hip_fail(e, "empty state passing");
        }
        return ok();
    }
    if (!dstates || !lam || !states_in) return fail(SSD_ERR_NULL, "dstates, lam and states_in are required");
    const void* v16[] = {dstates, initial_state, states_in, final_state};
    for (const void* q : v16)
        if (q && !aligned(q, 16)) return fail(SSD_ERR_ALIGN, "state buffers must be 16-byte aligned");
    if (!aligned(lam, 4)) return fail(SSD_ERR_ALIGN, "lam misaligned");
    const int64_t nst = s.Bz * nu * s.H * PN * 4;
    const Range rd = rng("dstates", dstates, nst), ro = rng("states_in", states_in, nst);
    if (overlap(rd, ro) && dstates != states_in)
        return fail(SSD_ERR_ALIAS, "states_in overlaps dstates without being identical");
    const Range rl = rng("lam", lam, s.Bz * s.H * nu * 4);
    const Range ri = rng("initial_state", initial_state, initial_state ? s.Bz * s.H * PN * 4 : 0);
    const Range rf = rng("final_state", final_state, final_state ? s.Bz * s.H * PN * 4 : 0);
    if (overlap(ro, rl) || overlap(ro, ri) || overlap(rf, rl) || overlap(rf, ri) || overlap(rf, rd) ||
        overlap(rf, ro))
        return fail(SSD_ERR_ALIAS, "an output overlaps an input");
    hipError_t e = ssd::launch_state_scan(s, nu, nu, dstates, lam, s.H * nu, nu,
                                          initial_state, states_in, 0, final_state, s.H * PN,
                                          reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "state passing launch");
    return ok();
}

ssd_status ssd_chunk_scan(const ssd_fwd_desc* desc, const void* X, const float* a, const void* B,
                          const void* C, const float* states_in, void* Y, void* stream) {
    if (!desc) return fail(SSD_ERR_NULL, "desc is NULL");
    ssd_fwd_desc d1 = *desc;
    d1.algo = SSD_ALGO_MFMA;
    if (d1.seg_chunks < 1) d1.seg_chunks = 1;
    Plan p;
    ssd_status st = make_plan(&d1, &p);
    if (st != SSD_OK) return st;
    const ssd::FwdShape& s = p.s;
    if (s.Bz == 0 || s.L == 0) return ok();
    st = check_fwd_io(p, X, a, B, C, nullptr, Y, nullptr);
    if (st != SSD_OK) return st;
    if (states_in) {
        if (!aligned(states_in, 16)) return fail(SSD_ERR_ALIGN, "states_in misaligned");
        const Range rs = rng("states_in", states_in, s.Bz * p.nseg * s.H * s.P * s.N * 4);
        if (overlap(rs, rng("Y", Y, s.Bz * s.L * s.H * s.P * 2))) return fail(SSD_ERR_ALIAS, "Y overlaps states_in");
    }
    const int64_t PN = s.P * s.N;
    ssd::StateSrc src{states_in, p.nseg * s.H * PN, states_in, p.nseg * s.H * PN, s.H * PN};
    hipError_t e = ssd::launch_fwd(s, p.sw, p.seg_chunks, p.nseg, X, a, B, C, src, Y, nullptr,
                                   reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "chunk scan launch");
    return ok();
}


ssd_status ssd_bwd_workspace_bytes(const ssd_fwd_desc* desc, size_t* bytes) {
    if (!bytes) return fail(SSD_ERR_NULL, "bytes is NULL");
    BwdPlan bp;
    ssd_status st = make_bwd_plan(desc, &bp);
    if (st != SSD_OK) return st;
    *bytes = bp.off[kBwdBufs];
    return ok();
}

ssd_status ssd_chunk_scan_bwd(const ssd_fwd_desc* desc, const void* X, const float* a,
                              const void* B, const void* C, const float* initial_state,
                              const void* dY, const float* dfinal_state, void* dX, float* da,
                              void* dB, void* dC, float* dinitial_state, void* workspace,
                              size_t workspace_bytes, void* stream) {
    BwdPlan bp;
    ssd_status st = make_bwd_plan(desc, &bp);
    if (st != SSD_OK) return st;
    const ssd::FwdShape& s = bp.s;
    const int64_t Bz = s.Bz, L = s.L, Lp = bp.sr.L, H = s.H, G = s.G, P = s.P, N = s.N;
    const int64_t nc = s.nc, PN = P * N, ns = bp.ns, es = bp.es;
    const size_t need = bp.off[kBwdBufs];
    if (Bz == 0) return ok();
    if (L > 0 && (!X || !a || !B || !C || !dY || !dX || !da || !dB || !dC))
        return fail(SSD_ERR_NULL, "X, a, B, C, dY, dX, da, dB and dC are required");
    const void* v16[] = {X, B, C, dY, dX, dB, dC, initial_state, dfinal_state, dinitial_state, workspace};
    const char* n16[] = {"X", "B", "C", "dY", "dX", "dB", "dC", "initial_state", "dfinal_state",
                         "dinitial_state", "workspace"};
    for (int i = 0; i < 11; ++i)
        if (v16[i] && !aligned(v16[i], 16)) return fail(SSD_ERR_ALIGN, "%s is not 16-byte aligned", n16[i]);
    if ((a && !aligned(a, 4)) || (da && !aligned(da, 4))) return fail(SSD_ERR_ALIGN, "a / da misaligned");
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(SSD_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu%s)", need, workspace_bytes,
                    workspace ? "" : ", NULL");
    const int64_t nX = Bz * L * H * P * es, nBC = Bz * L * G * N * es, nA = Bz * L * H * 4, nS = Bz * H * PN * 4;
    const Range ins[] = {rng("X", X, nX), rng("a", a, nA), rng("B", B, nBC), rng("C", C, nBC),
                         rng("initial_state", initial_state, initial_state ? nS : 0),
                         rng("dY", dY, nX), rng("dfinal_state", dfinal_state, dfinal_state ? nS : 0)};
    const Range outs[] = {rng("dX", dX, nX), rng("da", da, nA), rng("dB", dB, nBC), rng("dC", dC, nBC),
                          rng("dinitial_state", dinitial_state, dinitial_state ? nS : 0),
                          rng("workspace", workspace, need > 0 ? (int64_t)need : 0)};
    for (int i = 0; i < 6; ++i) {
        for (const Range& r : ins)
            if (overlap(outs[i], r)) return fail(SSD_ERR_ALIAS, "%s overlaps input %s", outs[i].name, r.name);
        for (int j = i + 1; j < 6; ++j)
            if (overlap(outs[i], outs[j])) return fail(SSD_ERR_ALIAS, "%s overlaps %s", outs[i].name, outs[j].name);
    }
    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    if (L == 0) {   // S_fin = S0: the adjoint passes straight through
        if (dinitial_state) {
            e = dfinal_state ? ssd::launch_copy_f32(dinitial_state, dfinal_state, Bz * H * PN, hs)
                             : ssd::launch_fill_zero(dinitial_state, Bz * H * PN, hs);
            if (e != hipSuccess) return hip_fail(e, "empty-sequence state gradient");
        }
        return ok();
    }
    char* ws = static_cast<char*>(workspace);
    auto F = [&](int i) { return reinterpret_cast<float*>(ws + bp.off[i]); };
    auto V = [&](int i) { return static_cast<void*>(ws + bp.off[i]); };
#define SSD_TRY(expr, what)                                  \
    do {                                                     \
        e = (expr);                                          \
        if (e != hipSuccess) return hip_fail(e, what);       \
    } while (0)
    // The bf16 plan reads the time-reversed problem in place when the sequence
    // is whole chunks (no padding) and the exchanged-dimension products run on
    // the MFMA kernel; otherwise its operands are copied out reversed.
    const bool rin = !bp.f32 && bp.xg && Lp == L && L % 64 == 0;
    const void* dYr = rin ? dY : V(W_DYR);
    const void* Cr = rin ? C : V(W_CR);
    const void* Br = rin ? B : V(W_BR);
    const float* ar = rin ? a : F(W_AR);
    if (bp.f32) {
        // fp32: the VALU forward gives the chunk states (and, on the reversed
        // problem, dX, G_0 and the adjoint's chunk states in one pass); the
        // rest follows the bf16 path's plan with VALU kernels
        SSD_TRY(ssd::launch_valu_fwd(s, false, X, a, B, C, initial_state, nullptr, nullptr, hs, F(W_SFW)),
                "bwd: chunk states");
        SSD_TRY(ssd::launch_remap_rows(V(W_DYR), dY, Bz, Lp, L, Lp - 1, -1, H * P * es, hs), "bwd: reverse dY");
        SSD_TRY(ssd::launch_remap_rows(V(W_CR), C, Bz, Lp, L, Lp - 1, -1, G * N * es, hs), "bwd: reverse C");
        SSD_TRY(ssd::launch_remap_rows(V(W_BR), B, Bz, Lp, L, Lp - 1, -1, G * N * es, hs), "bwd: reverse B");
        SSD_TRY(ssd::launch_remap_a(F(W_AR), a, Bz, Lp, L, Lp, -1, H, 1, hs), "bwd: reverse a");
        SSD_TRY(ssd::launch_valu_fwd(bp.sr, false, V(W_DYR), F(W_AR), V(W_CR), V(W_BR), dfinal_state,
                                     V(W_DXR), dinitial_state, hs, F(W_SREV)), "bwd: dX pass");
        SSD_TRY(ssd::launch_remap_rows(dX, V(W_DXR), Bz, L, Lp, Lp - 1, -1, H * P * es, hs), "bwd: dX order");
        if (dinitial_state)
            SSD_TRY(ssd::launch_scale_state_by_a0(dinitial_state, a, Bz, L, H, PN, hs), "bwd: dS0");
        SSD_TRY(ssd::launch_bwd_da_valu(s, (const float*)X, (const float*)dY, a, (const float*)B,
                                        (const float*)C, F(W_SFW), F(W_SREV), da, hs), "bwd: da");
    } else {
    // 1. the state entering every forward chunk, and 2. the adjoint's: the
    // adjoint recurrence runs backwards in time, on the reversed sequence
    // (padded at its start to whole chunks, so that reversed chunks coincide
    // with forward ones), with the decay of reversed step t' = a at forward
    // step Lp - t' (zero where that is past the end).  Its chunk states give
    // dX = G B, G being the state of the reversed problem (dy as X, C as B,
    // B as C, dS_fin as its initial state); its final state is G_0.  A
    // sequence of whole chunks needs no padding, and the kernels read (and
    // write) the reversed problem in place, both state passes in one launch;
    // otherwise it is copied out reversed.
    if (rin) {
        const ssd::StatePass pf{X, a, B, F(W_SFW), F(W_LAMFW), 0};
        const ssd::StatePass pr{dYr, ar, Cr, F(W_SREV), F(W_LAMREV), 1};
        SSD_TRY(ssd::launch_mfma_state_pair(s, 1, nc - 1, nc, pf, pr, hs), "bwd: chunk states");
    } else {
        SSD_TRY(ssd::launch_mfma_state(s, 1, nc - 1, nc, X, a, B, F(W_SFW), F(W_LAMFW), hs), "bwd: chunk states");
        SSD_TRY(ssd::launch_remap_rows(V(W_DYR), dY, Bz, Lp, L, Lp - 1, -1, H * P * es, hs), "bwd: reverse dY");
        SSD_TRY(ssd::launch_remap_rows(V(W_CR), C, Bz, Lp, L, Lp - 1, -1, G * N * es, hs), "bwd: reverse C");
        SSD_TRY(ssd::launch_remap_rows(V(W_BR), B, Bz, Lp, L, Lp - 1, -1, G * N * es, hs), "bwd: reverse B");
        SSD_TRY(ssd::launch_remap_a(F(W_AR), a, Bz, Lp, L, Lp, -1, H, 1, hs), "bwd: reverse a");
        SSD_TRY(ssd::launch_mfma_state(bp.sr, 1, nc - 1, nc, dYr, ar, Cr, F(W_SREV), F(W_LAMREV), hs, false),
                "bwd: adjoint chunk states");
    }
    {
        // both chunk-state scans (forward time from S0, reversed time from
        // dS_fin) in one launch; each writes its last chunk's entering state
        // into the last slot
        const ssd::ScanJob jf{F(W_SFW), F(W_LAMFW), H * nc, nc, initial_state, F(W_SFW), 0,
                              F(W_SFW) + (nc - 1) * H * PN, nc * H * PN};
        const ssd::ScanJob jr{F(W_SREV), F(W_LAMREV), H * nc, nc, dfinal_state, F(W_SREV), 0,
                              F(W_SREV) + (nc - 1) * H * PN, nc * H * PN};
        // with them, the da kernel's C B^T tiles (shared by each group's heads)
        const ssd::CbJob cbj{B, C, F(W_CBT), L, nc, (int)Bz, (int)G, (int)s.Q, (int)N};
        SSD_TRY(ssd::launch_state_scan_pair(s, nc - 1, nc, jf, jr, &cbj, hs), "bwd: state scans");
    }
    {
        // the fused forward pass on the reversed problem, one chunk per segment
        ssd::StateSrc src{dfinal_state, H * PN, F(W_SREV), nc * H * PN, H * PN};
        int64_t k1 = 1;
        int sw1 = 4;
        auto_plan(bp.sr, 1, 0, SIZE_MAX, &k1, &sw1);
        // its final state G_0 times e^{a_0} is d(initial state)
        SSD_TRY(ssd::launch_fwd(bp.sr, sw1, 1, nc, dYr, ar, Cr, Br, src, rin ? dX : V(W_DXR), dinitial_state,
                                hs, rin, a, L * H), "bwd: dX pass");
    }
    if (!rin)
        SSD_TRY(ssd::launch_remap_rows(dX, V(W_DXR), Bz, L, Lp, Lp - 1, -1, H * P * es, hs), "bwd: dX order");
    // 4. da from the chunk-local four-term form
    SSD_TRY(ssd::launch_bwd_da(s, X, dY, a, B, C, F(W_SFW), F(W_SREV), F(W_CBT), true, da, hs), "bwd: da");
    }
    if (bp.xg) {
        // 5-6. dC = S^T dy and dB = G^T x: the products with the state's two
        // dimensions exchanged (headdim 64 over the state's 64-wide column
        // pieces, state = the layer's headdim), entering each chunk from the
        // transposed chunk states already at hand: S for dC (forward time),
        // the adjoint for dB (reversed time)
        ssd::FwdShape sc = s;
        sc.H = H * ns; sc.P = 64; sc.N = P; sc.G = H;
        ssd::StateSrc srcc{initial_state, H * PN, F(W_SFW), nc * H * PN, H * PN};
        ssd::StateSrc srcb{dfinal_state, H * PN, F(W_SREV), nc * H * PN, H * PN};
        if (!rin)
            SSD_TRY(ssd::launch_remap_rows(V(W_XR), X, Bz, Lp, L, Lp - 1, -1, H * P * es, hs), "bwd: reverse X");
        // dC on forward time (B as X, x as B, dy as C); dB on reversed time
        // (C as X, dy as B, x as C): one launch.  Read in place, the reversed
        // problem also writes its per-head dB in forward order.
        const ssd::XgPass pc{B, a, X, dY, srcc, F(W_DCH), L, 0};
        const ssd::XgPass pb{Cr, ar, dYr, rin ? X : V(W_XR), srcb, F(W_DBH), Lp, rin ? 1 : 0};
        SSD_TRY(ssd::launch_mfma_out_xg_pair(sc, G, pc, pb, hs), "bwd: dC and dB passes");
        // both group sums in one launch (dB's per-head rows are in reversed
        // order when they were computed on a reversed copy)
        const ssd::GsJob gc{dC, V(W_DCH), L, 0, 1};
        const ssd::GsJob gb = rin ? ssd::GsJob{dB, V(W_DBH), L, 0, 1} : ssd::GsJob{dB, V(W_DBH), Lp, Lp - 1, -1};
        SSD_TRY(ssd::launch_group_sum_pair(gc, gb, Bz, L, H, G, N, false, true, hs), "bwd: dC and dB group sums");
        return ok();
    }
    // 5. dC = S^T dy: forward-time product, state dimensions exchanged
    SSD_TRY(ssd::launch_bcast_heads(V(W_BEXP), B, Bz, L, L, 0, 1, H, G, N * es, hs), "bwd: B per head");
    SSD_TRY(ssd::launch_remap_a(F(W_AEXP), a, Bz, L, L, 0, 1, H, ns, hs), "bwd: a per sub-head");
    if (initial_state)
        SSD_TRY(ssd::launch_state_transpose(F(W_S0T), initial_state, Bz * H, P, N, hs), "bwd: S0^T");
    st = run_fwd(bp.pc, V(W_BEXP), F(W_AEXP), X, dY, initial_state ? F(W_S0T) : nullptr, V(W_DCH),
                 nullptr, V(W_INNER), hs, true);
    if (st != SSD_OK) return st;
    SSD_TRY(ssd::launch_group_sum(dC, V(W_DCH), Bz, L, L, 0, 1, H, G, N, false, !bp.f32, hs), "bwd: dC group sum");
    // 6. dB = G^T x: reversed-time product, state dimensions exchanged
    SSD_TRY(ssd::launch_bcast_heads(V(W_CREXP), C, Bz, Lp, L, Lp - 1, -1, H, G, N * es, hs), "bwd: C per head");
    SSD_TRY(ssd::launch_remap_rows(V(W_XR), X, Bz, Lp, L, Lp - 1, -1, H * P * es, hs), "bwd: reverse X");
    SSD_TRY(ssd::launch_remap_a(F(W_AREXP), a, Bz, Lp, L, Lp, -1, H, ns, hs), "bwd: reverse a per sub-head");
    if (dfinal_state)
        SSD_TRY(ssd::launch_state_transpose(F(W_DSFT), dfinal_state, Bz * H, P, N, hs), "bwd: dS_fin^T");
    st = run_fwd(bp.pb, V(W_CREXP), F(W_AREXP), V(W_DYR), V(W_XR), dfinal_state ? F(W_DSFT) : nullptr,
                 V(W_DBH), nullptr, V(W_INNER), hs, true);
    if (st != SSD_OK) return st;
    SSD_TRY(ssd::launch_group_sum(dB, V(W_DBH), Bz, L, Lp, Lp - 1, -1, H, G, N, false, !bp.f32, hs), "bwd: dB group sum");
#undef SSD_TRY
    return ok();
}

ssd_status ssd_bwd_da_workspace_bytes(const ssd_fwd_desc* desc, size_t* bytes) {
    if (!bytes) return fail(SSD_ERR_NULL, "bytes is NULL");
    BwdPlan bp;
    ssd_status st = make_bwd_plan(desc, &bp);
    if (st != SSD_OK) return st;
    if (bp.f32) return fail(SSD_ERR_UNSUPPORTED, "the da stage entry point runs the bf16 MFMA kernel");
    *bytes = (size_t)ssd::cb_tiles_bytes(bp.s);
    return ok();
}

ssd_status ssd_bwd_da(const ssd_fwd_desc* desc, const void* X, const float* a, const void* B,
                      const void* C, const void* dY, const float* states_in,
                      const float* adjoint_in, float* da, void* workspace, size_t workspace_bytes,
                      void* stream) {
    BwdPlan bp;
    ssd_status st = make_bwd_plan(desc, &bp);
    if (st != SSD_OK) return st;
    if (bp.f32) return fail(SSD_ERR_UNSUPPORTED, "the da stage entry point runs the bf16 MFMA kernel");
    const ssd::FwdShape& s = bp.s;
    if (s.Bz == 0 || s.L == 0) return ok();
    if (!X || !a || !B || !C || !dY || !states_in || !adjoint_in || !da)
        return fail(SSD_ERR_NULL, "X, a, B, C, dY, states_in, adjoint_in and da are required");
    const void* v16[] = {X, B, C, dY, states_in, adjoint_in};
    for (const void* q : v16)
        if (!aligned(q, 16)) return fail(SSD_ERR_ALIGN, "X, B, C, dY and the state arrays must be 16-byte aligned");
    if (!aligned(a, 4) || !aligned(da, 4)) return fail(SSD_ERR_ALIGN, "a / da misaligned");
    const size_t need = (size_t)ssd::cb_tiles_bytes(s);
    if (!workspace || workspace_bytes < need)
        return fail(SSD_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu%s)", need, workspace_bytes,
                    workspace ? "" : ", NULL");
    if (!aligned(workspace, 16)) return fail(SSD_ERR_ALIGN, "workspace is not 16-byte aligned");
    const int64_t nX = s.Bz * s.L * s.H * s.P * 2, nBC = s.Bz * s.L * s.G * s.N * 2;
    const int64_t nSt = s.Bz * s.nc * s.H * s.P * s.N * 4, nA = s.Bz * s.L * s.H * 4;
    const Range ins[] = {rng("X", X, nX), rng("a", a, nA), rng("B", B, nBC), rng("C", C, nBC),
                         rng("dY", dY, nX), rng("states_in", states_in, nSt),
                         rng("adjoint_in", adjoint_in, nSt)};
    const Range outs[] = {rng("da", da, nA), rng("workspace", workspace, (int64_t)need)};
    for (const Range& o : outs)
        for (const Range& r : ins)
            if (overlap(o, r)) return fail(SSD_ERR_ALIAS, "%s overlaps %s", o.name, r.name);
    if (overlap(outs[0], outs[1])) return fail(SSD_ERR_ALIAS, "da overlaps workspace");
    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    float* cbt = static_cast<float*>(workspace);
    const ssd::CbJob cbj{B, C, cbt, s.L, s.nc, (int)s.Bz, (int)s.G, (int)s.Q, (int)s.N};
    hipError_t e = ssd::launch_cb_tiles(cbj, hs);
    if (e != hipSuccess) return hip_fail(e, "C B^T tiles launch");
    e = ssd::launch_bwd_da(s, X, dY, a, B, C, states_in, adjoint_in, cbt, false, da, hs);
    if (e != hipSuccess) return hip_fail(e, "da launch");
    return ok();
}

}  // extern "C"
