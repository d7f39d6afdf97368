// ssd_launch.hpp -- host-side launchers of the gfx950 kernels.  Arguments are
// already validated by the C ABI layer (api.cpp); these only enqueue.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

// State wavefronts of the forward MFMA kernel's workgroup (each carries one
// 32-wide head-dim slice of one head's state).
constexpr int kMfmaStateWaves = 6;

struct FwdShape {
    int64_t Bz, L, H, P, N, G, Q;
    int64_t nc;  // ceil(L / Q)
};

// Entering-state source for a segment: segment 0 reads first + b*first_bstride
// + h*P*N, segment s >= 1 reads Sin + b*bstride + s*sstride + h*P*N; a null
// pointer means zeros.
struct StateSrc {
    const float* first;
    int64_t first_bstride;
    const float* Sin;
    int64_t bstride, sstride;
};

// ---- VALU path (any dtype; fp32 arithmetic, exact segment sums) -------------
// Y may be null; S_chunks (optional) receives the state entering every chunk
// [Bz][nc][H][P][N]; y_f32 writes Y in fp32 for bf16 inputs.
hipError_t launch_valu_fwd(const FwdShape& s, bool bf16, const void* X, const float* a,
                           const void* B, const void* C, const float* S0, void* Y,
                           float* S_fin, hipStream_t st, float* S_chunks = nullptr,
                           bool y_f32 = false);
bool valu_fwd_supported(const FwdShape& s);

// ---- stage 1: in-chunk prefix sums ---------------------------------------------
hipError_t launch_chunk_cumsum(const FwdShape& s, const float* a, float* cs, float* lam,
                               hipStream_t st);

// ---- stage 4 / segment scan: S_{u+1} = exp(lam_u) S_u + D_u ---------------------
// D, Sout: [Bz][ustride][H][P*N] (units 0..nu-1 used);
// lam: lam[b*lam_bstride + h*lam_hstride + u];
// Sout[u] receives the state entering unit u for u >= u_write (units below
// u_write are not written); final (optional) the state after the last unit at
// final + b*final_bstride + h*P*N.  D may equal Sout.
hipError_t launch_state_scan(const FwdShape& s, int64_t nu, int64_t ustride, const float* D,
                             const float* lam,
                             int64_t lam_bstride, int64_t lam_hstride, const float* S0,
                             float* Sout, int64_t u_write, float* final_, int64_t final_bstride,
                             hipStream_t st);
// One scan of two independent state sequences of the same shape in one
// launch (the backward's forward-time and reversed-time chunk states).
struct ScanJob {
    const float* D;
    const float* lam;
    int64_t lam_bs, lam_hs;
    const float* S0;
    float* Sout;
    int64_t u_write;
    float* fin;
    int64_t fin_bs;
};
struct CbJob;
// cb (optional): the da kernel's C B^T tiles, formed by extra workgroups of the
// same launch
hipError_t launch_state_scan_pair(const FwdShape& s, int64_t nu, int64_t ustride, const ScanJob& j0,
                                  const ScanJob& j1, const CbJob* cb, hipStream_t st);

// ---- MFMA segmented path (bf16) ----------------------------------------------------
bool mfma_supported(int64_t Q, int64_t P, int64_t N);
// heads sharing B and C in one MFMA workgroup (kMfmaStateWaves / (P / 32))
int64_t mfma_heads_per_workgroup(int64_t P, int64_t N);
// Pass A: for segments [0, nseg_run) of seg_chunks chunks each, the state at
// the end of the segment starting from zero -> Sseg [Bz][nseg_total][H][P][N]
// (slot s), and the segment's total log-decay -> lamseg [Bz][H][nseg_total]
// (lamseg may be null).  rev: the time-reversed problem read in place, as
// for launch_fwd.
hipError_t launch_mfma_state(const FwdShape& s, int64_t seg_chunks, int64_t nseg_run,
                             int64_t nseg_total, const void* X, const float* a,
                             const void* B, float* Sseg, float* lamseg, hipStream_t st,
                             bool rev = false);
// Two state-only passes of the same shape in one launch (the backward's
// forward-time and reversed-time chunk states); each names its X, a and B
// arrays, its outputs and whether it reads the time-reversed problem in place.
struct StatePass {
    const void* X;
    const float* a;
    const void* B;
    float* Sseg;
    float* lamseg;
    int rev;
};
// The C B^T tiles of the backward's da kernel: for every (batch, chunk,
// group) the lower-triangle 32x32 fp32 tiles of C_I B_J^T (cb_tiles_bytes
// bytes at cbt; N and Q as the layer's).
struct CbJob {
    const void* B;
    const void* C;
    float* cbt;
    int64_t L, nc;
    int Bz, G, Q, N;
};
hipError_t launch_cb_tiles(const CbJob& j, hipStream_t st);
hipError_t launch_mfma_state_pair(const FwdShape& s, int64_t seg_chunks, int64_t nseg_run, int64_t nseg_total,
                                  const StatePass& p0, const StatePass& p1, hipStream_t st);
// The fused forward pass (kernels_fwd.hip): sw (4, 5 or 6) units -- 32-wide
// head-dim slices of heads -- per workgroup, for every segment starting from
// its entering state; writes Y and (last segment) the final state.  rev
// (s.L a multiple of 64, headdim 64): the time-reversed problem read and written in
// place -- step t is step s.L - 1 - t of X, B, C and Y, with the decay a at
// step s.L - t (none for t = 0).
// fin_a (optional): the final state is also multiplied by exp(fin_a[b *
// fin_a_bstride + h]) (the backward's d(initial state) = e^{a_0} G_0)
hipError_t launch_fwd(const FwdShape& s, int sw, int64_t seg_chunks, int64_t nseg, const void* X,
                      const float* a, const void* B, const void* C, StateSrc src, void* Y,
                      float* S_fin, hipStream_t st, bool rev = false, const float* fin_a = nullptr,
                      int64_t fin_a_bstride = 0);
int64_t fwd_workgroups(const FwdShape& s, int64_t nseg, int sw);
bool fwd_units_supported(int64_t P, int sw);

// The backward's exchanged-dimension products (headdim 64, state 64, one chunk
// per segment), two in one launch that share every size in s but the sequence
// length (p0.L, p1.L; each must have s.nc chunks) and the time order (rev: the
// time-reversed problem read and written in place, as for launch_fwd; L a
// multiple of 64): X [Bz][L][x_groups][(H/G)*64]
// bf16 shared by the H/G heads of a group (head hl reads columns hl*64 ..), a
// [Bz][L][G] (one decay per group), and the entering state of segment s read
// transposed from the [64][(H/G)*64] state of group grp in src (segment 0 from
// src.first, s >= 1 from src.Sin).  Y is fp32 [Bz][L][H][64].
struct XgPass {
    const void* X;
    const float* a;
    const void* B;
    const void* C;
    StateSrc src;
    float* Y;
    int64_t L;
    int rev;
};
hipError_t launch_mfma_out_xg_pair(const FwdShape& s, int64_t x_groups, const XgPass& p0, const XgPass& p1,
                                   hipStream_t st);

// ---- decode step ---------------------------------------------------------------------
hipError_t launch_step(int64_t Bz, int64_t H, int64_t P, int64_t N, int64_t G, bool bf16,
                       float* state, const void* x, const float* a, const void* B,
                       const void* C, void* y, hipStream_t st);

// ---- backward: operand rearrangements and da ------------------------------------
// Time maps: output step t of Lout reads source step s = off + dir * t of Lin;
// steps with s outside [0, Lin) are zero.
// rows of row_bytes (a multiple of 16): out[b][t][:] = in[b][s][:]
hipError_t launch_remap_rows(void* out, const void* in, int64_t Bz, int64_t Lout, int64_t Lin,
                             int64_t off, int64_t dir, int64_t row_bytes, hipStream_t st);
// B or C per head: out[b][t][h][:] = in[b][s][h / (H/G)][:] (rows of row_bytes, a
// multiple of 16)
hipError_t launch_bcast_heads(void* out, const void* in, int64_t Bz, int64_t Lout, int64_t Lin,
                              int64_t off, int64_t dir, int64_t H, int64_t G, int64_t row_bytes,
                              hipStream_t st);
// out[b][t][h * ns + k] = a[b][s][h]
hipError_t launch_remap_a(float* out, const float* a, int64_t Bz, int64_t Lout, int64_t Lin,
                          int64_t off, int64_t dir, int64_t H, int64_t ns, hipStream_t st);
// out[bh][n][p] = in[bh][p][n]
hipError_t launch_state_transpose(float* out, const float* in, int64_t BH, int64_t P, int64_t N,
                                  hipStream_t st);
// out[b][t][g][n] = sum over the group's heads of in[b][s][h][n] (fp32 sum, rounded
// once to out's type): in_bf16 / out_bf16 choose bf16 or fp32 elements (N times the
// element size a multiple of 16 bytes)
hipError_t launch_group_sum(void* out, const void* in, int64_t Bz, int64_t Lout, int64_t Lin,
                            int64_t off, int64_t dir, int64_t H, int64_t G, int64_t N, bool in_bf16,
                            bool out_bf16, hipStream_t st);
// Two group sums of the same output shape in one launch (the backward's dB
// and dC): each job names its output, its input, the input's length and its
// row map (input row off + dir * t for output row t).
struct GsJob {
    void* out;
    const void* in;
    int64_t Lin, off, dir;
};
hipError_t launch_group_sum_pair(const GsJob& j0, const GsJob& j1, int64_t Bz, int64_t Lout, int64_t H,
                                 int64_t G, int64_t N, bool in_bf16, bool out_bf16, hipStream_t st);
// state[b][h][:] *= exp(a[b][0][h])
hipError_t launch_scale_state_by_a0(float* state, const float* a, int64_t Bz, int64_t L,
                                    int64_t H, int64_t PN, hipStream_t st);
// da from the chunk-entering states Sin [Bz][nc][H][P][N] of the forward and
// the right adjoints Srev [Bz][nc][H][P][N]: the adjoint at the first step of
// chunk c + 1 (dS_fin for the last chunk) in slot c, or in slot nc - 1 - c
// when adj_reversed (the order of the time-reversed problem's chunk states).
bool bwd_da_supported(int64_t Q, int64_t P, int64_t N);
// the fp32 VALU da (fp32 inputs), Srev in the reversed problem's slot order
hipError_t launch_bwd_da_valu(const FwdShape& s, const float* X, const float* dY, const float* a,
                              const float* B, const float* C, const float* Sin, const float* Srev,
                              float* da, hipStream_t st);
// C B^T tiles of every (batch, chunk, group) for the da kernel:
// cb_tiles_bytes(s) bytes of fp32 at cbt.
int64_t cb_tiles_bytes(const FwdShape& s);
hipError_t launch_bwd_da(const FwdShape& s, const void* X, const void* dY, const float* a,
                         const void* B, const void* C, const float* Sin, const float* Srev,
                         const float* cbt, bool adj_reversed, float* da, hipStream_t st);

// The forward of the C ABI with a fixed workspace region of ws_cap bytes
// (api.cpp): plans within the cap, validates every argument on the host, then
// asks get_ws for the region's device address and enqueues.
}  // namespace ssd
#include "ssd.h"
namespace ssd {
ssd_status fwd_with_fixed_workspace(const ssd_fwd_desc* desc, const void* X, const float* a,
                                    const void* B, const void* C, const float* initial_state,
                                    void* Y, float* final_state, size_t ws_cap,
                                    hipError_t (*get_ws)(void**), void* stream);

// in-place data[i] *= s over n4 float4 (the decode step's HBM ceiling)
hipError_t launch_stream_rmw(float* data, int64_t n4, float s, int per_thread, bool nontemporal,
                             hipStream_t st);

// zero-fill (used for empty sequences: final state = 0)
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t st);
hipError_t launch_copy_f32(float* dst, const float* src, int64_t n, hipStream_t st);

}  // namespace ssd
