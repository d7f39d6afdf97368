/*
 * ssd.h -- C ABI of the MI355X (gfx950) SSD layer library (libssd.so).
 *
 * The layer evaluates, for every batch b and head h, the selective state
 * space model with a scalar decay per step -- a 1-semiseparable SSM, which
 * the CiteArk page of "Transformers are SSMs" (section "AI research summary")
 * says is computed by a block-decomposed matrix-multiplication algorithm,
 * and which the same page (section "what this means") identifies with
 * structured masked attention and constant-memory inference:
 *
 *     S_t = exp(a_t) * S_{t-1} + X_t (x) B_t        (S is P x N, S_{-1} = S0)
 *     Y_t = S_t C_t                                  (Y_t[p] = sum_n S_t[p][n] C_t[n])
 *
 * i.e. Y = (Lmask o (C B^T)) X with Lmask[t][s] = exp(a_{s+1} + ... + a_t)
 * for t >= s and 0 above the diagonal (the semiseparable matrix of the wiki
 * review's "Core concepts").  Head h reads B/C group g = h * ngroups / nheads.
 *
 * Data layout (dense, row-major, last index fastest):
 *   X, Y           [batch][seqlen][nheads][headdim]     dtype of the call
 *   a              [batch][seqlen][nheads]              float32
 *   B, C           [batch][seqlen][ngroups][dstate]     dtype of the call
 *   states         [batch][nheads][headdim][dstate]     float32
 *   per-chunk data [batch][nchunks][nheads][headdim][dstate] float32
 * nchunks = ceil(seqlen / chunk); the last chunk may be shorter.
 *
 * Ownership: the caller allocates every buffer (device memory) and the
 * workspace; the library never allocates, keeps no state between calls and
 * never synchronises.  Every call validates all arguments on the host before
 * touching the GPU; on any error nothing is enqueued and no output is
 * written.  Work is enqueued on `stream` (a hipStream_t passed as void*;
 * NULL = the null stream) and is complete only once that stream has been
 * synchronised.  Asynchronous device faults surface at that synchronisation,
 * not as a return code.  Values are not inspected: NaN/Inf propagate within
 * their (batch, head) slice and a_t > 0 is computed as written.
 * Calls are thread-safe; ssd_last_error() is per calling thread.
 */
#ifndef SSD_H
#define SSD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ssd_status {
    SSD_OK = 0,
    SSD_ERR_NULL = 1,        /* a required pointer is NULL                   */
    SSD_ERR_SHAPE = 2,       /* negative size, nheads % ngroups != 0, chunk<1 */
    SSD_ERR_DTYPE = 3,       /* dtype is not one of ssd_dtype                 */
    SSD_ERR_ALIGN = 4,       /* a buffer is not 16-byte aligned               */
    SSD_ERR_UNSUPPORTED = 5, /* valid shape outside the compiled kernels      */
    SSD_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than required       */
    SSD_ERR_HIP = 7,         /* a HIP launch failed (see ssd_last_error)      */
    SSD_ERR_ALIAS = 8        /* an output overlaps an input it must not       */
} ssd_status;

typedef enum ssd_dtype {
    SSD_F32 = 0,  /* float32 X, B, C, Y                                       */
    SSD_BF16 = 1  /* bfloat16 X, B, C, Y; accumulation is always float32;     */
                  /* Y is rounded to nearest even                             */
} ssd_dtype;

typedef enum ssd_algo {
    SSD_ALGO_AUTO = 0,    /* MFMA path when compiled for the shape, else VALU  */
    SSD_ALGO_VALU = 1,    /* per-(b,h) sequential VALU kernel, fp32 math, any  */
                          /* dtype; exact segment sums (the fp32 path)         */
    SSD_ALGO_MFMA = 2     /* bf16 MFMA segmented kernels only                  */
} ssd_algo;

/* Forward problem.  chunk is the block size Q of the decomposition: the
 * diagonal Q x Q blocks are evaluated in the quadratic (masked attention)
 * form and everything across blocks through the carried state.  The result
 * does not depend on chunk beyond rounding.  seg_chunks (MFMA path) is the
 * number of consecutive chunks one workgroup walks while carrying the state
 * in registers; 0 lets the library choose from the shape.  wg_units (MFMA
 * path) is the number of 32-wide head-dim slices of heads (units) one
 * workgroup of the fused forward pass carries, 4, 5 or 6; 0 lets the library
 * choose.  Neither changes the result beyond rounding order. */
typedef struct ssd_fwd_desc {
    int64_t batch, seqlen, nheads, headdim, dstate, ngroups, chunk;
    int32_t dtype;      /* ssd_dtype */
    int32_t algo;       /* ssd_algo  */
    int64_t seg_chunks; /* 0 = automatic */
    int32_t wg_units;   /* 0 = automatic, else 4, 5 or 6 */
    int32_t reserved;   /* must be 0 */
} ssd_fwd_desc;

typedef struct ssd_step_desc {
    int64_t batch, nheads, headdim, dstate, ngroups;
    int32_t dtype;      /* ssd_dtype of x, B, C, y */
    int32_t reserved;   /* must be 0 */
} ssd_step_desc;

/* Bytes of device workspace ssd_chunk_scan_fwd needs for *desc (0 is
 * possible).  Errors as for ssd_chunk_scan_fwd's validation. */
ssd_status ssd_fwd_workspace_bytes(const ssd_fwd_desc* desc, size_t* bytes);

/* The chunk/segment plan the library uses for *desc: *algo receives the
 * ssd_algo that runs, *seg_chunks the chunks per segment (MFMA path), *nseg
 * the number of segments and *wg_units the units per workgroup of the fused
 * pass (MFMA path; 0 otherwise).  Any output pointer may be NULL.  Host only. */
ssd_status ssd_fwd_plan(const ssd_fwd_desc* desc, int32_t* algo, int64_t* seg_chunks,
                        int64_t* nseg, int32_t* wg_units);

/* Full forward: the four stages (segment sums, intra-chunk masked product,
 * chunk states with the inter-chunk state scan, state-to-output) over the
 * whole sequence.  Reads X, a, B, C and the optional initial_state (NULL =
 * zero state); writes Y and, if final_state != NULL, the state after the
 * last step.  Y and final_state must not overlap any input.
 * workspace: device buffer of at least ssd_fwd_workspace_bytes() bytes
 * (may be NULL when that is 0); its contents on entry are ignored. */
ssd_status ssd_chunk_scan_fwd(const ssd_fwd_desc* desc, const void* X, const float* a,
                              const void* B, const void* C, const float* initial_state,
                              void* Y, float* final_state, void* workspace,
                              size_t workspace_bytes, void* stream);

/* ssd_chunk_scan_fwd for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same computation and arguments without the workspace.
 * The segmented plan's workspace is a device array inside the library, one
 * per GPU, of SSD_NOALLOC_SCRATCH_BYTES (held until the process ends).  The
 * automatic plan is restricted to plans whose workspace fits it (a single
 * segment needs none, so every shape the forward takes has one; for shapes
 * whose unrestricted plan needs more, the plan and so the rounding may differ
 * from ssd_chunk_scan_fwd's).  A plan fixed by desc->seg_chunks that needs
 * more is rejected with SSD_ERR_WORKSPACE.  Calls no allocating routine.
 * Calls that overlap in time on one GPU share that array and race: order
 * them on one stream (or synchronise between them). */
#define SSD_NOALLOC_SCRATCH_BYTES (64u << 20)
ssd_status ssd_chunk_scan_fwd_noalloc(const ssd_fwd_desc* desc, const void* X, const float* a,
                                      const void* B, const void* C, const float* initial_state,
                                      void* Y, float* final_state, void* stream);

/* Single-token recurrent decode step for every (b, h) (constant-memory
 * inference): state <- exp(a) * state + x (x) B, then y = state C.
 * state [batch][nheads][headdim][dstate] float32 is updated in place;
 * x, y [batch][nheads][headdim] and B, C [batch][ngroups][dstate] in the
 * call's dtype; a [batch][nheads] float32.  y must not overlap state or the
 * inputs. */
ssd_status ssd_step(const ssd_step_desc* desc, float* state, const void* x, const float* a,
                    const void* B, const void* C, void* y, void* stream);

/* The HBM ceiling ssd_step is measured against: data[i] *= scale in place
 * for i < n (n a multiple of 4; data fp32, 16-byte aligned, on the device),
 * the same read-modify-write stream as the decode step's state with no other
 * traffic.  per_thread in {1, 2, 4, 8} float4 per thread; nontemporal 1 uses
 * the nontemporal load/store hints of the decode kernel, 0 plain accesses.
 * n / 4 must be below 2^32.  Errors: SSD_ERR_SHAPE / SSD_ERR_UNSUPPORTED /
 * SSD_ERR_NULL / SSD_ERR_ALIGN before anything is enqueued, SSD_ERR_HIP if
 * the launch fails. */
ssd_status ssd_stream_rmw(float* data, int64_t n, float scale, int32_t per_thread, int32_t nontemporal,
                          void* stream);

/* ---- Backward (gradients of the full forward) ----
 *
 * For a scalar loss l with upstream gradients dY = dl/dY and (optional)
 * dfinal_state = dl/dS_fin, the adjoint of the recurrence above --
 * G_t = dl/dS_t = dY_t C_t^T + exp(a_{t+1}) G_{t+1}, G_{L-1} also receiving
 * dS_fin -- gives
 *     dX_t = G_t B_t,   dB_t = sum_{h in group} G_t^T X_t,
 *     dC_t = sum_{h in group} S_t^T dY_t,   da_t = exp(a_t) <G_t, S_{t-1}>,
 *     dinitial_state = exp(a_0) G_0
 * (the reverse-mode derivative of the 1-semiseparable product that the
 * CiteArk page of "Transformers are SSMs", section "AI research summary",
 * names; the page's mention of training optimisations is what it serves).
 * bf16 inputs: chunk in {64,128,256}, headdim in {32,64}, dstate in {64,128}
 * (MFMA kernels; desc->algo AUTO or MFMA).  fp32 inputs: every shape the fp32
 * forward takes with nheads*headdim a multiple of 4 and dstate a multiple of
 * 8 (VALU kernels in fp32; desc->algo AUTO or VALU).  seg_chunks is ignored.
 * Reads X, a, B, C, initial_state (NULL = zero) and dY, dfinal_state (NULL =
 * zero); writes dX, dB, dC (in the inputs' dtype; bf16 rounded once from fp32
 * sums, dB and dC after summing the heads' fp32 contributions), da (fp32)
 * and, if dinitial_state != NULL, that gradient (fp32).  No output may
 * overlap an input, another output or the workspace.  The workspace holds
 * the per-chunk forward states and the adjoint's per-chunk states, the
 * per-head dB and dC contributions in fp32, the chunks' C_i.B_j tiles of the
 * da stage and, when the sequence is not a whole number of chunks,
 * time-reversed copies of the operands (about
 * 2 * batch * nchunks * nheads * headdim * dstate * 4 bytes plus a few
 * sequence-sized arrays); its size comes from ssd_bwd_workspace_bytes
 * and its contents on entry are ignored.  Errors as for ssd_chunk_scan_fwd. */
ssd_status ssd_bwd_workspace_bytes(const ssd_fwd_desc* desc, size_t* bytes);
ssd_status ssd_chunk_scan_bwd(const ssd_fwd_desc* desc, const void* X, const float* a,
                              const void* B, const void* C, const float* initial_state,
                              const void* dY, const float* dfinal_state, void* dX, float* da,
                              void* dB, void* dC, float* dinitial_state, void* workspace,
                              size_t workspace_bytes, void* stream);

/* The backward's da stage on its own (the dominant kernel of the backward):
 * for each chunk c, with the state entering it states_in[b][c][h] and the
 * adjoint adjoint_in[b][c][h] = dl/dS_t at the first step t of chunk c + 1
 * (dfinal_state, or 0, for the last chunk), both fp32
 * [batch][nchunks][nheads][headdim][dstate], and R = exp(a_t) adjoint_in
 * (R = adjoint_in for the last chunk):
 *   da_t = sum_{i>=t>j} exp(cs_i - cs_j)(dY_i.X_j)(C_i.B_j)
 *        + sum_{i>=t} exp(cs_i) dY_i.(S_in C_i) + sum_{j<t} exp(Lam - cs_j) X_j.(R B_j)
 *        + exp(Lam) <R, S_in>
 * over the chunk's steps (cs the chunk's prefix sums of a, Lam its total).
 * This equals da of ssd_chunk_scan_bwd when the states are the true ones.
 * Shapes and supported sizes as for ssd_chunk_scan_bwd (bf16 only).  The
 * workspace (16-byte aligned, at least ssd_bwd_da_workspace_bytes bytes,
 * contents on entry ignored) receives the chunks' C_i.B_j tiles, which the
 * heads of a group share: batch * nchunks * ngroups * T(T+1)/2 * 4 KiB with
 * T = chunk / 32.  da must not overlap an input or the workspace. */
ssd_status ssd_bwd_da_workspace_bytes(const ssd_fwd_desc* desc, size_t* bytes);
ssd_status ssd_bwd_da(const ssd_fwd_desc* desc, const void* X, const float* a, const void* B,
                      const void* C, const void* dY, const float* states_in,
                      const float* adjoint_in, float* da, void* workspace, size_t workspace_bytes,
                      void* stream);

/* ---- Stage entry points (the same kernels' building blocks, exposed so
 * each stage can be checked and timed on its own).  bf16 MFMA path only,
 * except ssd_chunk_cumsum which takes any dtype descriptor.  Stages 3-5 work
 * on units of desc->seg_chunks consecutive chunks (0 or 1: one chunk per
 * unit; the last unit may be shorter): U = ceil(nchunks / units) units, the
 * grouping the full forward's segments use.  Per-unit arrays are indexed by
 * the unit u in place of the chunk c. ---- */

/* Stage 1, segment sums: cs[b][h][c][i] = a_{cQ} + ... + a_{cQ+i} (fp32
 * wavefront prefix sums; entries past a ragged end are 0) and
 * lam[b][h][c] = the chunk's total. */
ssd_status ssd_chunk_cumsum(const ssd_fwd_desc* desc, const float* a, float* cs, float* lam,
                            void* stream);

/* Stage 3, chunk states: dstates[b][u][h][p][n] =
 * sum_j exp(a_{j+1} + ... + a_{end of unit}) X_j[p] B_j[n] over the unit. */
ssd_status ssd_chunk_state(const ssd_fwd_desc* desc, const void* X, const float* a,
                           const void* B, float* dstates, void* stream);

/* Stage 4, inter-chunk state scan: states_in[b][0][h] = initial_state (or 0),
 * states_in[b][u+1][h] = exp(lam[b][h][u]) states_in[b][u][h] + dstates[b][u][h],
 * with lam[b][h][u] the unit's total log-decay (the sum of its chunks' lam);
 * final_state (optional) receives the state after the last unit.
 * states_in may alias dstates exactly (in-place scan). */
ssd_status ssd_state_passing(const ssd_fwd_desc* desc, const float* dstates, const float* lam,
                             const float* initial_state, float* states_in, float* final_state,
                             void* stream);

/* Stages 2 and 5, chunk output: Y = masked product inside the unit + exp(cs) *
 * (C states_in^T) per unit, written once, with states_in[b][u][h] the state
 * entering unit u.  states_in NULL means zero states (Y is then the part
 * from inside each unit alone). */
ssd_status ssd_chunk_scan(const ssd_fwd_desc* desc, const void* X, const float* a,
                          const void* B, const void* C, const float* states_in, void* Y,
                          void* stream);

/* Static description of a status code. */
const char* ssd_status_str(ssd_status s);
/* Detail of the calling thread's most recent error ("" if none). */
const char* ssd_last_error(void);
/* Library version, major * 10000 + minor * 100 + patch. */
int32_t ssd_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SSD_H */
