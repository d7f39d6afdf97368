/*
 * ssd_oracle.c -- plain fp64 CPU oracle for the SSD layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this file: only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg do.  It shares no code, header, table or
 * helper with the HIP library.
 *
 * What it computes.  The layer is a selective state space model whose
 * per-step transition is a scalar times the identity, i.e. a 1-semiseparable
 * SSM ("Transformers are SSMs", CiteArk page, section "AI research summary":
 * a block-decomposed matmul algorithm that computes 1-semiseparable selective
 * SSMs; same page, section "what this means": such SSMs are exactly structured
 * masked attention, with constant-memory inference).  The discretised linear
 * recurrence it instantiates is the one walked through on the Mamba paper
 * digest (lryc.cn page, section "State Space Models": discretise, then run a
 * linear recurrence).  Written out, per batch b and head h, with the state
 * stored transposed as S = h^T of shape (P, N):
 *
 *     S_t[p][n] = exp(a_t) * S_{t-1}[p][n] + X_t[p] * B_t[n]      (S_{-1} = S0)
 *     Y_t[p]    = sum_n C_t[n] * S_t[p][n]
 *
 * a_t decays the previous state, the current input enters undecayed and the
 * output reads the post-update state.  Head h reads B/C group g = h*G/H.
 *
 * Everything is fp64; inputs are passed already widened to double (an exact
 * conversion from fp32 or bf16).  libm exp(), no fast-math.
 *
 * Layouts (row-major, last index fastest):
 *   X, Y   [batch][seqlen][nheads][headdim]
 *   a      [batch][seqlen][nheads]
 *   B, C   [batch][seqlen][ngroups][dstate]
 *   states [batch][nheads][headdim][dstate]
 *
 * Parity pins for every function here live in tests/test_oracle.py.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int64_t batch, seqlen, nheads, headdim, dstate, ngroups;
} oracle_dims;

/* ------------------------------------------------------------------------ */
/* Sequential recurrence (the definition).                                   */
/* ------------------------------------------------------------------------ */

/* One (b, h) slice, walked in time order.  S is the (P, N) state, updated in
 * place; Y receives every output step. */
static void recurrence_slice(const oracle_dims* d, int64_t b, int64_t h,
                             const double* X, const double* a, const double* B,
                             const double* C, double* Y, double* S)
{
    const int64_t L = d->seqlen, H = d->nheads, P = d->headdim, N = d->dstate;
    const int64_t G = d->ngroups;
    const int64_t g = h * G / H;
    for (int64_t t = 0; t < L; ++t) {
        const double decay = exp(a[(b * L + t) * H + h]);
        const double* x = X + ((b * L + t) * H + h) * P;
        const double* Bt = B + ((b * L + t) * G + g) * N;
        const double* Ct = C + ((b * L + t) * G + g) * N;
        double* y = Y + ((b * L + t) * H + h) * P;
        for (int64_t p = 0; p < P; ++p) {
            double* row = S + p * N;
            double acc = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                row[n] = decay * row[n] + x[p] * Bt[n];
                acc += Ct[n] * row[n];
            }
            y[p] = acc;
        }
    }
}

typedef struct {
    const oracle_dims* d;
    const double *X, *a, *B, *C, *S0;
    double *Y, *S_fin;
    int64_t first, step;
} fwd_job;

static void* fwd_worker(void* arg)
{
    fwd_job* j = (fwd_job*)arg;
    const oracle_dims* d = j->d;
    const int64_t PN = d->headdim * d->dstate;
    double* S = (double*)malloc((size_t)PN * sizeof(double));
    for (int64_t bh = j->first; bh < d->batch * d->nheads; bh += j->step) {
        const int64_t b = bh / d->nheads, h = bh % d->nheads;
        if (j->S0) memcpy(S, j->S0 + bh * PN, (size_t)PN * sizeof(double));
        else memset(S, 0, (size_t)PN * sizeof(double));
        recurrence_slice(d, b, h, j->X, j->a, j->B, j->C, j->Y, S);
        if (j->S_fin) memcpy(j->S_fin + bh * PN, S, (size_t)PN * sizeof(double));
    }
    free(S);
    return NULL;
}

/* Forward over the whole sequence.  S0 (initial state) and S_fin may be NULL
 * (NULL S0 means a zero initial state).  The (b, h) slices are independent,
 * so they are spread over nthreads POSIX threads; each slice is sequential. */
int oracle_fwd(const oracle_dims* d, const double* X, const double* a,
               const double* B, const double* C, const double* S0, double* Y,
               double* S_fin, int nthreads)
{
    if (!d || !X || !a || !B || !C || !Y) return 1;
    if (d->ngroups <= 0 || d->nheads % d->ngroups != 0) return 2;
    if (nthreads < 1) nthreads = 1;
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
    fwd_job* jobs = (fwd_job*)malloc(sizeof(fwd_job) * (size_t)nthreads);
    for (int i = 0; i < nthreads; ++i) {
        fwd_job j = {d, X, a, B, C, S0, Y, S_fin, i, nthreads};
        jobs[i] = j;
        if (nthreads == 1) fwd_worker(&jobs[i]);
        else pthread_create(&th[i], NULL, fwd_worker, &jobs[i]);
    }
    if (nthreads > 1)
        for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
    free(th);
    free(jobs);
    return 0;
}

/* One recurrent step for every (b, h): the same update as one iteration of
 * the forward loop, applied to a caller-held state (the constant-memory
 * inference mode).  Layouts: state [batch][nheads][P][N] (in/out),
 * x, y [batch][nheads][P], a [batch][nheads], B, C [batch][ngroups][N]. */
int oracle_step(const oracle_dims* d, double* state, const double* x,
                const double* a, const double* B, const double* C, double* y)
{
    if (!d || !state || !x || !a || !B || !C || !y) return 1;
    if (d->ngroups <= 0 || d->nheads % d->ngroups != 0) return 2;
    const int64_t H = d->nheads, P = d->headdim, N = d->dstate, G = d->ngroups;
    for (int64_t b = 0; b < d->batch; ++b)
        for (int64_t h = 0; h < H; ++h) {
            const int64_t g = h * G / H;
            const double decay = exp(a[b * H + h]);
            const double* Bt = B + (b * G + g) * N;
            const double* Ct = C + (b * G + g) * N;
            for (int64_t p = 0; p < P; ++p) {
                double* row = state + ((b * H + h) * P + p) * N;
                const double xp = x[(b * H + h) * P + p];
                double acc = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    row[n] = decay * row[n] + xp * Bt[n];
                    acc += Ct[n] * row[n];
                }
                y[(b * H + h) * P + p] = acc;
            }
        }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Chunked four-stage form, fp64, exposing every intermediate.               */
/* ------------------------------------------------------------------------ */
/*
 * The same map evaluated through the block decomposition of the
 * semiseparable matrix M = L o (C B^T) (wiki review of the paper, section
 * "Core concepts": semiseparable matrices, structured masked attention and
 * the block-decomposition SSD algorithm).  The sequence is cut into chunks
 * of Q steps (the last may be shorter).  Within chunk c, with steps
 * indexed locally i = 0..Lc-1:
 *
 *   cs[i]      = a_0 + ... + a_i                      (inclusive, in-chunk)
 *   Lam        = cs[Lc-1]
 *   seg(i, j)  = a_{j+1} + ... + a_i  for i >= j      (summed directly)
 *   Ydiag[i]   = sum_{j<=i} exp(seg(i,j)) (C_i . B_j) X_j
 *   dS[p][n]   = sum_j exp(a_{j+1} + ... + a_{Lc-1}) X_j[p] B_j[n]
 *   S_in(0)    = S0 (or 0);  S_in(c+1) = exp(Lam_c) S_in(c) + dS_c
 *   Yoff[i][p] = exp(cs[i]) sum_n C_i[n] S_in(c)[p][n]
 *   Y          = Ydiag + Yoff;   S_fin = S_in(nc)
 *
 * Segment and suffix sums are accumulated term by term (never as
 * differences of prefix sums), so this form carries no cancellation.
 *
 * Output layouts (any pointer may be NULL to skip it):
 *   cs    [batch][nheads][nc][Q]   (entries past a ragged end are 0)
 *   lam   [batch][nheads][nc]
 *   dS    [batch][nc][nheads][P][N]
 *   S_in  [batch][nc][nheads][P][N]   state entering each chunk
 *   Ydiag, Yoff, Y  [batch][seqlen][nheads][P]
 *   S_fin [batch][nheads][P][N]
 */
int oracle_chunked_fwd(const oracle_dims* d, int64_t Q, const double* X,
                       const double* a, const double* B, const double* C,
                       const double* S0, double* cs_out, double* lam_out,
                       double* dS_out, double* Sin_out, double* Ydiag,
                       double* Yoff, double* Y, double* S_fin)
{
    if (!d || !X || !a || !B || !C || Q < 1) return 1;
    if (d->ngroups <= 0 || d->nheads % d->ngroups != 0) return 2;
    const int64_t Bz = d->batch, L = d->seqlen, H = d->nheads, P = d->headdim;
    const int64_t N = d->dstate, G = d->ngroups;
    const int64_t nc = (L + Q - 1) / Q;
    double* S = (double*)malloc((size_t)(P * N) * sizeof(double));
    double* dS = (double*)malloc((size_t)(P * N) * sizeof(double));
    double* cs = (double*)malloc((size_t)Q * sizeof(double));
    for (int64_t b = 0; b < Bz; ++b)
        for (int64_t h = 0; h < H; ++h) {
            const int64_t g = h * G / H;
            if (S0) memcpy(S, S0 + (b * H + h) * P * N, (size_t)(P * N) * sizeof(double));
            else memset(S, 0, (size_t)(P * N) * sizeof(double));
#define A_AT(t) a[(b * L + (t)) * H + h]
#define X_AT(t) (X + ((b * L + (t)) * H + h) * P)
#define B_AT(t) (B + ((b * L + (t)) * G + g) * N)
#define C_AT(t) (C + ((b * L + (t)) * G + g) * N)
            for (int64_t c = 0; c < nc; ++c) {
                const int64_t t0 = c * Q;
                const int64_t Lc = (L - t0 < Q) ? (L - t0) : Q;
                /* stage 1: in-chunk inclusive prefix sums and chunk total */
                double run = 0.0;
                for (int64_t i = 0; i < Q; ++i) {
                    if (i < Lc) run += A_AT(t0 + i);
                    cs[i] = (i < Lc) ? run : 0.0;
                }
                const double lam = cs[Lc - 1];
                if (cs_out) memcpy(cs_out + ((b * H + h) * nc + c) * Q, cs, (size_t)Q * sizeof(double));
                if (lam_out) lam_out[(b * H + h) * nc + c] = lam;
                /* state entering this chunk */
                if (Sin_out)
                    memcpy(Sin_out + ((b * nc + c) * H + h) * P * N, S, (size_t)(P * N) * sizeof(double));
                /* stage 2 (intra-chunk) and stage 5 (state to output) */
                for (int64_t i = 0; i < Lc; ++i) {
                    const double* Ci = C_AT(t0 + i);
                    double* yd = Ydiag ? Ydiag + ((b * L + t0 + i) * H + h) * P : NULL;
                    double* yo = Yoff ? Yoff + ((b * L + t0 + i) * H + h) * P : NULL;
                    double* yy = Y ? Y + ((b * L + t0 + i) * H + h) * P : NULL;
                    for (int64_t p = 0; p < P; ++p) {
                        double acc = 0.0, seg = 0.0;
                        for (int64_t j = i; j >= 0; --j) {
                            if (j < i) seg += A_AT(t0 + j + 1);
                            const double* Bj = B_AT(t0 + j);
                            double cb = 0.0;
                            for (int64_t n = 0; n < N; ++n) cb += Ci[n] * Bj[n];
                            acc += exp(seg) * cb * X_AT(t0 + j)[p];
                        }
                        double off = 0.0;
                        for (int64_t n = 0; n < N; ++n) off += Ci[n] * S[p * N + n];
                        off *= exp(cs[i]);
                        if (yd) yd[p] = acc;
                        if (yo) yo[p] = off;
                        if (yy) yy[p] = acc + off;
                    }
                }
                /* stage 3: chunk state, decays summed from the chunk end */
                memset(dS, 0, (size_t)(P * N) * sizeof(double));
                double suffix = 0.0;
                for (int64_t j = Lc - 1; j >= 0; --j) {
                    if (j < Lc - 1) suffix += A_AT(t0 + j + 1);
                    const double w = exp(suffix);
                    const double* xj = X_AT(t0 + j);
                    const double* Bj = B_AT(t0 + j);
                    for (int64_t p = 0; p < P; ++p)
                        for (int64_t n = 0; n < N; ++n) dS[p * N + n] += w * xj[p] * Bj[n];
                }
                if (dS_out)
                    memcpy(dS_out + ((b * nc + c) * H + h) * P * N, dS, (size_t)(P * N) * sizeof(double));
                /* stage 4: pass the state across the chunk boundary */
                const double e = exp(lam);
                for (int64_t k = 0; k < P * N; ++k) S[k] = e * S[k] + dS[k];
            }
            if (S_fin) memcpy(S_fin + (b * H + h) * P * N, S, (size_t)(P * N) * sizeof(double));
#undef A_AT
#undef X_AT
#undef B_AT
#undef C_AT
        }
    free(S);
    free(dS);
    free(cs);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Gradients: the adjoint of the recurrence (reverse-mode chain rule).       */
/* ------------------------------------------------------------------------ */
/*
 * For a scalar loss l with dY = dl/dY and dS_fin = dl/dS_fin (either may be
 * all zero), the adjoint state G_t = dl/dS_t of each (b, h) slice obeys, in
 * reverse time,
 *
 *   G_{L-1}  = dS_fin + dY_{L-1} (x) C_{L-1}
 *   G_t      = dY_t (x) C_t + exp(a_{t+1}) G_{t+1}
 *
 * (S_t feeds Y_t directly and S_{t+1} through the decay exp(a_{t+1})), and
 * each input's gradient is the chain rule through the one step that reads it:
 *
 *   dX_t[p]  = sum_n G_t[p][n] B_t[n]              (S_t = ... + X_t (x) B_t)
 *   dB_t[n] += sum_p G_t[p][n] X_t[p]              (summed over the group's heads)
 *   dC_t[n] += sum_p dY_t[p] S_t[p][n]             (Y_t = S_t C_t; group sum)
 *   da_t     = exp(a_t) sum_{p,n} G_t[p][n] S_{t-1}[p][n]
 *   dS0      = exp(a_0) G_0
 *
 * The reverse sweep needs the forward states S_t.  They are recomputed one
 * segment of K steps at a time from checkpoints stored every K steps by a
 * forward sweep, so memory stays at (L/K + K) states per slice; the arithmetic
 * is exactly the forward recurrence's, so the recomputed states are the
 * forward's bit for bit.
 *
 * Layouts as above; dX like X, da like a, dB/dC like B/C, dS0 like S0.
 * S0, dS_fin and dS0 may be NULL (zero initial state / no final-state
 * gradient / not wanted).
 */
int oracle_bwd(const oracle_dims* d, const double* X, const double* a, const double* B,
               const double* C, const double* S0, const double* dY, const double* dS_fin,
               double* dX, double* da, double* dB, double* dC, double* dS0)
{
    if (!d || !X || !a || !B || !C || !dY || !dX || !da || !dB || !dC) return 1;
    if (d->ngroups <= 0 || d->nheads % d->ngroups != 0) return 2;
    const int64_t Bz = d->batch, L = d->seqlen, H = d->nheads, P = d->headdim;
    const int64_t N = d->dstate, G = d->ngroups, PN = P * N;
    const int64_t K = 64;                         /* steps per recomputed segment */
    const int64_t nck = (L + K - 1) / K;
    double* ck = (double*)malloc(sizeof(double) * (size_t)((nck > 0 ? nck : 1) * PN));
    double* seg = (double*)malloc(sizeof(double) * (size_t)(K * PN));
    double* S = (double*)malloc(sizeof(double) * (size_t)PN);
    double* Gs = (double*)malloc(sizeof(double) * (size_t)PN);
    if (!ck || !seg || !S || !Gs) {
        free(ck); free(seg); free(S); free(Gs);
        return 3;
    }
    memset(dB, 0, sizeof(double) * (size_t)(Bz * L * G * N));
    memset(dC, 0, sizeof(double) * (size_t)(Bz * L * G * N));
#define X_AT(t, p) X[((b * L + (t)) * H + h) * P + (p)]
#define DX_AT(t, p) dX[((b * L + (t)) * H + h) * P + (p)]
#define DY_AT(t, p) dY[((b * L + (t)) * H + h) * P + (p)]
#define A_AT(t) a[(b * L + (t)) * H + h]
#define B_AT(t, n) B[((b * L + (t)) * G + g) * N + (n)]
#define C_AT(t, n) C[((b * L + (t)) * G + g) * N + (n)]
    for (int64_t b = 0; b < Bz; ++b)
        for (int64_t h = 0; h < H; ++h) {
            const int64_t g = h * G / H;
            /* forward sweep: ck[m] = the state entering step m*K */
            for (int64_t k = 0; k < PN; ++k) S[k] = S0 ? S0[(b * H + h) * PN + k] : 0.0;
            for (int64_t t = 0; t < L; ++t) {
                if (t % K == 0) memcpy(ck + (t / K) * PN, S, sizeof(double) * (size_t)PN);
                const double e = exp(A_AT(t));
                for (int64_t p = 0; p < P; ++p)
                    for (int64_t n = 0; n < N; ++n)
                        S[p * N + n] = e * S[p * N + n] + X_AT(t, p) * B_AT(t, n);
            }
            /* reverse sweep */
            for (int64_t k = 0; k < PN; ++k) Gs[k] = dS_fin ? dS_fin[(b * H + h) * PN + k] : 0.0;
            for (int64_t m = nck - 1; m >= 0; --m) {
                const int64_t t0 = m * K, t1 = (t0 + K < L) ? t0 + K : L;
                /* recompute the segment's post-update states */
                memcpy(S, ck + m * PN, sizeof(double) * (size_t)PN);
                for (int64_t t = t0; t < t1; ++t) {
                    const double e = exp(A_AT(t));
                    for (int64_t p = 0; p < P; ++p)
                        for (int64_t n = 0; n < N; ++n)
                            S[p * N + n] = e * S[p * N + n] + X_AT(t, p) * B_AT(t, n);
                    memcpy(seg + (t - t0) * PN, S, sizeof(double) * (size_t)PN);
                }
                for (int64_t t = t1 - 1; t >= t0; --t) {
                    const double* St = seg + (t - t0) * PN;
                    const double* Sprev = (t > t0) ? seg + (t - t0 - 1) * PN : ck + m * PN;
                    /* G_t = dY_t (x) C_t + (decayed later contributions, already in Gs) */
                    for (int64_t p = 0; p < P; ++p)
                        for (int64_t n = 0; n < N; ++n) Gs[p * N + n] += DY_AT(t, p) * C_AT(t, n);
                    for (int64_t n = 0; n < N; ++n) {
                        double sc = 0.0, sb = 0.0;
                        for (int64_t p = 0; p < P; ++p) {
                            sc += DY_AT(t, p) * St[p * N + n];
                            sb += Gs[p * N + n] * X_AT(t, p);
                        }
                        dC[((b * L + t) * G + g) * N + n] += sc;
                        dB[((b * L + t) * G + g) * N + n] += sb;
                    }
                    for (int64_t p = 0; p < P; ++p) {
                        double s = 0.0;
                        for (int64_t n = 0; n < N; ++n) s += Gs[p * N + n] * B_AT(t, n);
                        DX_AT(t, p) = s;
                    }
                    const double e = exp(A_AT(t));
                    double s = 0.0;
                    for (int64_t k = 0; k < PN; ++k) s += Gs[k] * Sprev[k];
                    da[(b * L + t) * H + h] = e * s;
                    for (int64_t k = 0; k < PN; ++k) Gs[k] *= e;   /* now dl/dS_{t-1} */
                }
            }
            if (dS0) memcpy(dS0 + (b * H + h) * PN, Gs, sizeof(double) * (size_t)PN);
        }
#undef X_AT
#undef DX_AT
#undef DY_AT
#undef A_AT
#undef B_AT
#undef C_AT
    free(ck);
    free(seg);
    free(S);
    free(Gs);
    return 0;
}
