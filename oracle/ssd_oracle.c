/*
 * ssd_oracle.c -- plain, slow, fp64 CPU oracle for the Mamba-2 SSD layer core.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark load this file's library.  It shares no
 * source, header or helper with the GPU library and never calls it.
 *
 * What it computes is the plain definition of the state-space recurrence
 * with a per-head scalar ("input-dependent diagonal") decay, token by token:
 *
 *   for each batch b and head h, with group g = h / (H / G) and state
 *   M = H0[b,h] (a P x N matrix, zeros when no initial state is given):
 *     for t = 0 .. L-1:
 *       r        = exp(dt[b,t,h] * A[h])
 *       M[p,n]   = r * M[p,n] + (dt[b,t,h] * x[b,t,h,p]) * B[b,t,g,n]
 *       y[b,t,h,p] = sum_{n=0..N-1} M[p,n] * C[b,t,g,n]  +  D[h] * x[b,t,h,p]
 *   final_state[b,h] = M after the last token.
 *
 * Sources: "Mamba-Family State-Space Model Kernels on a Programmable CGLA",
 * Sec. III-A (recurrent state h updated token after token / chunk after
 * chunk; A_c is an input-dependent diagonal matrix; the layer's in-projection
 * produces x, B, C and the step size); "Compiler-First State Space Duality and
 * Portable O(1) Autoregressive Caching for Inference", abstract (diagonal
 * per-head dynamics; a cached state carried across decode steps).  The
 * chunked evaluation the GPU uses reaches exactly this result, so the oracle
 * is the definition itself, with no chunking.
 *
 * Readings where the pages are silent: the input enters as dt*x*B^T with no
 * decay at its own step; the output reads the state after the update; dt is
 * used as given (already positive); D is one scalar per head; head h uses
 * group h / (H/G) (contiguous blocks of heads share B and C).
 *
 * Precision: every value is fp64 (inputs arrive as fp64 copies of the exact
 * bf16/fp32 values), exp() is the host libm, the n-sum runs in index order.
 * Parallel over (b,h) pairs only; nothing is reduced across threads, so the
 * result is bitwise identical for any thread count.
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_ERR_ARG (-1)
#define ORACLE_ERR_NOMEM (-2)

/* One token for one (b,h): decay the state, add the input, read the output. */
static void oracle_token(double *M, const double *xt, double dtv, double Ah,
                         const double *Bt, const double *Ct, double Dh,
                         double *yt, int P, int N)
{
    const double r = exp(dtv * Ah);
    for (int p = 0; p < P; ++p) {
        const double u = dtv * xt[p];
        double *row = M + (size_t)p * N;
        double acc = 0.0;
        for (int n = 0; n < N; ++n) {
            row[n] = r * row[n] + u * Bt[n];
            acc += row[n] * Ct[n];
        }
        yt[p] = acc + Dh * xt[p];
    }
}

static int shape_ok(int batch, int seqlen, int nheads, int headdim, int dstate, int ngroups)
{
    if (batch <= 0 || seqlen < 0 || nheads <= 0 || headdim <= 0 || dstate <= 0 || ngroups <= 0)
        return 0;
    if (nheads % ngroups != 0)
        return 0;
    return 1;
}

/*
 * Prefill over a whole sequence.
 *   x  [B,L,H,P]   dt [B,L,H]   A [H]   Bm, Cm [B,L,G,N]   D [H] or NULL (= 0)
 *   h0 [B,H,P,N] or NULL (= zeros)
 *   y  [B,L,H,P] (written)   hT [B,H,P,N] or NULL (written; may alias h0)
 * nthreads <= 0 means the OpenMP default.  Returns 0 or a negative code.
 */
int ssd_oracle_prefill(const double *x, const double *dt, const double *A,
                       const double *Bm, const double *Cm, const double *D,
                       const double *h0, double *y, double *hT,
                       int batch, int seqlen, int nheads, int headdim,
                       int dstate, int ngroups, int nthreads)
{
    if (!shape_ok(batch, seqlen, nheads, headdim, dstate, ngroups))
        return ORACLE_ERR_ARG;
    if (!A || (seqlen > 0 && (!x || !dt || !Bm || !Cm || !y)))
        return ORACLE_ERR_ARG;
    const int B = batch, L = seqlen, H = nheads, P = headdim, N = dstate, G = ngroups;
    const int heads_per_group = H / G;
    const long pairs = (long)B * H;
    int status = ORACLE_OK;
#ifdef _OPENMP
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (long bh = 0; bh < pairs; ++bh) {
        const int b = (int)(bh / H), h = (int)(bh % H);
        const int g = h / heads_per_group;
        double *M = (double *)malloc(sizeof(double) * (size_t)P * N);
        if (!M) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            status = ORACLE_ERR_NOMEM;
            continue;
        }
        const size_t sidx = ((size_t)b * H + h) * (size_t)P * N;
        if (h0)
            memcpy(M, h0 + sidx, sizeof(double) * (size_t)P * N);
        else
            memset(M, 0, sizeof(double) * (size_t)P * N);
        const double Dh = D ? D[h] : 0.0;
        for (int t = 0; t < L; ++t) {
            const size_t tok = (size_t)b * L + t;
            oracle_token(M, x + (tok * H + h) * P, dt[tok * H + h], A[h],
                         Bm + (tok * G + g) * N, Cm + (tok * G + g) * N, Dh,
                         y + (tok * H + h) * P, P, N);
        }
        if (hT)
            memcpy(hT + sidx, M, sizeof(double) * (size_t)P * N);
        free(M);
    }
    return status;
}

/*
 * One decode token for every (b,h), state updated in place.
 *   state [B,H,P,N]   x [B,H,P]   dt [B,H]   A [H]   Bm, Cm [B,G,N]
 *   D [H] or NULL     y [B,H,P] (written)
 */
int ssd_oracle_step(double *state, const double *x, const double *dt, const double *A,
                    const double *Bm, const double *Cm, const double *D, double *y,
                    int batch, int nheads, int headdim, int dstate, int ngroups, int nthreads)
{
    if (!shape_ok(batch, 1, nheads, headdim, dstate, ngroups))
        return ORACLE_ERR_ARG;
    if (!state || !x || !dt || !A || !Bm || !Cm || !y)
        return ORACLE_ERR_ARG;
    const int B = batch, H = nheads, P = headdim, N = dstate, G = ngroups;
    const int heads_per_group = H / G;
    const long pairs = (long)B * H;
#ifdef _OPENMP
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(static) num_threads(nthreads)
#endif
    for (long bh = 0; bh < pairs; ++bh) {
        const int b = (int)(bh / H), h = (int)(bh % H);
        const int g = h / heads_per_group;
        oracle_token(state + (size_t)bh * P * N, x + (size_t)bh * P, dt[bh], A[h],
                     Bm + ((size_t)b * G + g) * N, Cm + ((size_t)b * G + g) * N,
                     D ? D[h] : 0.0, y + (size_t)bh * P, P, N);
    }
    return ORACLE_OK;
}

/* Number of OpenMP threads a call with nthreads <= 0 would use. */
int ssd_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
