/*
 * gdr2_oracle.c -- plain fp64 CPU oracle for the Gated Delta Rule-2 operator.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code, no
 * header and no constant with the GPU library, and the GPU library never
 * calls it.
 *
 * What it computes is the plain definition of the operator, token by token, in
 * double precision (Gated DeltaNet-2 pages, "The Gated Delta Rule-2 State
 * Update", Steps 1-5 and the combined form Eq. 10):
 *
 *     S_bar = Diag(alpha_t) S_{t-1},  alpha_t = exp(g_t)   (Step 1, Eq. 12)
 *     r_t   = S_bar^T (b_t * k_t)                          (Step 2)
 *     z_t   = w_t * v_t                                    (Step 3)
 *     S_t   = S_bar + k_t (z_t - r_t)^T                    (Step 4)
 *     o_t   = S_t^T q_t                                    (Step 5)
 *
 * The state is dk x dv, row i is key channel i, column j is value channel j.
 * The decay is applied before the edit, and the output reads the updated
 * state.  There is no query scaling.  Packed variable-length batches restart
 * from their own initial state at every sequence boundary (pages, Appendix
 * C.6: the chunk index construction resets the state at each boundary).  The
 * single-token decode step is the same loop body applied once (pages,
 * Appendix C.5).
 *
 * Layouts (all fp64, row-major, last index fastest):
 *   q, k, g, b : [Ttot][H][dk]     v, w : [Ttot][H][dv]
 *   S0, ST     : [N][H][dk][dv]    o    : [Ttot][H][dv]
 *   cu         : [N+1] token offsets of each sequence inside Ttot.
 * S0 == NULL means a zero initial state; ST == NULL means "do not store".
 * A (sequence, head) pair is skipped when mask != NULL and mask[n*H+h] == 0;
 * its outputs are then left untouched.
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* One token of Eq. 10 on one head, in place on S (dk x dv), o gets S_t^T q_t. */
static void gdr2_token(double *S, int dk, int dv,
                       const double *q, const double *k, const double *v,
                       const double *g, const double *b, const double *w,
                       double *o, double *r /* scratch, dv */)
{
    /* Step 1: channel-wise decay along the key axis. */
    for (int i = 0; i < dk; ++i) {
        const double alpha = exp(g[i]);
        for (int j = 0; j < dv; ++j) S[i * dv + j] *= alpha;
    }
    /* Step 2: read the decayed state along the gated erase direction b*k. */
    for (int j = 0; j < dv; ++j) r[j] = 0.0;
    for (int i = 0; i < dk; ++i) {
        const double e = b[i] * k[i];
        for (int j = 0; j < dv; ++j) r[j] += S[i * dv + j] * e;
    }
    /* Steps 3-4: write the residual between the gated target w*v and the
       read, along the un-gated key k. */
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) S[i * dv + j] += k[i] * (w[j] * v[j] - r[j]);
    /* Step 5: read the updated state with the query. */
    for (int j = 0; j < dv; ++j) o[j] = 0.0;
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) o[j] += S[i * dv + j] * q[i];
}

int gdr2_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Chunk-free forward over packed sequences.  Returns 0, or -1 on bad sizes or
   allocation failure. */
int gdr2_oracle_fwd(const double *q, const double *k, const double *v,
                    const double *g, const double *b, const double *w,
                    const double *S0, double *o, double *ST,
                    const long long *cu, int N, int H, int dk, int dv,
                    const unsigned char *mask, int nthreads)
{
    if (N < 0 || H <= 0 || dk <= 0 || dv <= 0 || !cu) return -1;
    for (int n = 0; n < N; ++n)
        if (cu[n] < 0 || cu[n + 1] < cu[n]) return -1;
    int bad = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for schedule(dynamic, 1) reduction(|| : bad)
    for (long long nh = 0; nh < (long long)N * H; ++nh) {
        const int n = (int)(nh / H), h = (int)(nh % H);
        if (mask && !mask[nh]) continue;
        double *S = (double *)malloc(sizeof(double) * (size_t)dk * dv);
        double *r = (double *)malloc(sizeof(double) * (size_t)dv);
        if (!S || !r) { free(S); free(r); bad = 1; continue; }
        const size_t sz = (size_t)dk * dv;
        if (S0) memcpy(S, S0 + (size_t)nh * sz, sizeof(double) * sz);
        else memset(S, 0, sizeof(double) * sz);
        for (long long t = cu[n]; t < cu[n + 1]; ++t) {
            const size_t xk = ((size_t)t * H + h) * dk, xv = ((size_t)t * H + h) * dv;
            gdr2_token(S, dk, dv, q + xk, k + xk, v + xv, g + xk, b + xk, w + xv,
                       o + xv, r);
        }
        if (ST) memcpy(ST + (size_t)nh * sz, S, sizeof(double) * sz);
        free(S);
        free(r);
    }
    return bad ? -1 : 0;
}

/* One decode step for N sequences: inputs [N][H][d], state [N][H][dk][dv]
   updated in place, o [N][H][dv]. */
int gdr2_oracle_decode(const double *q, const double *k, const double *v,
                       const double *g, const double *b, const double *w,
                       double *S, double *o, int N, int H, int dk, int dv, int nthreads)
{
    if (N < 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
    int bad = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for schedule(static) reduction(|| : bad)
    for (long long nh = 0; nh < (long long)N * H; ++nh) {
        double *r = (double *)malloc(sizeof(double) * (size_t)dv);
        if (!r) { bad = 1; continue; }
        const size_t xk = (size_t)nh * dk, xv = (size_t)nh * dv;
        gdr2_token(S + (size_t)nh * dk * dv, dk, dv, q + xk, k + xk, v + xv, g + xk,
                   b + xk, w + xv, o + xv, r);
        free(r);
    }
    return bad ? -1 : 0;
}
