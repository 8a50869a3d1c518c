/*
 * gdr2_oracle_bwd.c -- plain fp64 CPU oracle of the Gated Delta Rule-2
 * backward pass (reverse-mode differentiation of the token recurrence).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code, no
 * header and no constant with the GPU library, and the GPU library never
 * calls it.
 *
 * The forward is the recurrence of Eq. 10 (Gated DeltaNet-2 pages, "The Gated
 * Delta Rule-2 State Update", Steps 1-5), per token and head:
 *
 *     S_bar = Diag(alpha) S,          alpha = exp(g)       (Step 1)
 *     r     = S_bar^T e,              e = b * k            (Step 2)
 *     delta = z - r,                  z = w * v            (Step 3)
 *     S'    = S_bar + k delta^T                            (Step 4)
 *     o     = S'^T q                                       (Step 5)
 *
 * Given dL/do for every token and dL/dS_T for the final state, this file
 * applies the chain rule to those five steps in reverse token order (the
 * pages' backward flow: output path, state path, then the gates and the
 * log-decay, "Gate-Aware Backward Pass"):
 *
 *     dS'   += q do^T;                dq = S' do
 *     ddelta = dS'^T k;               dk = dS' delta
 *     dz = ddelta: dw = dz * v, dv = dz * w;    dr = -ddelta
 *     dS_bar = dS' + e dr^T;          de = S_bar dr
 *     db = de * k;                    dk += de * b
 *     dalpha_i = sum_j dS_bar_ij S_ij; dg = dalpha * alpha
 *     dS (before the token) = Diag(alpha) dS_bar
 *
 * Memory: the state before every 64th token is kept from a first forward
 * sweep, and each 64-token segment is re-run forward before its tokens are
 * differentiated, so a (sequence, head) costs (T/64 + 65) dk x dv doubles.
 *
 * Layouts as in gdr2_oracle.c: q, k, g, b [Ttot][H][dk]; v, w [Ttot][H][dv];
 * S0, dST, dS0 [N][H][dk][dv]; cu [N+1].  S0 == NULL means zero initial
 * state, dST == NULL means dL/dS_T = 0, dS0 == NULL means "do not store".
 * Outputs for pairs with mask[n*H+h] == 0 are left untouched.
 */
#include <stddef.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define SEG 64

/* State after one token of Eq. 10, in place (no output). */
static void step_state(double *S, int dk, int dv, const double *k, const double *v,
                       const double *g, const double *b, const double *w, double *r)
{
    for (int i = 0; i < dk; ++i) {
        const double a = exp(g[i]);
        for (int j = 0; j < dv; ++j) S[i * dv + j] *= a;
    }
    for (int j = 0; j < dv; ++j) r[j] = 0.0;
    for (int i = 0; i < dk; ++i) {
        const double e = b[i] * k[i];
        for (int j = 0; j < dv; ++j) r[j] += S[i * dv + j] * e;
    }
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) S[i * dv + j] += k[i] * (w[j] * v[j] - r[j]);
}

/* Reverse step of one token.  S holds the state before the token; dS holds
   dL/dS after it on entry and dL/dS before it on return. */
static void back_token(const double *S, double *dS, int dk, int dv,
                       const double *q, const double *k, const double *v,
                       const double *g, const double *b, const double *w, const double *dout,
                       double *dq, double *dk_, double *dv_, double *dg, double *db, double *dw,
                       double *Sb, double *Sn, double *r, double *delta, double *dr)
{
    /* recompute the token: S_bar, r, delta, S' */
    for (int i = 0; i < dk; ++i) {
        const double a = exp(g[i]);
        for (int j = 0; j < dv; ++j) Sb[i * dv + j] = a * S[i * dv + j];
    }
    for (int j = 0; j < dv; ++j) r[j] = 0.0;
    for (int i = 0; i < dk; ++i) {
        const double e = b[i] * k[i];
        for (int j = 0; j < dv; ++j) r[j] += Sb[i * dv + j] * e;
    }
    for (int j = 0; j < dv; ++j) delta[j] = w[j] * v[j] - r[j];
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) Sn[i * dv + j] = Sb[i * dv + j] + k[i] * delta[j];

    /* Step 5: o = S'^T q */
    for (int i = 0; i < dk; ++i) {
        double acc = 0.0;
        for (int j = 0; j < dv; ++j) {
            dS[i * dv + j] += q[i] * dout[j];
            acc += Sn[i * dv + j] * dout[j];
        }
        dq[i] = acc;
    }
    /* Step 4: S' = S_bar + k delta^T */
    for (int j = 0; j < dv; ++j) dr[j] = 0.0;
    for (int i = 0; i < dk; ++i) {
        double acc = 0.0;
        for (int j = 0; j < dv; ++j) {
            acc += dS[i * dv + j] * delta[j];
            dr[j] += dS[i * dv + j] * k[i];      /* ddelta, for now */
        }
        dk_[i] = acc;
    }
    /* Step 3: delta = z - r with z = w * v */
    for (int j = 0; j < dv; ++j) {
        dw[j] = dr[j] * v[j];
        dv_[j] = dr[j] * w[j];
        dr[j] = -dr[j];                          /* dL/dr */
    }
    /* Step 2: r = S_bar^T e with e = b * k; dS_bar = dS' + e dr^T */
    for (int i = 0; i < dk; ++i) {
        const double e = b[i] * k[i];
        double de = 0.0;
        for (int j = 0; j < dv; ++j) {
            de += Sb[i * dv + j] * dr[j];
            dS[i * dv + j] += e * dr[j];
        }
        db[i] = de * k[i];
        dk_[i] += de * b[i];
    }
    /* Step 1: S_bar = Diag(exp(g)) S */
    for (int i = 0; i < dk; ++i) {
        const double a = exp(g[i]);
        double da = 0.0;
        for (int j = 0; j < dv; ++j) {
            da += dS[i * dv + j] * S[i * dv + j];
            dS[i * dv + j] *= a;
        }
        dg[i] = da * a;
    }
}

int gdr2_oracle_bwd_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

int gdr2_oracle_bwd(const double *q, const double *k, const double *v,
                    const double *g, const double *b, const double *w,
                    const double *S0, const double *dO, const double *dST,
                    double *dq, double *dk, double *dv, double *dg, double *db, double *dw,
                    double *dS0, const long long *cu, int N, int H, int dk_, int dv_,
                    const unsigned char *mask, int nthreads)
{
    if (N < 0 || H <= 0 || dk_ <= 0 || dv_ <= 0 || !cu) return -1;
    for (int n = 0; n < N; ++n)
        if (cu[n] < 0 || cu[n + 1] < cu[n]) return -1;
    const int DK = dk_, DV = dv_;
    const size_t sz = (size_t)DK * DV;
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
        const long long t0 = cu[n], L = cu[n + 1] - cu[n];
        const long long nseg = (L + SEG - 1) / SEG;
        double *ck = (double *)malloc(sizeof(double) * sz * (size_t)(nseg + 1));
        double *seg = (double *)malloc(sizeof(double) * sz * (SEG + 1));
        double *dS = (double *)malloc(sizeof(double) * sz);
        double *Sb = (double *)malloc(sizeof(double) * sz);
        double *Sn = (double *)malloc(sizeof(double) * sz);
        double *tmp = (double *)malloc(sizeof(double) * (size_t)DV * 3);
        if (!ck || !seg || !dS || !Sb || !Sn || !tmp) {
            free(ck); free(seg); free(dS); free(Sb); free(Sn); free(tmp);
            bad = 1;
            continue;
        }
        double *r = tmp, *delta = tmp + DV, *dr = tmp + 2 * DV;
        /* forward sweep: the state before every segment */
        if (S0) memcpy(ck, S0 + (size_t)nh * sz, sizeof(double) * sz);
        else memset(ck, 0, sizeof(double) * sz);
        for (long long s = 0; s < nseg; ++s) {
            memcpy(ck + (size_t)(s + 1) * sz, ck + (size_t)s * sz, sizeof(double) * sz);
            const long long e = (s + 1) * SEG < L ? (s + 1) * SEG : L;
            for (long long t = s * SEG; t < e; ++t) {
                const size_t xk = ((size_t)(t0 + t) * H + h) * DK, xv = ((size_t)(t0 + t) * H + h) * DV;
                step_state(ck + (size_t)(s + 1) * sz, DK, DV, k + xk, v + xv, g + xk, b + xk,
                           w + xv, r);
            }
        }
        if (dST) memcpy(dS, dST + (size_t)nh * sz, sizeof(double) * sz);
        else memset(dS, 0, sizeof(double) * sz);
        /* backward, segment by segment from the last */
        for (long long s = nseg - 1; s >= 0; --s) {
            const long long e = (s + 1) * SEG < L ? (s + 1) * SEG : L, len = e - s * SEG;
            memcpy(seg, ck + (size_t)s * sz, sizeof(double) * sz);
            for (long long j = 0; j < len - 1; ++j) {   /* seg[j] = state before token j */
                const long long t = s * SEG + j;
                const size_t xk = ((size_t)(t0 + t) * H + h) * DK, xv = ((size_t)(t0 + t) * H + h) * DV;
                memcpy(seg + (size_t)(j + 1) * sz, seg + (size_t)j * sz, sizeof(double) * sz);
                step_state(seg + (size_t)(j + 1) * sz, DK, DV, k + xk, v + xv, g + xk, b + xk,
                           w + xv, r);
            }
            for (long long j = len - 1; j >= 0; --j) {
                const long long t = s * SEG + j;
                const size_t xk = ((size_t)(t0 + t) * H + h) * DK, xv = ((size_t)(t0 + t) * H + h) * DV;
                back_token(seg + (size_t)j * sz, dS, DK, DV, q + xk, k + xk, v + xv, g + xk,
                           b + xk, w + xv, dO + xv, dq + xk, dk + xk, dv + xv, dg + xk, db + xk,
                           dw + xv, Sb, Sn, r, delta, dr);
            }
        }
        if (dS0) memcpy(dS0 + (size_t)nh * sz, dS, sizeof(double) * sz);
        free(ck); free(seg); free(dS); free(Sb); free(Sn); free(tmp);
    }
    return bad ? -1 : 0;
}
