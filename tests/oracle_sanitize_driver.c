/*
 * oracle_sanitize_driver.c -- drives the fp64 oracle (test infrastructure)
 * through every option of its C interface on tiny inputs, for a host build
 * under AddressSanitizer and UndefinedBehaviorSanitizer
 * (tests/test_oracle_sanitizers.py):
 *   - the forward over packed sequences of lengths 5, 0 and 17, with and
 *     without S0, S_T and a (sequence, head) mask;
 *   - decode run token by token, which must reproduce the forward's outputs
 *     and end states (the same recurrence, Eq. 10 of the pages' "The Gated
 *     Delta Rule-2 State Update");
 *   - the backward with and without S0, dS_T and dS0.
 * Exit status 0 on success, 1 on a mismatch, 2 on an oracle error.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int gdr2_oracle_fwd(const double *q, const double *k, const double *v, const double *g,
                    const double *b, const double *w, const double *S0, double *o, double *ST,
                    const long long *cu, int N, int H, int dk, int dv, const unsigned char *mask,
                    int nthreads);
int gdr2_oracle_decode(const double *q, const double *k, const double *v, const double *g,
                       const double *b, const double *w, double *S, double *o, int N, int H,
                       int dk, int dv, int nthreads);
int gdr2_oracle_bwd(const double *q, const double *k, const double *v, const double *g,
                    const double *b, const double *w, const double *S0, const double *dO,
                    const double *dST, double *dq, double *dk, double *dv, double *dg, double *db,
                    double *dw, double *dS0, const long long *cu, int N, int H, int dk_, int dv_,
                    const unsigned char *mask, int nthreads);

static unsigned long long seed = 12345;
static double urand(void) {  /* uniform in [0, 1): 64-bit LCG, top 53 bits */
    seed = seed * 6364136223846793005ULL + 1442695040888963407ULL;
    return (double)(seed >> 11) / 9007199254740992.0;
}
static double *fill(size_t n, double lo, double hi) {
    double *x = (double *)malloc(sizeof(double) * (n ? n : 1));
    for (size_t i = 0; i < n; ++i) x[i] = lo + (hi - lo) * urand();
    return x;
}

int main(void) {
    enum { N = 3, H = 2, DK = 4, DV = 3 };
    const long long cu[N + 1] = {0, 5, 5, 22};
    const long long T = cu[N];
    const size_t nk = (size_t)T * H * DK, nv = (size_t)T * H * DV, ns = (size_t)N * H * DK * DV;
    double *q = fill(nk, -1, 1), *k = fill(nk, -1, 1), *g = fill(nk, -0.5, 0), *b = fill(nk, 0, 2);
    double *v = fill(nv, -1, 1), *w = fill(nv, 0, 1), *S0 = fill(ns, -0.1, 0.1);
    double *o = fill(nv, 0, 0), *ST = fill(ns, 0, 0);
    if (gdr2_oracle_fwd(q, k, v, g, b, w, S0, o, ST, cu, N, H, DK, DV, NULL, 1)) return 2;

    /* decode, token by token, from S0 */
    double *S = (double *)malloc(sizeof(double) * ns);
    memcpy(S, S0, sizeof(double) * ns);
    double err = 0.0;
    for (int n = 0; n < N; ++n)
        for (long long t = cu[n]; t < cu[n + 1]; ++t) {
            double od[H * DV];
            const size_t xk = (size_t)t * H * DK, xv = (size_t)t * H * DV;
            if (gdr2_oracle_decode(q + xk, k + xk, v + xv, g + xk, b + xk, w + xv,
                                   S + (size_t)n * H * DK * DV, od, 1, H, DK, DV, 1))
                return 2;
            for (int i = 0; i < H * DV; ++i) err = fmax(err, fabs(od[i] - o[xv + i]));
        }
    for (size_t i = 0; i < ns; ++i) err = fmax(err, fabs(S[i] - ST[i]));
    if (err > 1e-12) {
        fprintf(stderr, "decode vs forward: %g\n", err);
        return 1;
    }

    /* the optional pointers and the mask */
    const unsigned char mask[N * H] = {1, 0, 1, 1, 0, 1};
    double *o2 = fill(nv, 0, 0);
    if (gdr2_oracle_fwd(q, k, v, g, b, w, NULL, o2, NULL, cu, N, H, DK, DV, mask, 1)) return 2;
    if (gdr2_oracle_fwd(q, k, v, g, b, w, S0, o2, ST, cu, 0, H, DK, DV, NULL, 1)) return 2;

    /* backward, with and without the optional state tensors */
    double *dO = fill(nv, -1, 1), *dST = fill(ns, -0.1, 0.1);
    double *dq = fill(nk, 0, 0), *dkk = fill(nk, 0, 0), *dg = fill(nk, 0, 0), *db = fill(nk, 0, 0);
    double *dvv = fill(nv, 0, 0), *dw = fill(nv, 0, 0), *dS0 = fill(ns, 0, 0);
    if (gdr2_oracle_bwd(q, k, v, g, b, w, S0, dO, dST, dq, dkk, dvv, dg, db, dw, dS0, cu, N, H, DK,
                        DV, NULL, 1))
        return 2;
    if (gdr2_oracle_bwd(q, k, v, g, b, w, NULL, dO, NULL, dq, dkk, dvv, dg, db, dw, NULL, cu, N, H,
                        DK, DV, mask, 1))
        return 2;
    for (size_t i = 0; i < nk; ++i)
        if (!isfinite(dq[i]) || !isfinite(dkk[i]) || !isfinite(dg[i]) || !isfinite(db[i])) return 1;

    free(q); free(k); free(g); free(b); free(v); free(w); free(S0); free(o); free(ST); free(S);
    free(o2); free(dO); free(dST); free(dq); free(dkk); free(dg); free(db); free(dvv); free(dw);
    free(dS0);
    printf("oracle sanitizer driver: ok (decode vs forward %g)\n", err);
    return 0;
}
