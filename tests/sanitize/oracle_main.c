/* Runs the fp64 oracle's three entry points on small inputs (fixed and packed
 * sequences, an empty sequence, a partial last segment of its 64-token
 * checkpoints, one and two threads) under the address and undefined-behaviour
 * sanitizers, and checks two facts that need no reference: a packed run
 * equals separate runs, and one step equals a one-token forward pass.
 * Prints "oracle sanitize: ok" or exits 1. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_fwd(int B, int T, int H, int Dk, int Dv, int N, const int32_t *cu_seqlens, const double *q,
               const double *k, const double *v, const double *beta, const double *g, const double *h0,
               double *o, double *hT, int nthreads);
int oracle_bwd(int B, int T, int H, int Dk, int Dv, int N, const int32_t *cu_seqlens, const double *q,
               const double *k, const double *v, const double *beta, const double *g, const double *h0,
               const double *dO, const double *dhT, double *dq, double *dk, double *dv, double *dbeta,
               double *dg, double *dh0, int nthreads);
int oracle_step(int B, int H, int Dk, int Dv, const double *q, const double *k, const double *v,
                const double *beta, const double *g, double *state, double *o, int nthreads);

static uint64_t rng = 88172645463325252ull;
static double urand(void) { /* xorshift64, uniform in (-1, 1) */
    rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
    return (double)(rng >> 11) / (double)(1ull << 52) - 1.0;
}
static double *alloc(size_t n, int fill) {
    double *p = (double *)malloc((n ? n : 1) * sizeof(double));
    for (size_t i = 0; i < n; ++i) p[i] = fill ? urand() : 0.0;
    return p;
}
static void fail(const char *what) { fprintf(stderr, "oracle sanitize: %s\n", what); exit(1); }

int main(void) {
    const int H = 2, Dk = 8, Dv = 12;
    const int lens[4] = {70, 0, 1, 130};
    const int N = 4, T = 201;
    const int32_t cu[5] = {0, 70, 70, 71, 201};
    double *q = alloc((size_t)T * H * Dk, 1), *k = alloc((size_t)T * H * Dk, 1);
    double *v = alloc((size_t)T * H * Dv, 1), *beta = alloc((size_t)T * H, 1), *g = alloc((size_t)T * H, 1);
    double *h0 = alloc((size_t)N * H * Dk * Dv, 1), *dO = alloc((size_t)T * H * Dv, 1);
    double *dhT = alloc((size_t)N * H * Dk * Dv, 1);
    for (int i = 0; i < T * H; ++i) { beta[i] = 0.5 + 0.4 * beta[i]; g[i] = -0.1 * fabs(g[i]); }
    for (int t = 0; t < T * H; ++t) { /* unit keys */
        double s = 0; for (int d = 0; d < Dk; ++d) s += k[t * Dk + d] * k[t * Dk + d];
        for (int d = 0; d < Dk; ++d) k[t * Dk + d] /= sqrt(s);
    }
    double *o = alloc((size_t)T * H * Dv, 0), *hT = alloc((size_t)N * H * Dk * Dv, 0);
    for (int nt = 1; nt <= 2; ++nt) {
        if (oracle_fwd(1, T, H, Dk, Dv, N, cu, q, k, v, beta, g, h0, o, hT, nt)) fail("fwd");
        double *dq = alloc((size_t)T * H * Dk, 0), *dk = alloc((size_t)T * H * Dk, 0), *dv = alloc((size_t)T * H * Dv, 0);
        double *db = alloc((size_t)T * H, 0), *dg = alloc((size_t)T * H, 0), *dh0 = alloc((size_t)N * H * Dk * Dv, 0);
        if (oracle_bwd(1, T, H, Dk, Dv, N, cu, q, k, v, beta, g, h0, dO, dhT, dq, dk, dv, db, dg, dh0, nt)) fail("bwd");
        if (oracle_bwd(1, T, H, Dk, Dv, N, cu, q, k, v, beta, NULL, NULL, dO, NULL, dq, dk, dv, db, NULL, NULL, nt))
            fail("bwd ungated");
        free(dq); free(dk); free(dv); free(db); free(dg); free(dh0);
    }
    /* invalid arguments are refused */
    if (!oracle_fwd(2, T, H, Dk, Dv, N, cu, q, k, v, beta, g, h0, o, hT, 1)) fail("B != 1 with offsets");
    if (!oracle_bwd(1, T, H, Dk, Dv, N, cu, q, k, v, beta, g, h0, dO, dhT, o, o, o, o, NULL, NULL, 1)) fail("g/dg");
    /* packed = separate runs, bit for bit */
    for (int n = 0; n < N; ++n) {
        const int L = lens[n], s = cu[n];
        double *o1 = alloc((size_t)L * H * Dv, 0), *h1 = alloc((size_t)H * Dk * Dv, 0);
        if (oracle_fwd(1, L, H, Dk, Dv, 1, NULL, q + (size_t)s * H * Dk, k + (size_t)s * H * Dk, v + (size_t)s * H * Dv,
                       beta + (size_t)s * H, g + (size_t)s * H, h0 + (size_t)n * H * Dk * Dv, o1, h1, 1))
            fail("fwd separate");
        if (memcmp(o1, o + (size_t)s * H * Dv, sizeof(double) * L * H * Dv)) fail("packed o");
        if (memcmp(h1, hT + (size_t)n * H * Dk * Dv, sizeof(double) * H * Dk * Dv)) fail("packed hT");
        free(o1); free(h1);
    }
    /* one step = a one-token forward pass */
    {
        double *st = alloc((size_t)H * Dk * Dv, 0), *os = alloc((size_t)H * Dv, 0);
        double *o1 = alloc((size_t)H * Dv, 0), *h1 = alloc((size_t)H * Dk * Dv, 0);
        memcpy(st, h0, sizeof(double) * H * Dk * Dv);
        if (oracle_step(1, H, Dk, Dv, q, k, v, beta, g, st, os, 1)) fail("step");
        if (oracle_fwd(1, 1, H, Dk, Dv, 1, NULL, q, k, v, beta, g, h0, o1, h1, 1)) fail("fwd 1");
        for (int i = 0; i < H * Dv; ++i) if (fabs(os[i] - o1[i]) > 1e-12) fail("step o");
        for (int i = 0; i < H * Dk * Dv; ++i) if (fabs(st[i] - h1[i]) > 1e-12) fail("step state");
        free(st); free(os); free(o1); free(h1);
    }
    free(q); free(k); free(v); free(beta); free(g); free(h0); free(dO); free(dhT); free(o); free(hT);
    printf("oracle sanitize: ok\n");
    return 0;
}
