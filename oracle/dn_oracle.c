/*
 * fp64 CPU oracle for the (gated) delta rule -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the package's smoke check and the benchmark's CPU-baseline
 * leg may call this.  It shares no code with the HIP library and is slow on
 * purpose: a plain token-by-token recurrence in double precision.
 *
 * What it computes (Gated DeltaNet review thread, "Gated Delta Networks:
 * Improving Mamba2 with Delta Rule", Table 1, rows "DeltaNet" and
 * "Gated DeltaNet"):
 *
 *     S_t = alpha_t * S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *     o_t = S_t q_t
 *
 * with S_t a d_v x d_k matrix, alpha_t = exp(g_t) (alpha == 1 when there is no
 * gate), no query scaling.  The chunkwise/WY method of "Parallelizing Linear
 * Transformers with the Delta Rule over Sequence Length" (page 1, answer Q1/Q2;
 * page 3, abstract) is an exact refactoring of this loop, so the loop itself
 * is the definition the parallel path must reproduce.
 *
 * Layouts (same as the library's):
 *   q, k  [B, T, H, Dk]      v, o  [B, T, H, Dv]     beta, g  [B, T, H]
 *   h0, hT, dh0, dhT  [N, H, Dk, Dv]  holding h = S^T (d_k x d_v)
 *   cu_seqlens (host, int32 [N+1]) or NULL: with it, B == 1 and sequence n
 *   covers tokens [cu[n], cu[n+1]); without it, N == B and each batch row is
 *   one sequence of T tokens.
 *
 * Backward: reverse-mode derivative of the same loop (sequential adjoint).
 * The loss is L = sum_t <dO_t, o_t> + <dhT, hT>.  For t = last..first, with
 * G = dL/dS_t accumulated from later steps:
 *     G    += dO_t q_t^T,            dq_t = S_t^T dO_t
 *     M     = I - beta_t k_t k_t^T
 *     dg_t  = alpha_t <G, S_{t-1} M>
 *     dbeta = (v_t - alpha_t S_{t-1} k_t) . (G k_t)
 *     dv_t  = beta_t G k_t
 *     dk_t  = -alpha_t beta_t (S_{t-1}^T G + G^T S_{t-1}) k_t + beta_t G^T v_t
 *     G    <- alpha_t G M
 * and dh0 = G^T at the end.  S_{t-1} is recomputed from checkpoints taken
 * every 64 tokens (a memory plan of the oracle, nothing more).
 *
 * Threads: independent (sequence, head) pairs run in parallel (OpenMP); each
 * pair is strictly sequential over its tokens.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define SEG 64

typedef struct {
    int B, T, H, Dk, Dv, N;
    const int32_t *cu;
} dims_t;

static size_t tok_off(const dims_t *d, int b, int t, int h, int D)
{
    return (((size_t)b * d->T + t) * d->H + h) * (size_t)D;
}

static size_t sc_off(const dims_t *d, int b, int t, int h)
{
    return ((size_t)b * d->T + t) * d->H + h;
}

static size_t st_off(const dims_t *d, int n, int h)
{
    return ((size_t)n * d->H + h) * (size_t)d->Dk * d->Dv;
}

/* token range [t0, t1) and batch row b of sequence n */
static void seq_range(const dims_t *d, int n, int *b, int *t0, int *t1)
{
    if (d->cu) {
        *b = 0;
        *t0 = d->cu[n];
        *t1 = d->cu[n + 1];
    } else {
        *b = n;
        *t0 = 0;
        *t1 = d->T;
    }
}

/* One step of the recurrence on S (Dv x Dk, row-major: S[i*Dk + j]).
 * sk is scratch of length Dv. */
static void step(double *S, int Dk, int Dv, const double *k, const double *v,
                 double beta, double alpha, double *sk)
{
    for (int i = 0; i < Dv; ++i) {
        double acc = 0.0;
        for (int j = 0; j < Dk; ++j) acc += S[(size_t)i * Dk + j] * k[j];
        sk[i] = acc;
    }
    /* S <- alpha * (S - beta (S k) k^T) + beta v k^T */
    for (int i = 0; i < Dv; ++i)
        for (int j = 0; j < Dk; ++j) {
            double s = S[(size_t)i * Dk + j];
            S[(size_t)i * Dk + j] = alpha * (s - beta * sk[i] * k[j]) + beta * v[i] * k[j];
        }
}

static void load_state(double *S, const double *h, int Dk, int Dv)
{
    /* S = h^T */
    if (!h) {
        memset(S, 0, sizeof(double) * (size_t)Dk * Dv);
        return;
    }
    for (int i = 0; i < Dv; ++i)
        for (int j = 0; j < Dk; ++j) S[(size_t)i * Dk + j] = h[(size_t)j * Dv + i];
}

static void store_state(double *h, const double *S, int Dk, int Dv)
{
    for (int j = 0; j < Dk; ++j)
        for (int i = 0; i < Dv; ++i) h[(size_t)j * Dv + i] = S[(size_t)i * Dk + j];
}

static int n_threads(int want)
{
#ifdef _OPENMP
    return want > 0 ? want : omp_get_max_threads();
#else
    (void)want;
    return 1;
#endif
}

/* Forward.  o may not be NULL; hT may be NULL. */
int oracle_fwd(int B, int T, int H, int Dk, int Dv, int N, const int32_t *cu_seqlens,
               const double *q, const double *k, const double *v, const double *beta,
               const double *g, const double *h0, double *o, double *hT, int nthreads)
{
    dims_t d = {B, T, H, Dk, Dv, N, cu_seqlens};
    if (B <= 0 || T < 0 || H <= 0 || Dk <= 0 || Dv <= 0 || N <= 0) return 1;
    if (cu_seqlens && B != 1) return 1;
    if (!cu_seqlens && N != B) return 1;
    int pairs = N * H;
    int nt = n_threads(nthreads);
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
    for (int p = 0; p < pairs; ++p) {
        int n = p / H, h = p % H, b, t0, t1;
        seq_range(&d, n, &b, &t0, &t1);
        double *S = (double *)malloc(sizeof(double) * (size_t)Dk * Dv);
        double *sk = (double *)malloc(sizeof(double) * (size_t)Dv);
        if (!S || !sk) {
#pragma omp atomic write
            err = 2;
            free(S);
            free(sk);
            continue;
        }
        load_state(S, h0 ? h0 + st_off(&d, n, h) : NULL, Dk, Dv);
        for (int t = t0; t < t1; ++t) {
            const double *kt = k + tok_off(&d, b, t, h, Dk);
            const double *vt = v + tok_off(&d, b, t, h, Dv);
            const double *qt = q + tok_off(&d, b, t, h, Dk);
            size_t s = sc_off(&d, b, t, h);
            double alpha = g ? exp(g[s]) : 1.0;
            step(S, Dk, Dv, kt, vt, beta[s], alpha, sk);
            double *ot = o + tok_off(&d, b, t, h, Dv);
            for (int i = 0; i < Dv; ++i) {
                double acc = 0.0;
                for (int j = 0; j < Dk; ++j) acc += S[(size_t)i * Dk + j] * qt[j];
                ot[i] = acc;
            }
        }
        if (hT) store_state(hT + st_off(&d, n, h), S, Dk, Dv);
        free(S);
        free(sk);
    }
    return err;
}

/* Backward (sequential adjoint).  dO is required; dhT, h0, g may be NULL.
 * dg must be non-NULL exactly when g is; dh0 may be NULL. */
int oracle_bwd(int B, int T, int H, int Dk, int Dv, int N, const int32_t *cu_seqlens,
               const double *q, const double *k, const double *v, const double *beta,
               const double *g, const double *h0, const double *dO, const double *dhT,
               double *dq, double *dk, double *dv, double *dbeta, double *dg, double *dh0,
               int nthreads)
{
    dims_t d = {B, T, H, Dk, Dv, N, cu_seqlens};
    if (B <= 0 || T < 0 || H <= 0 || Dk <= 0 || Dv <= 0 || N <= 0) return 1;
    if (cu_seqlens && B != 1) return 1;
    if (!cu_seqlens && N != B) return 1;
    if ((g == NULL) != (dg == NULL)) return 1;
    int pairs = N * H;
    int nt = n_threads(nthreads);
    size_t DD = (size_t)Dk * Dv;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
    for (int p = 0; p < pairs; ++p) {
        int n = p / H, h = p % H, b, t0, t1;
        seq_range(&d, n, &b, &t0, &t1);
        int L = t1 - t0;
        int nseg = (L + SEG - 1) / SEG;
        double *ckpt = (double *)malloc(sizeof(double) * DD * (nseg > 0 ? nseg : 1));
        double *seg = (double *)malloc(sizeof(double) * DD * (SEG + 1));
        double *G = (double *)malloc(sizeof(double) * DD);
        double *sk = (double *)malloc(sizeof(double) * (size_t)Dv);
        double *gk = (double *)malloc(sizeof(double) * (size_t)Dv);
        double *tmp = (double *)malloc(sizeof(double) * (size_t)Dk);
        if (!ckpt || !seg || !G || !sk || !gk || !tmp) {
#pragma omp atomic write
            err = 2;
            free(ckpt); free(seg); free(G); free(sk); free(gk); free(tmp);
            continue;
        }
        /* forward sweep: checkpoint the state entering every segment */
        double *S = seg; /* reuse slot 0 as the running state */
        load_state(S, h0 ? h0 + st_off(&d, n, h) : NULL, Dk, Dv);
        for (int t = t0; t < t1; ++t) {
            if ((t - t0) % SEG == 0) memcpy(ckpt + DD * ((t - t0) / SEG), S, sizeof(double) * DD);
            size_t s = sc_off(&d, b, t, h);
            step(S, Dk, Dv, k + tok_off(&d, b, t, h, Dk), v + tok_off(&d, b, t, h, Dv),
                 beta[s], g ? exp(g[s]) : 1.0, sk);
        }
        /* G = dL/dS_T = dhT^T */
        load_state(G, dhT ? dhT + st_off(&d, n, h) : NULL, Dk, Dv);
        for (int sgi = nseg - 1; sgi >= 0; --sgi) {
            int start = t0 + sgi * SEG;
            int len = (t1 - start) < SEG ? (t1 - start) : SEG;
            memcpy(seg, ckpt + DD * sgi, sizeof(double) * DD);
            for (int r = 0; r < len; ++r) {
                int t = start + r;
                size_t s = sc_off(&d, b, t, h);
                memcpy(seg + DD * (r + 1), seg + DD * r, sizeof(double) * DD);
                step(seg + DD * (r + 1), Dk, Dv, k + tok_off(&d, b, t, h, Dk),
                     v + tok_off(&d, b, t, h, Dv), beta[s], g ? exp(g[s]) : 1.0, sk);
            }
            for (int r = len - 1; r >= 0; --r) {
                int t = start + r;
                size_t s = sc_off(&d, b, t, h);
                const double *Sp = seg + DD * r;       /* S_{t-1} */
                const double *Sc = seg + DD * (r + 1); /* S_t     */
                const double *qt = q + tok_off(&d, b, t, h, Dk);
                const double *kt = k + tok_off(&d, b, t, h, Dk);
                const double *vt = v + tok_off(&d, b, t, h, Dv);
                const double *dot = dO + tok_off(&d, b, t, h, Dv);
                double alpha = g ? exp(g[s]) : 1.0, bt = beta[s];
                /* o_t = S_t q_t */
                for (int i = 0; i < Dv; ++i)
                    for (int j = 0; j < Dk; ++j) G[(size_t)i * Dk + j] += dot[i] * qt[j];
                double *dqt = dq + tok_off(&d, b, t, h, Dk);
                for (int j = 0; j < Dk; ++j) {
                    double acc = 0.0;
                    for (int i = 0; i < Dv; ++i) acc += Sc[(size_t)i * Dk + j] * dot[i];
                    dqt[j] = acc;
                }
                /* S_t = alpha S_{t-1} M + beta v k^T */
                for (int i = 0; i < Dv; ++i) {
                    double a1 = 0.0, a2 = 0.0;
                    for (int j = 0; j < Dk; ++j) {
                        a1 += Sp[(size_t)i * Dk + j] * kt[j];
                        a2 += G[(size_t)i * Dk + j] * kt[j];
                    }
                    sk[i] = a1;
                    gk[i] = a2;
                }
                double gs = 0.0, gksk = 0.0, db = 0.0;
                for (size_t e = 0; e < DD; ++e) gs += G[e] * Sp[e];
                for (int i = 0; i < Dv; ++i) {
                    gksk += gk[i] * sk[i];
                    db += (vt[i] - alpha * sk[i]) * gk[i];
                }
                if (dg) dg[s] = alpha * (gs - bt * gksk);
                dbeta[s] = db;
                double *dvt = dv + tok_off(&d, b, t, h, Dv);
                for (int i = 0; i < Dv; ++i) dvt[i] = bt * gk[i];
                /* dk = -alpha beta (S^T G k + G^T S k) + beta G^T v */
                double *dkt = dk + tok_off(&d, b, t, h, Dk);
                for (int j = 0; j < Dk; ++j) {
                    double a1 = 0.0, a2 = 0.0, a3 = 0.0;
                    for (int i = 0; i < Dv; ++i) {
                        a1 += Sp[(size_t)i * Dk + j] * gk[i];
                        a2 += G[(size_t)i * Dk + j] * sk[i];
                        a3 += G[(size_t)i * Dk + j] * vt[i];
                    }
                    tmp[j] = -alpha * bt * (a1 + a2) + bt * a3;
                }
                memcpy(dkt, tmp, sizeof(double) * (size_t)Dk);
                /* G <- alpha G (I - beta k k^T) */
                for (int i = 0; i < Dv; ++i)
                    for (int j = 0; j < Dk; ++j) {
                        double gv = G[(size_t)i * Dk + j];
                        G[(size_t)i * Dk + j] = alpha * (gv - bt * gk[i] * kt[j]);
                    }
            }
        }
        if (dh0) store_state(dh0 + st_off(&d, n, h), G, Dk, Dv);
        free(ckpt); free(seg); free(G); free(sk); free(gk); free(tmp);
    }
    return err;
}

/* One recurrent step per (b, h): q, k [B,H,Dk], v, o [B,H,Dv],
 * beta, g [B,H] (g may be NULL), state [B,H,Dk,Dv] = S^T, updated in place. */
int oracle_step(int B, int H, int Dk, int Dv, const double *q, const double *k,
                const double *v, const double *beta, const double *g, double *state,
                double *o, int nthreads)
{
    if (B <= 0 || H <= 0 || Dk <= 0 || Dv <= 0) return 1;
    int pairs = B * H;
    int nt = n_threads(nthreads);
    size_t DD = (size_t)Dk * Dv;
    int err = 0;
#pragma omp parallel for schedule(static) num_threads(nt)
    for (int p = 0; p < pairs; ++p) {
        double *S = (double *)malloc(sizeof(double) * DD);
        double *sk = (double *)malloc(sizeof(double) * (size_t)Dv);
        if (!S || !sk) {
#pragma omp atomic write
            err = 2;
            free(S);
            free(sk);
            continue;
        }
        load_state(S, state + DD * p, Dk, Dv);
        double alpha = g ? exp(g[p]) : 1.0;
        step(S, Dk, Dv, k + (size_t)p * Dk, v + (size_t)p * Dv, beta[p], alpha, sk);
        const double *qt = q + (size_t)p * Dk;
        for (int i = 0; i < Dv; ++i) {
            double acc = 0.0;
            for (int j = 0; j < Dk; ++j) acc += S[(size_t)i * Dk + j] * qt[j];
            o[(size_t)p * Dv + i] = acc;
        }
        store_state(state + DD * p, S, Dk, Dv);
        free(S);
        free(sk);
    }
    return err;
}
