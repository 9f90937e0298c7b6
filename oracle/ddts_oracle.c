/*
 * ddts_oracle.c -- fp64 CPU oracle for the DDTS gated linear-attention
 * recurrence of Rodimus.  TEST INFRASTRUCTURE ONLY: it exists to check the
 * HIP kernels and is never part of the product path.  It shares no code,
 * header, table or helper with the GPU library.
 *
 * What it computes (the plain definition, token by token, per head):
 *   alpha_t     = exp(-g_t * tau_t)                 elementwise over dk
 *   alpha_hat_t = g_t ^ tau_t                        elementwise over dk
 *   k'_t        = alpha_hat_t * k_t                  (dk)
 *   v'_t        = beta_hat_t * v_t                   (dv)
 *   S_t         = diag(alpha_t) S_{t-1} + k'_t v'_t^T   (dk x dv)
 *   o_t         = S_t^T q_t                          (dv)
 *
 * Sources:
 *  - the two gate formulas: "Rodimus*" digest (digest.lyk-ai.com), section
 *    "Method", bullet on the selection gate g_t and temperature gate tau_t;
 *  - beta_hat as the low-rank gate acting on the value side: same digest,
 *    section "Method", the low-rank bullet;
 *  - selection only along n (= dk, the state rows): the authors' OpenReview
 *    rebuttal (paperhub.cn), answer to "technical contribution is limited",
 *    bullet "Efficient Parallelization";
 *  - the state is n x m per head, rows along the expansion factor n: the same
 *    rebuttal's answer on the "State size n x m" column of Table 4;
 *  - the pages do not print the recurrence's body (their Eq. 11 is only
 *    referenced).  Reading taken: the state update is applied first and the
 *    readout uses the updated state, so o_t includes the current token, and
 *    q is not rescaled inside the operation.
 *  pow() follows IEEE semantics: 0^tau = 0 for tau > 0 and x^0 = 1.
 *
 * Layouts (all row-major, contiguous):
 *   q, k, g, tau : [B, T, H, dk]      v, beta_hat : [B, T, H, dv]
 *   S0, S_final  : [B, H, dk, dv]     out         : [B, T, H, dv]
 *
 * Parallelism: independent (b, h) pairs are spread over POSIX threads.
 * The arithmetic of one pair never depends on the thread count.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fPIC -shared -pthread -lm
 * (no fast-math; no FMA contraction, so every product is rounded once).
 */
#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

typedef struct {
    int B, T, H, dk, dv;
    const double *q, *k, *g, *tau, *v, *beta_hat, *S0;
    double *out, *S_final;
    int next_pair;          /* shared work counter, guarded by lock */
    pthread_mutex_t lock;
} fwd_job;

/* One (b, h) pair: the recurrence above, token by token. */
static void fwd_pair(const fwd_job *J, int b, int h, double *S, double *a,
                     double *kk, double *vv)
{
    const int T = J->T, H = J->H, dk = J->dk, dv = J->dv;
    if (J->S0)
        memcpy(S, J->S0 + ((size_t)b * H + h) * dk * dv, sizeof(double) * dk * dv);
    else
        memset(S, 0, sizeof(double) * dk * dv);

    for (int t = 0; t < T; ++t) {
        const size_t rk = (((size_t)b * T + t) * H + h) * dk;
        const size_t rv = (((size_t)b * T + t) * H + h) * dv;
        /* gates along dk: forget alpha and input alpha_hat */
        for (int i = 0; i < dk; ++i) {
            const double gi = J->g[rk + i], ti = J->tau[rk + i];
            a[i] = exp(-gi * ti);
            kk[i] = pow(gi, ti) * J->k[rk + i];
        }
        /* value-side gate beta_hat */
        for (int j = 0; j < dv; ++j)
            vv[j] = J->beta_hat[rv + j] * J->v[rv + j];
        /* S <- diag(alpha) S + k' v'^T */
        for (int i = 0; i < dk; ++i) {
            double *Si = S + (size_t)i * dv;
            for (int j = 0; j < dv; ++j)
                Si[j] = a[i] * Si[j] + kk[i] * vv[j];
        }
        /* o_t = S_t^T q_t, summed over i in ascending order */
        double *o = J->out + rv;
        for (int j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int i = 0; i < dk; ++i)
                acc += J->q[rk + i] * S[(size_t)i * dv + j];
            o[j] = acc;
        }
    }
    if (J->S_final)
        memcpy(J->S_final + ((size_t)b * H + h) * dk * dv, S, sizeof(double) * dk * dv);
}

static void *fwd_worker(void *arg)
{
    fwd_job *J = (fwd_job *)arg;
    double *S = malloc(sizeof(double) * (size_t)J->dk * J->dv);
    double *a = malloc(sizeof(double) * J->dk);
    double *kk = malloc(sizeof(double) * J->dk);
    double *vv = malloc(sizeof(double) * J->dv);
    if (!S || !a || !kk || !vv) {
        free(S); free(a); free(kk); free(vv);
        return (void *)1;
    }
    for (;;) {
        pthread_mutex_lock(&J->lock);
        const int p = J->next_pair++;
        pthread_mutex_unlock(&J->lock);
        if (p >= J->B * J->H) break;
        fwd_pair(J, p / J->H, p % J->H, S, a, kk, vv);
    }
    free(S); free(a); free(kk); free(vv);
    return NULL;
}

static int resolve_threads(int nthreads, int work)
{
    if (nthreads <= 0) {
        long n = sysconf(_SC_NPROCESSORS_ONLN);
        nthreads = n > 0 ? (int)n : 1;
    }
    if (nthreads > work) nthreads = work;
    if (nthreads < 1) nthreads = 1;
    return nthreads;
}

/* Forward over whole sequences.  S0 and S_final may be NULL.  Returns the
 * number of threads used, or -1 on bad arguments / allocation failure. */
int ddts_oracle_fwd(int B, int T, int H, int dk, int dv,
                    const double *q, const double *k, const double *g,
                    const double *tau, const double *v, const double *beta_hat,
                    const double *S0, double *out, double *S_final, int nthreads)
{
    if (B <= 0 || T < 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
    if (!q || !k || !g || !tau || !v || !beta_hat || !out) return -1;
    fwd_job J = {B, T, H, dk, dv, q, k, g, tau, v, beta_hat, S0, out, S_final, 0};
    pthread_mutex_init(&J.lock, NULL);
    const int nt = resolve_threads(nthreads, B * H);
    pthread_t *th = malloc(sizeof(pthread_t) * nt);
    if (!th) return -1;
    int failed = 0;
    for (int i = 0; i < nt; ++i)
        if (pthread_create(&th[i], NULL, fwd_worker, &J) != 0) { failed = 1; th[i] = 0; }
    for (int i = 0; i < nt; ++i) {
        void *rc = NULL;
        if (th[i]) { pthread_join(th[i], &rc); if (rc) failed = 1; }
    }
    free(th);
    pthread_mutex_destroy(&J.lock);
    return failed ? -1 : nt;
}

/* One recurrent step for N independent sequences: the same update applied to
 * a resident state, in place.  Layouts: q,k,g,tau [N,H,dk]; v,beta_hat
 * [N,H,dv]; state [N,H,dk,dv]; out [N,H,dv].  This is ddts_oracle_fwd with
 * T = 1 and S_final aliasing S0, written out on its own. */
int ddts_oracle_decode(int N, int H, int dk, int dv,
                       const double *q, const double *k, const double *g,
                       const double *tau, const double *v, const double *beta_hat,
                       double *state, double *out)
{
    if (N <= 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
    if (!q || !k || !g || !tau || !v || !beta_hat || !state || !out) return -1;
    double *a = malloc(sizeof(double) * dk);
    double *kk = malloc(sizeof(double) * dk);
    double *vv = malloc(sizeof(double) * dv);
    if (!a || !kk || !vv) { free(a); free(kk); free(vv); return -1; }
    for (int p = 0; p < N * H; ++p) {
        const size_t rk = (size_t)p * dk, rv = (size_t)p * dv;
        double *S = state + (size_t)p * dk * dv;
        for (int i = 0; i < dk; ++i) {
            a[i] = exp(-g[rk + i] * tau[rk + i]);
            kk[i] = pow(g[rk + i], tau[rk + i]) * k[rk + i];
        }
        for (int j = 0; j < dv; ++j)
            vv[j] = beta_hat[rv + j] * v[rv + j];
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j)
                S[(size_t)i * dv + j] = a[i] * S[(size_t)i * dv + j] + kk[i] * vv[j];
        for (int j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int i = 0; i < dk; ++i)
                acc += q[rk + i] * S[(size_t)i * dv + j];
            out[rv + j] = acc;
        }
    }
    free(a); free(kk); free(vv);
    return 1;
}

/* ------------------------------------------------------------------------
 * Backward (reverse mode) of the forward above, written out directly from
 * the recurrence: with D the adjoint of the state (dL/dS_t, dk x dv),
 * walking t = T .. 1,
 *   D      += q_t dO_t^T                 (o_t = S_t^T q_t)
 *   dq_t    = S_t dO_t
 *   dk'_t   = D v'_t,   dv'_t = D^T k'_t
 *   dalpha_t[i] = sum_j D[i][j] S_{t-1}[i][j]
 *   D       = diag(alpha_t) D            (S_t = diag(alpha_t) S_{t-1} + ...)
 * and dS_0 = D after t = 1, D starting from dL/dS_T (or zero).  Then the
 * gate chain rule: dk = alpha_hat dk', dalpha_hat = k dk', dv = beta_hat
 * dv', dbeta_hat = v dv', and with alpha = exp(-g tau), alpha_hat = g^tau:
 *   dg   = -tau alpha dalpha + tau g^(tau-1) dalpha_hat
 *   dtau = -g   alpha dalpha + ln(g) g^tau   dalpha_hat.
 * Reading at g = 0 (where g^tau is not differentiable): the alpha_hat terms
 * are taken as 0 there.  S_{t-1} comes from checkpoints every CK tokens and
 * a forward recomputation of each segment.
 * ------------------------------------------------------------------------ */
#define CK 64

typedef struct {
    int B, T, H, dk, dv;
    const double *q, *k, *g, *tau, *v, *beta_hat, *S0, *dout, *dSf;
    double *dq, *dk_, *dg, *dtau, *dv_, *dbeta, *dS0;
    int next_pair;
    pthread_mutex_t lock;
} bwd_job;

static void gates(const bwd_job *J, size_t rk, size_t rv, double *a, double *ah, double *kk,
                  double *vv)
{
    for (int i = 0; i < J->dk; ++i) {
        const double gi = J->g[rk + i], ti = J->tau[rk + i];
        a[i] = exp(-gi * ti);
        ah[i] = pow(gi, ti);
        kk[i] = ah[i] * J->k[rk + i];
    }
    for (int j = 0; j < J->dv; ++j)
        vv[j] = J->beta_hat[rv + j] * J->v[rv + j];
}

static void step(int dk, int dv, const double *a, const double *kk, const double *vv,
                 const double *Sprev, double *S)
{
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j)
            S[(size_t)i * dv + j] = a[i] * Sprev[(size_t)i * dv + j] + kk[i] * vv[j];
}

/* work arrays: cp (ncp states), seg (CK + 1 states), D (one state), vectors */
static void bwd_pair(const bwd_job *J, int b, int h, double *cp, double *seg, double *D,
                     double *a, double *ah, double *kk, double *vv, double *dkk, double *dvv,
                     double *da)
{
    const int T = J->T, H = J->H, dk = J->dk, dv = J->dv;
    const size_t SZ = (size_t)dk * dv;
    /* forward pass keeping the state before every CK-th token */
    double *S = seg;                                   /* scratch for the sweep */
    if (J->S0)
        memcpy(S, J->S0 + ((size_t)b * H + h) * SZ, sizeof(double) * SZ);
    else
        memset(S, 0, sizeof(double) * SZ);
    for (int t = 0; t < T; ++t) {
        if (t % CK == 0) memcpy(cp + (size_t)(t / CK) * SZ, S, sizeof(double) * SZ);
        const size_t rk = (((size_t)b * T + t) * H + h) * dk;
        const size_t rv = (((size_t)b * T + t) * H + h) * dv;
        gates(J, rk, rv, a, ah, kk, vv);
        step(dk, dv, a, kk, vv, S, S);
    }
    /* reverse pass */
    if (J->dSf)
        memcpy(D, J->dSf + ((size_t)b * H + h) * SZ, sizeof(double) * SZ);
    else
        memset(D, 0, sizeof(double) * SZ);
    const int nseg = (T + CK - 1) / CK;
    for (int s = nseg - 1; s >= 0; --s) {
        const int t0 = s * CK, t1 = t0 + CK < T ? t0 + CK : T;
        /* seg[u] = state before token t0 + u, u = 0 .. t1 - t0 */
        memcpy(seg, cp + (size_t)s * SZ, sizeof(double) * SZ);
        for (int t = t0; t < t1; ++t) {
            const size_t rk = (((size_t)b * T + t) * H + h) * dk;
            const size_t rv = (((size_t)b * T + t) * H + h) * dv;
            gates(J, rk, rv, a, ah, kk, vv);
            step(dk, dv, a, kk, vv, seg + (size_t)(t - t0) * SZ, seg + (size_t)(t - t0 + 1) * SZ);
        }
        for (int t = t1 - 1; t >= t0; --t) {
            const size_t rk = (((size_t)b * T + t) * H + h) * dk;
            const size_t rv = (((size_t)b * T + t) * H + h) * dv;
            const double *St = seg + (size_t)(t - t0 + 1) * SZ, *Sp = seg + (size_t)(t - t0) * SZ;
            const double *qt = J->q + rk, *dot = J->dout + rv;
            gates(J, rk, rv, a, ah, kk, vv);
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j)
                    D[(size_t)i * dv + j] += qt[i] * dot[j];
            for (int i = 0; i < dk; ++i) {
                double acc = 0.0;
                for (int j = 0; j < dv; ++j) acc += St[(size_t)i * dv + j] * dot[j];
                J->dq[rk + i] = acc;
            }
            for (int i = 0; i < dk; ++i) {
                double acc = 0.0, accs = 0.0;
                for (int j = 0; j < dv; ++j) {
                    acc += D[(size_t)i * dv + j] * vv[j];
                    accs += D[(size_t)i * dv + j] * Sp[(size_t)i * dv + j];
                }
                dkk[i] = acc;
                da[i] = accs;
            }
            for (int j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int i = 0; i < dk; ++i) acc += D[(size_t)i * dv + j] * kk[i];
                dvv[j] = acc;
            }
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j)
                    D[(size_t)i * dv + j] *= a[i];
            for (int i = 0; i < dk; ++i) {
                const double gi = J->g[rk + i], ti = J->tau[rk + i];
                const double dah = J->k[rk + i] * dkk[i];
                J->dk_[rk + i] = ah[i] * dkk[i];
                double dgi = -ti * a[i] * da[i], dti = -gi * a[i] * da[i];
                if (gi > 0.0) {
                    dgi += ti * pow(gi, ti - 1.0) * dah;
                    dti += log(gi) * ah[i] * dah;
                }
                J->dg[rk + i] = dgi;
                J->dtau[rk + i] = dti;
            }
            for (int j = 0; j < dv; ++j) {
                J->dv_[rv + j] = J->beta_hat[rv + j] * dvv[j];
                J->dbeta[rv + j] = J->v[rv + j] * dvv[j];
            }
        }
    }
    if (J->dS0) memcpy(J->dS0 + ((size_t)b * H + h) * SZ, D, sizeof(double) * SZ);
}

static void *bwd_worker(void *arg)
{
    bwd_job *J = (bwd_job *)arg;
    const size_t SZ = (size_t)J->dk * J->dv;
    const int ncp = J->T > 0 ? (J->T + CK - 1) / CK : 1;
    double *cp = malloc(sizeof(double) * SZ * ncp);
    double *seg = malloc(sizeof(double) * SZ * (CK + 1));
    double *D = malloc(sizeof(double) * SZ);
    double *vec = malloc(sizeof(double) * (5 * (size_t)J->dk + 2 * (size_t)J->dv));
    if (!cp || !seg || !D || !vec) {
        free(cp); free(seg); free(D); free(vec);
        return (void *)1;
    }
    double *a = vec, *ah = a + J->dk, *kk = ah + J->dk, *dkk = kk + J->dk, *da = dkk + J->dk;
    double *vv = da + J->dk, *dvv = vv + J->dv;
    for (;;) {
        pthread_mutex_lock(&J->lock);
        const int p = J->next_pair++;
        pthread_mutex_unlock(&J->lock);
        if (p >= J->B * J->H) break;
        bwd_pair(J, p / J->H, p % J->H, cp, seg, D, a, ah, kk, vv, dkk, dvv, da);
    }
    free(cp); free(seg); free(D); free(vec);
    return NULL;
}

/* Gradients of L w.r.t. every input, given dL/dout [B,T,H,dv] and optionally
 * dL/dS_T [B,H,dk,dv] (NULL = 0).  Outputs have the inputs' shapes; dS0 may be
 * NULL.  Returns the number of threads used, or -1. */
int ddts_oracle_bwd(int B, int T, int H, int dk, int dv,
                    const double *q, const double *k, const double *g,
                    const double *tau, const double *v, const double *beta_hat,
                    const double *S0, const double *dout, const double *dSf,
                    double *dq, double *dk_, double *dg, double *dtau, double *dv_,
                    double *dbeta, double *dS0, int nthreads)
{
    if (B <= 0 || T < 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
    if (!q || !k || !g || !tau || !v || !beta_hat || !dout) return -1;
    if (!dq || !dk_ || !dg || !dtau || !dv_ || !dbeta) return -1;
    bwd_job J = {B, T, H, dk, dv, q, k, g, tau, v, beta_hat, S0, dout, dSf,
                 dq, dk_, dg, dtau, dv_, dbeta, dS0, 0};
    pthread_mutex_init(&J.lock, NULL);
    const int nt = resolve_threads(nthreads, B * H);
    pthread_t *th = malloc(sizeof(pthread_t) * nt);
    if (!th) return -1;
    int failed = 0;
    for (int i = 0; i < nt; ++i)
        if (pthread_create(&th[i], NULL, bwd_worker, &J) != 0) { failed = 1; th[i] = 0; }
    for (int i = 0; i < nt; ++i) {
        void *rc = NULL;
        if (th[i]) { pthread_join(th[i], &rc); if (rc) failed = 1; }
    }
    free(th);
    pthread_mutex_destroy(&J.lock);
    return failed ? -1 : nt;
}
