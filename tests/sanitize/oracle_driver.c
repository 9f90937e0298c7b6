/*
 * oracle_driver.c -- runs the fp64 oracle's three entry points (forward,
 * decode step, reverse mode) on small seeded inputs of awkward shapes, for a
 * build with AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).
 * Exits 0 when every call returns success and every output is finite.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

int ddts_oracle_fwd(int B, int T, int H, int dk, int dv, const double *q, const double *k,
                    const double *g, const double *tau, const double *v, const double *beta_hat,
                    const double *S0, double *out, double *S_final, int nthreads);
int ddts_oracle_decode(int N, int H, int dk, int dv, const double *q, const double *k,
                       const double *g, const double *tau, const double *v,
                       const double *beta_hat, double *state, double *out);
int ddts_oracle_bwd(int B, int T, int H, int dk, int dv, const double *q, const double *k,
                    const double *g, const double *tau, const double *v, const double *beta_hat,
                    const double *S0, const double *d_out, const double *d_final_state,
                    double *dq, double *dk_, double *dg, double *dtau, double *dv_,
                    double *dbeta_hat, double *d_initial_state, int nthreads);

static unsigned long long rng = 88172645463325252ULL;
static double uni(void)                 /* xorshift64, in [0, 1) */
{
    rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
    return (double)(rng >> 11) / 9007199254740992.0;
}

static double *arr(size_t n, double lo, double hi)
{
    double *a = malloc((n ? n : 1) * sizeof(double));
    for (size_t i = 0; i < n; ++i) a[i] = lo + (hi - lo) * uni();
    return a;
}

static int finite_all(const double *a, size_t n)
{
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(a[i])) return 0;
    return 1;
}

static int run(int B, int T, int H, int dk, int dv, int threads, int with_s0)
{
    const size_t nk = (size_t)B * T * H * dk, nv = (size_t)B * T * H * dv, ns = (size_t)B * H * dk * dv;
    double *q = arr(nk, -1, 1), *k = arr(nk, -1, 1), *g = arr(nk, 0, 1), *tau = arr(nk, 0, 1);
    double *v = arr(nv, -1, 1), *bh = arr(nv, 0, 1), *s0 = with_s0 ? arr(ns, -1, 1) : NULL;
    double *out = arr(nv, 0, 0), *sf = arr(ns, 0, 0), *dout = arr(nv, -1, 1), *dsf = arr(ns, -1, 1);
    double *dq = arr(nk, 0, 0), *dkk = arr(nk, 0, 0), *dg = arr(nk, 0, 0), *dt = arr(nk, 0, 0);
    double *dvv = arr(nv, 0, 0), *db = arr(nv, 0, 0), *ds0 = arr(ns, 0, 0);
    int ok = ddts_oracle_fwd(B, T, H, dk, dv, q, k, g, tau, v, bh, s0, out, sf, threads) >= 0 &&
             finite_all(out, nv) && finite_all(sf, ns);
    ok = ok && ddts_oracle_bwd(B, T, H, dk, dv, q, k, g, tau, v, bh, s0, dout, dsf, dq, dkk, dg,
                               dt, dvv, db, ds0, threads) >= 0 &&
         finite_all(dq, nk) && finite_all(dg, nk) && finite_all(dvv, nv) && finite_all(ds0, ns);
    if (T >= 1) {
        /* one decode step over the first token of every sequence */
        const size_t pk = (size_t)B * H * dk, pv = (size_t)B * H * dv;
        double *st = arr(ns, -1, 1), *o = arr(pv, 0, 0);
        ok = ok && ddts_oracle_decode(B, H, dk, dv, q, k, g, tau, v, bh, st, o) >= 0 &&
             finite_all(o, pv) && finite_all(st, ns);
        (void)pk;
        free(st); free(o);
    }
    double *all[] = {q, k, g, tau, v, bh, s0, out, sf, dout, dsf, dq, dkk, dg, dt, dvv, db, ds0};
    for (size_t i = 0; i < sizeof(all) / sizeof(all[0]); ++i) free(all[i]);
    printf("B%d T%d H%d dk%d dv%d threads %d s0 %d: %s\n", B, T, H, dk, dv, threads, with_s0,
           ok ? "ok" : "FAILED");
    return ok;
}

int main(void)
{
    int ok = 1;
    ok &= run(1, 0, 1, 4, 4, 1, 1);
    ok &= run(1, 1, 1, 1, 1, 1, 0);
    ok &= run(2, 65, 3, 3, 5, 4, 1);
    ok &= run(1, 130, 2, 16, 16, 2, 0);
    ok &= run(3, 7, 5, 2, 9, 0, 1);
    return ok ? 0 : 1;
}
