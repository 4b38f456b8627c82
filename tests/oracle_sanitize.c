/* Driver that runs the C oracle under AddressSanitizer and UndefinedBehaviorSanitizer
 * (tests/test_oracle_sanitizers.py builds and runs it; test infrastructure only).
 *
 * Over shapes with edge cases (one token, ragged lengths, several groups, no skip term,
 * no initial state, an empty sequence) it checks that every output is finite, that a
 * prefill equals the same tokens run one decode step at a time bit for bit (both apply the
 * same per-token update), and that invalid arguments are refused.  Exit status 0 = pass. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int ssd_oracle_prefill(const double *x, const double *dt, const double *A, const double *Bm, const double *Cm,
                       const double *D, const double *h0, double *y, double *hT, int batch, int seqlen, int nheads,
                       int headdim, int dstate, int ngroups, int nthreads);
int ssd_oracle_step(double *state, const double *x, const double *dt, const double *A, const double *Bm,
                    const double *Cm, const double *D, double *y, int batch, int nheads, int headdim, int dstate,
                    int ngroups, int nthreads);

static unsigned long long rng = 88172645463325252ull;
static double unif(void)
{
    rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
    return (double)(rng >> 11) / 9007199254740992.0;
}
static double *fill(size_t n, double lo, double hi)
{
    double *p = malloc((n ? n : 1) * sizeof(double));
    for (size_t i = 0; i < n; ++i) p[i] = lo + (hi - lo) * unif();
    return p;
}

static int run(int B, int L, int H, int P, int N, int G, int with_D, int with_h0)
{
    const size_t nx = (size_t)B * L * H * P, ndt = (size_t)B * L * H, nbc = (size_t)B * L * G * N;
    const size_t ns = (size_t)B * H * P * N;
    double *x = fill(nx, -1, 1), *dt = fill(ndt, 0.001, 0.1), *Bm = fill(nbc, -0.3, 0.3), *Cm = fill(nbc, -0.3, 0.3);
    double *A = fill(H, -4, -0.5), *D = with_D ? fill(H, -1, 1) : NULL, *h0 = with_h0 ? fill(ns, -0.1, 0.1) : NULL;
    double *y = fill(nx, 0, 0), *hT = fill(ns, 0, 0);
    int bad = 0;
    if (ssd_oracle_prefill(x, dt, A, Bm, Cm, D, h0, y, hT, B, L, H, P, N, G, 0) != 0) bad = 1;
    for (size_t i = 0; i < nx && !bad; ++i) bad = !isfinite(y[i]);
    for (size_t i = 0; i < ns && !bad; ++i) bad = !isfinite(hT[i]);
    /* the same tokens one decode step at a time */
    double *st = fill(ns, 0, 0), *yt = fill((size_t)B * H * P, 0, 0);
    if (h0) memcpy(st, h0, ns * sizeof(double));
    double *xt = fill((size_t)B * H * P, 0, 0), *dtt = fill((size_t)B * H, 0, 0);
    double *bt = fill((size_t)B * G * N, 0, 0), *ct = fill((size_t)B * G * N, 0, 0);
    for (int t = 0; t < L && !bad; ++t) {
        for (int b = 0; b < B; ++b) {
            memcpy(xt + (size_t)b * H * P, x + ((size_t)b * L + t) * H * P, (size_t)H * P * sizeof(double));
            memcpy(dtt + (size_t)b * H, dt + ((size_t)b * L + t) * H, (size_t)H * sizeof(double));
            memcpy(bt + (size_t)b * G * N, Bm + ((size_t)b * L + t) * G * N, (size_t)G * N * sizeof(double));
            memcpy(ct + (size_t)b * G * N, Cm + ((size_t)b * L + t) * G * N, (size_t)G * N * sizeof(double));
        }
        if (ssd_oracle_step(st, xt, dtt, A, bt, ct, D, yt, B, H, P, N, G, 0) != 0) bad = 2;
        for (int b = 0; b < B && !bad; ++b)
            if (memcmp(yt + (size_t)b * H * P, y + ((size_t)b * L + t) * H * P, (size_t)H * P * sizeof(double)))
                bad = 3;
    }
    if (!bad && memcmp(st, hT, ns * sizeof(double))) bad = 4;
    free(x); free(dt); free(Bm); free(Cm); free(A); free(D); free(h0); free(y); free(hT);
    free(st); free(yt); free(xt); free(dtt); free(bt); free(ct);
    if (bad) printf("FAIL (%d) B=%d L=%d H=%d P=%d N=%d G=%d D=%d h0=%d\n", bad, B, L, H, P, N, G, with_D, with_h0);
    return bad;
}

int main(void)
{
    int fails = 0;
    fails += run(1, 1, 1, 1, 1, 1, 1, 1) != 0;
    fails += run(2, 7, 3, 5, 4, 1, 1, 0) != 0;
    fails += run(1, 33, 4, 8, 6, 2, 0, 1) != 0;
    fails += run(3, 17, 6, 4, 3, 3, 1, 1) != 0;
    fails += run(1, 0, 2, 4, 4, 1, 1, 1) != 0;   /* empty sequence: the final state is the initial one */
    /* invalid arguments are refused, nothing is read */
    double a = -1.0, v = 0.0;
    if (ssd_oracle_prefill(&v, &v, &a, &v, &v, NULL, NULL, &v, NULL, 1, 1, 3, 1, 1, 2, 0) == 0) ++fails;  /* H % G */
    if (ssd_oracle_prefill(NULL, &v, &a, &v, &v, NULL, NULL, &v, NULL, 1, 1, 1, 1, 1, 1, 0) == 0) ++fails;
    if (ssd_oracle_step(NULL, &v, &v, &a, &v, &v, NULL, &v, 1, 1, 1, 1, 1, 0) == 0) ++fails;
    if (ssd_oracle_prefill(&v, &v, &a, &v, &v, NULL, NULL, &v, NULL, 0, 1, 1, 1, 1, 1, 0) == 0) ++fails;
    printf(fails ? "sanitized oracle: %d failures\n" : "sanitized oracle: ok\n", fails);
    return fails ? 1 : 0;
}
