/* Host driver for the fp64 oracles, built with AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_sanitize_cpu.py): runs both
 * oracles over shapes that reach their edge cases (T = 0, one step, a
 * ragged replay stretch, N = 1, no (b,h)) and checks statuses and that
 * every output is finite. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int wkv7_oracle_forward(const double *, const double *, const double *, const double *, const double *,
                        const double *, const double *, double *, double *, int64_t, int64_t, int64_t,
                        int64_t, int);
int wkv7_oracle_backward(const double *, const double *, const double *, const double *, const double *,
                         const double *, const double *, const double *, const double *, double *,
                         double *, double *, double *, double *, double *, double *, int64_t, int64_t,
                         int64_t, int64_t, int);
int rwkv8_oracle_forward(const double *, const double *, const double *, const double *, const double *,
                         double *, double *, double *, int64_t, int64_t, int64_t, int64_t, int64_t,
                         int64_t, int);
int rwkv8_oracle_backward(const double *, const double *, const double *, const double *, const double *,
                          const double *, const double *, const double *, double *, double *, double *,
                          double *, double *, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, int);

static int fails;
#define CHECK(c) do { if (!(c)) { fprintf(stderr, "CHECK failed line %d: %s\n", __LINE__, #c); fails++; } } while (0)

static double *rnd(size_t n, double lo, double hi)
{
    double *p = malloc((n ? n : 1) * sizeof(double));
    for (size_t i = 0; i < n; i++) p[i] = lo + (hi - lo) * (rand() / (double)RAND_MAX);
    return p;
}

static int finite(const double *p, size_t n)
{
    for (size_t i = 0; i < n; i++)
        if (!isfinite(p[i])) return 0;
    return 1;
}

static void wkv7_case(int64_t B, int64_t T, int64_t H, int64_t N)
{
    const size_t nv = (size_t)(B * T * H * N), ns = (size_t)(B * H * N * N);
    double *r = rnd(nv, -1, 1), *w = rnd(nv, 0.5, 1), *k = rnd(nv, -1, 1), *v = rnd(nv, -1, 1);
    double *a = rnd(nv, -0.3, 0.3), *b = rnd(nv, -0.3, 0.3), *dy = rnd(nv, -1, 1);
    double *s0 = rnd(ns, -1, 1), *dsT = rnd(ns, -1, 1);
    double *y = rnd(nv, 0, 0), *sT = rnd(ns, 0, 0), *ds0 = rnd(ns, 0, 0);
    double *g[6];
    for (int i = 0; i < 6; i++) g[i] = rnd(nv, 0, 0);
    CHECK(wkv7_oracle_forward(r, w, k, v, a, b, s0, y, sT, B, T, H, N, 3) == 0);
    CHECK(wkv7_oracle_backward(r, w, k, v, a, b, dy, s0, dsT, g[0], g[1], g[2], g[3], g[4], g[5], ds0, B, T,
                               H, N, 3) == 0);
    CHECK(wkv7_oracle_backward(r, w, k, v, a, b, dy, NULL, NULL, g[0], g[1], g[2], g[3], g[4], g[5], NULL, B,
                               T, H, N, 2) == 0);
    CHECK(finite(y, nv) && finite(sT, ns) && finite(ds0, ns));
    for (int i = 0; i < 6; i++) CHECK(finite(g[i], nv));
    free(r); free(w); free(k); free(v); free(a); free(b); free(dy); free(s0); free(dsT);
    free(y); free(sT); free(ds0);
    for (int i = 0; i < 6; i++) free(g[i]);
}

static void rwkv8_case(int64_t B, int64_t T, int64_t H, int64_t Hv, int64_t L, int64_t E)
{
    const size_t nq = (size_t)(B * H * T * L), nv = (size_t)(B * Hv * T * E), ny = (size_t)(B * H * T * E);
    const size_t nr = (size_t)(B * H * L * E), nn = (size_t)(B * H * L);
    double *q = rnd(nq, 0, 1), *v = rnd(nv, -1, 1), *d = rnd((size_t)(H * L), 0.5, 1), *dy = rnd(ny, -1, 1);
    double *R0 = rnd(nr, -1, 1), *n0 = rnd(nn, 0.5, 2), *dRT = rnd(nr, -1, 1), *dnT = rnd(nn, -1, 1);
    double *y = rnd(ny, 0, 0), *RT = rnd(nr, 0, 0), *nT = rnd(nn, 0, 0);
    double *dq = rnd(nq, 0, 0), *dv = rnd(ny, 0, 0), *dd = rnd(nn, 0, 0), *dR0 = rnd(nr, 0, 0), *dn0 = rnd(nn, 0, 0);
    CHECK(rwkv8_oracle_forward(q, v, d, R0, n0, y, RT, nT, B, T, H, Hv, L, E, 3) == 0);
    CHECK(rwkv8_oracle_backward(q, v, d, R0, n0, dy, dRT, dnT, dq, dv, dd, dR0, dn0, B, T, H, Hv, L, E, 3) == 0);
    CHECK(rwkv8_oracle_backward(q, v, d, NULL, NULL, dy, NULL, NULL, dq, dv, dd, NULL, NULL, B, T, H, Hv, L, E,
                                2) == 0);
    CHECK(finite(y, ny) && finite(RT, nr) && finite(nT, nn) && finite(dq, nq) && finite(dv, ny));
    CHECK(finite(dd, nn) && finite(dR0, nr) && finite(dn0, nn));
    free(q); free(v); free(d); free(dy); free(R0); free(n0); free(dRT); free(dnT);
    free(y); free(RT); free(nT); free(dq); free(dv); free(dd); free(dR0); free(dn0);
}

int main(void)
{
    srand(1);
    wkv7_case(2, 0, 3, 4);
    wkv7_case(1, 1, 2, 5);
    wkv7_case(2, 130, 2, 3);
    wkv7_case(1, 9, 1, 1);
    wkv7_case(0, 7, 2, 4);
    rwkv8_case(2, 0, 3, 3, 4, 5);
    rwkv8_case(1, 1, 2, 2, 3, 2);
    rwkv8_case(2, 131, 3, 1, 3, 4);
    rwkv8_case(1, 65, 2, 2, 1, 1);
    CHECK(wkv7_oracle_forward(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, -1, 1, 1, 1, 1) == -2);
    CHECK(rwkv8_oracle_forward(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1, 1, 3, 2, 1, 1, 1) == -2);
    printf("oracle driver: %d failures\n", fails);
    return fails == 0 ? 0 : 1;
}
