/*
 * wkv7_oracle.c -- plain fp64 CPU oracle of the WKV7 (RWKV-7) recurrence and
 * of its reverse (backward-through-time) scan.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header or table with the
 * HIP library.
 *
 * What is computed (Foundry page "rwkvx/rx_pretrain.c", functions
 * rx_wkv7_forward_seq and rx_wkv7_backward, and the comment block that
 * states the three reverse-scan steps), restated for one (batch b, head h)
 * with state S[i][j] (i = value/output row, j = key/input column):
 *
 *   forward, t = 0 .. T-1, S starts at s0 (zeros when s0 is absent):
 *     sa[i]   = sum_j S[i][j] * a[j]                     (pre-update state)
 *     S[i][j] = S[i][j] * w[j] + v[i] * k[j] + sa[i] * b[j]
 *     y[i]    = sum_j S[i][j] * r[j]                     (post-update state)
 *   sT = S after the last step.
 *
 *   backward: G = dL/dS, seeded with dsT (zeros when absent -- the page seeds
 *   with zeros; a final-state gradient input is the extension the burn_mamba
 *   serial_recalculated backward.rs page makes with d_final_state), then for
 *   t = T-1 .. 0, with P = state before step t and St = state after it:
 *     (1) dr[j] = sum_i St[i][j] dy[i];          G[i][j] += dy[i] r[j]
 *     (2) dk[j] = sum_i G[i][j] v[i];  db[j] = sum_i G[i][j] sa[i]
 *         dw[j] = sum_i G[i][j] P[i][j]   (w is the multiplicative decay)
 *         dv[i] = sum_j G[i][j] k[j];  dsa[i] = sum_j G[i][j] b[j]
 *     (3) da[j] = sum_i dsa[i] P[i][j];  G[i][j] = G[i][j] w[j] + dsa[i] a[j]
 *   ds0 = G after t = 0.
 *
 * Layout: vectors [B][T][H][N], states [B][H][N][N] row-major, all fp64.
 * The backward caches every pre-step state of one (b,h) (T*N*N doubles), as
 * the page does; (b,h) pairs are independent and are spread over threads.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <pthread.h>

typedef struct {
    const double *r, *w, *k, *v, *a, *b, *dy, *s0, *dsT;
    double *y, *sT, *dr, *dw, *dk, *dv, *da, *db, *ds0;
    int64_t B, T, H, N;
    int64_t next;          /* next (b,h) unit to take */
    int failed;
    pthread_mutex_t lock;
} job_t;

static inline size_t vix(const job_t *J, int64_t b, int64_t t, int64_t h, int64_t n)
{
    return (size_t)(((b * J->T + t) * J->H + h) * J->N + n);
}

static inline size_t six(const job_t *J, int64_t b, int64_t h, int64_t i, int64_t j)
{
    return (size_t)(((b * J->H + h) * J->N + i) * J->N + j);
}

static int take_unit(job_t *J, int64_t *unit)
{
    pthread_mutex_lock(&J->lock);
    int ok = J->next < J->B * J->H && !J->failed;
    if (ok) *unit = J->next++;
    pthread_mutex_unlock(&J->lock);
    return ok;
}

static void fail(job_t *J)
{
    pthread_mutex_lock(&J->lock);
    J->failed = 1;
    pthread_mutex_unlock(&J->lock);
}

/* Load the initial state of (b,h) into S (N*N), zeros when s0 is absent. */
static void load_s0(const job_t *J, int64_t b, int64_t h, double *S)
{
    const int64_t N = J->N;
    for (int64_t i = 0; i < N; i++)
        for (int64_t j = 0; j < N; j++)
            S[i * N + j] = J->s0 ? J->s0[six(J, b, h, i, j)] : 0.0;
}

/* One forward step of (b,h) at time t, in place on S; writes sa (N) and,
 * when y_out is non-NULL, y (N values at y_out). */
static void step_forward(const job_t *J, int64_t b, int64_t t, int64_t h,
                         double *S, double *sa, double *y_out)
{
    const int64_t N = J->N;
    for (int64_t i = 0; i < N; i++) {
        double acc = 0.0;
        for (int64_t j = 0; j < N; j++)
            acc += S[i * N + j] * J->a[vix(J, b, t, h, j)];
        sa[i] = acc;
    }
    for (int64_t i = 0; i < N; i++) {
        const double vi = J->v[vix(J, b, t, h, i)];
        double yy = 0.0;
        for (int64_t j = 0; j < N; j++) {
            const size_t q = vix(J, b, t, h, j);
            S[i * N + j] = S[i * N + j] * J->w[q] + vi * J->k[q] + sa[i] * J->b[q];
            yy += S[i * N + j] * J->r[q];
        }
        if (y_out) y_out[i] = yy;
    }
}

static void *forward_worker(void *arg)
{
    job_t *J = (job_t *)arg;
    const int64_t N = J->N;
    double *S = (double *)malloc((size_t)N * N * sizeof(double));
    double *sa = (double *)malloc((size_t)N * sizeof(double));
    double *yt = (double *)malloc((size_t)N * sizeof(double));
    if (!S || !sa || !yt) { fail(J); free(S); free(sa); free(yt); return NULL; }
    int64_t u;
    while (take_unit(J, &u)) {
        const int64_t b = u / J->H, h = u % J->H;
        load_s0(J, b, h, S);
        for (int64_t t = 0; t < J->T; t++) {
            step_forward(J, b, t, h, S, sa, yt);
            if (J->y)
                for (int64_t i = 0; i < N; i++) J->y[vix(J, b, t, h, i)] = yt[i];
        }
        if (J->sT)
            for (int64_t i = 0; i < N; i++)
                for (int64_t j = 0; j < N; j++) J->sT[six(J, b, h, i, j)] = S[i * N + j];
    }
    free(S); free(sa); free(yt);
    return NULL;
}

static void *backward_worker(void *arg)
{
    job_t *J = (job_t *)arg;
    const int64_t N = J->N, T = J->T, NN = N * N;
    double *S = (double *)malloc((size_t)NN * sizeof(double));
    double *St = (double *)malloc((size_t)NN * sizeof(double));
    double *G = (double *)malloc((size_t)NN * sizeof(double));
    double *dsa = (double *)malloc((size_t)N * sizeof(double));
    double *Pc = (double *)malloc((size_t)(T > 0 ? T : 1) * NN * sizeof(double));
    double *sac = (double *)malloc((size_t)(T > 0 ? T : 1) * N * sizeof(double));
    if (!S || !St || !G || !dsa || !Pc || !sac) {
        fail(J);
        free(S); free(St); free(G); free(dsa); free(Pc); free(sac);
        return NULL;
    }
    int64_t u;
    while (take_unit(J, &u)) {
        const int64_t b = u / J->H, h = u % J->H;
        /* forward, keeping every pre-step state and every sa */
        load_s0(J, b, h, S);
        for (int64_t t = 0; t < T; t++) {
            memcpy(Pc + (size_t)t * NN, S, (size_t)NN * sizeof(double));
            step_forward(J, b, t, h, S, sac + (size_t)t * N, NULL);
        }
        /* seed */
        for (int64_t i = 0; i < N; i++)
            for (int64_t j = 0; j < N; j++)
                G[i * N + j] = J->dsT ? J->dsT[six(J, b, h, i, j)] : 0.0;
        /* reverse scan */
        for (int64_t t = T - 1; t >= 0; t--) {
            const double *P = Pc + (size_t)t * NN;
            const double *sa = sac + (size_t)t * N;
            /* state after step t, rebuilt from the cached pre-step state */
            for (int64_t i = 0; i < N; i++) {
                const double vi = J->v[vix(J, b, t, h, i)];
                for (int64_t j = 0; j < N; j++) {
                    const size_t q = vix(J, b, t, h, j);
                    St[i * N + j] = P[i * N + j] * J->w[q] + vi * J->k[q] + sa[i] * J->b[q];
                }
            }
            /* (1) read-out */
            for (int64_t j = 0; j < N; j++) {
                double acc = 0.0;
                for (int64_t i = 0; i < N; i++)
                    acc += St[i * N + j] * J->dy[vix(J, b, t, h, i)];
                J->dr[vix(J, b, t, h, j)] = acc;
            }
            for (int64_t i = 0; i < N; i++) {
                const double dyi = J->dy[vix(J, b, t, h, i)];
                for (int64_t j = 0; j < N; j++)
                    G[i * N + j] += dyi * J->r[vix(J, b, t, h, j)];
            }
            /* (2) update gradients */
            for (int64_t j = 0; j < N; j++) {
                double gk = 0.0, gb = 0.0, gw = 0.0;
                for (int64_t i = 0; i < N; i++) {
                    const double g = G[i * N + j];
                    gk += g * J->v[vix(J, b, t, h, i)];
                    gb += g * sa[i];
                    gw += g * P[i * N + j];
                }
                const size_t q = vix(J, b, t, h, j);
                J->dk[q] = gk;
                J->db[q] = gb;
                J->dw[q] = gw;
            }
            for (int64_t i = 0; i < N; i++) {
                double gv = 0.0, gs = 0.0;
                for (int64_t j = 0; j < N; j++) {
                    const size_t q = vix(J, b, t, h, j);
                    gv += G[i * N + j] * J->k[q];
                    gs += G[i * N + j] * J->b[q];
                }
                J->dv[vix(J, b, t, h, i)] = gv;
                dsa[i] = gs;
            }
            /* (3) in-context term and carry to t-1 */
            for (int64_t j = 0; j < N; j++) {
                double acc = 0.0;
                for (int64_t i = 0; i < N; i++)
                    acc += dsa[i] * P[i * N + j];
                J->da[vix(J, b, t, h, j)] = acc;
            }
            for (int64_t i = 0; i < N; i++)
                for (int64_t j = 0; j < N; j++) {
                    const size_t q = vix(J, b, t, h, j);
                    G[i * N + j] = G[i * N + j] * J->w[q] + dsa[i] * J->a[q];
                }
        }
        if (J->ds0)
            for (int64_t i = 0; i < N; i++)
                for (int64_t j = 0; j < N; j++) J->ds0[six(J, b, h, i, j)] = G[i * N + j];
    }
    free(S); free(St); free(G); free(dsa); free(Pc); free(sac);
    return NULL;
}

static int run(job_t *J, void *(*fn)(void *), int nthreads)
{
    if (J->B < 0 || J->T < 0 || J->H < 0 || J->N < 1) return -2;
    J->next = 0;
    J->failed = 0;
    pthread_mutex_init(&J->lock, NULL);
    int64_t units = J->B * J->H;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > units) nthreads = (int)(units > 0 ? units : 1);
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!th) { pthread_mutex_destroy(&J->lock); return -1; }
    int started = 0;
    for (int i = 0; i < nthreads; i++) {
        if (pthread_create(&th[i], NULL, fn, J) != 0) break;
        started++;
    }
    if (started == 0) fn(J);
    for (int i = 0; i < started; i++) pthread_join(th[i], NULL);
    free(th);
    pthread_mutex_destroy(&J->lock);
    return J->failed ? -1 : 0;
}

/* y, sT may be NULL (skipped).  Returns 0, -1 on allocation failure, -2 on
 * bad sizes. */
int wkv7_oracle_forward(const double *r, const double *w, const double *k,
                        const double *v, const double *a, const double *b,
                        const double *s0, double *y, double *sT,
                        int64_t B, int64_t T, int64_t H, int64_t N, int nthreads)
{
    job_t J;
    memset(&J, 0, sizeof J);
    J.r = r; J.w = w; J.k = k; J.v = v; J.a = a; J.b = b; J.s0 = s0;
    J.y = y; J.sT = sT;
    J.B = B; J.T = T; J.H = H; J.N = N;
    return run(&J, forward_worker, nthreads);
}

/* s0, dsT may be NULL (zeros); ds0 may be NULL (skipped).  All six input
 * gradients are required. */
int wkv7_oracle_backward(const double *r, const double *w, const double *k,
                         const double *v, const double *a, const double *b,
                         const double *dy, const double *s0, const double *dsT,
                         double *dr, double *dw, double *dk, double *dv,
                         double *da, double *db, double *ds0,
                         int64_t B, int64_t T, int64_t H, int64_t N, int nthreads)
{
    job_t J;
    memset(&J, 0, sizeof J);
    J.r = r; J.w = w; J.k = k; J.v = v; J.a = a; J.b = b; J.dy = dy;
    J.s0 = s0; J.dsT = dsT;
    J.dr = dr; J.dw = dw; J.dk = dk; J.dv = dv; J.da = da; J.db = db; J.ds0 = ds0;
    J.B = B; J.T = T; J.H = H; J.N = N;
    return run(&J, backward_worker, nthreads);
}
