/*
 * wkv7_oracle.c -- plain fp64 CPU oracle of the WKV7 (RWKV-7) recurrence and
 * of its exact gradient (backward through time).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header or table with the
 * HIP library.
 *
 * What is computed (Foundry page "rwkvx/rx_pretrain.c": the forward
 * recurrence of rx_wkv7_forward_seq, and rx_wkv7_backward, whose result is
 * the gradient of that forward), written as matrix operations for one
 * (batch b, head h), state S in R^{N x N} (row i = value index, column
 * j = key index), W_t = diag(w_t):
 *
 *   forward, t = 0 .. T-1, S_{-1} = s0 (zeros when absent):
 *     S_t = S_{t-1} W_t + v_t k_t^T + (S_{t-1} a_t) b_t^T
 *         = S_{t-1} M_t + v_t k_t^T,          M_t = W_t + a_t b_t^T
 *     y_t = S_t r_t                            (the state after step t)
 *   sT = S_{T-1}.
 *
 *   backward: the gradient of L = sum_t <dy_t, y_t> + <dsT, sT> (dsT zeros
 *   when absent -- the page starts from zeros; a final-state gradient input
 *   is the extension the burn_mamba serial_recalculated backward.rs page
 *   makes with d_final_state).  With G = dL/dS_t, reverse-mode through the
 *   two lines above gives, for t = T-1 .. 0:
 *     dr_t = S_t^T dy_t                        (from y_t = S_t r_t)
 *     G   += dy_t r_t^T
 *     dv_t = G k_t,   dk_t = G^T v_t           (from v_t k_t^T)
 *     dM   = S_{t-1}^T G                       (from S_{t-1} M_t), so
 *       dw_t = diag(dM)           i.e. dw_t[j] = sum_i S_{t-1}[i][j] G[i][j]
 *       da_t = dM b_t             = S_{t-1}^T (G b_t)
 *       db_t = dM^T a_t           = G^T (S_{t-1} a_t)
 *     dL/dS_{t-1} = G M_t^T = G W_t + (G b_t) a_t^T
 *   ds0 = dL/dS_{-1}.  w is the multiplicative decay itself (not a log).
 *
 * Memory: the backward needs S_{t-1} and S_t for every t, in reverse.  It
 * keeps the state before every REPLAY-th step from one forward pass, then
 * for each such stretch, last first, replays the forward from that kept
 * state (the same operations on the same numbers, so the same doubles) and
 * holds the stretch's states.  That bounds memory by (T/REPLAY + REPLAY)
 * states per thread without changing any arithmetic.
 *
 * Layout: vectors [B][T][H][N] (one step of one (b,h) is N contiguous
 * values), states [B][H][N][N] row-major, all fp64.  (b,h) pairs are
 * independent and are spread over threads.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <pthread.h>

enum { REPLAY = 64 };

/* ------------------------------------------------------------------ */
/* Matrix helpers: N x N row-major matrices, N-vectors.               */

/* out = M x */
static void mat_vec(const double *M, const double *x, double *out, int64_t N)
{
    for (int64_t i = 0; i < N; i++) {
        double s = 0.0;
        for (int64_t j = 0; j < N; j++) s += M[i * N + j] * x[j];
        out[i] = s;
    }
}

/* out = M^T x */
static void mat_t_vec(const double *M, const double *x, double *out, int64_t N)
{
    for (int64_t j = 0; j < N; j++) {
        double s = 0.0;
        for (int64_t i = 0; i < N; i++) s += M[i * N + j] * x[i];
        out[j] = s;
    }
}

/* M = M diag(d) */
static void scale_cols(double *M, const double *d, int64_t N)
{
    for (int64_t i = 0; i < N; i++)
        for (int64_t j = 0; j < N; j++) M[i * N + j] *= d[j];
}

/* M = M + u x^T */
static void add_outer(double *M, const double *u, const double *x, int64_t N)
{
    for (int64_t i = 0; i < N; i++)
        for (int64_t j = 0; j < N; j++) M[i * N + j] += u[i] * x[j];
}

/* out[j] = sum_i A[i][j] B[i][j], the diagonal of A^T B */
static void diag_t_prod(const double *A, const double *B, double *out, int64_t N)
{
    for (int64_t j = 0; j < N; j++) {
        double s = 0.0;
        for (int64_t i = 0; i < N; i++) s += A[i * N + j] * B[i * N + j];
        out[j] = s;
    }
}

/* dst = src (N x N), or zeros when src is NULL */
static void copy_or_zero(double *dst, const double *src, int64_t N)
{
    if (src) memcpy(dst, src, (size_t)(N * N) * sizeof(double));
    else memset(dst, 0, (size_t)(N * N) * sizeof(double));
}

/* ------------------------------------------------------------------ */

typedef struct {
    const double *r, *w, *k, *v, *a, *b, *dy, *s0, *dsT;
    double *y, *sT, *dr, *dw, *dk, *dv, *da, *db, *ds0;
    int64_t B, T, H, N;
    int64_t next;          /* next (b,h) unit to take */
    int failed;
    pthread_mutex_t lock;
} job_t;

/* Offset of the N-vector of (b, t, h) in a [B][T][H][N] tensor. */
static inline size_t vec_at(const job_t *J, int64_t b, int64_t t, int64_t h)
{
    return (size_t)(((b * J->T + t) * J->H + h) * J->N);
}

/* Offset of the N x N state of (b, h) in a [B][H][N][N] tensor. */
static inline size_t state_at(const job_t *J, int64_t b, int64_t h)
{
    return (size_t)((b * J->H + h) * J->N * J->N);
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

/* One forward step at offset o of the vector tensors:
 * S <- S W + v k^T + (S a) b^T, in place; sa is scratch (N). */
static void step(const job_t *J, size_t o, double *S, double *sa)
{
    const int64_t N = J->N;
    mat_vec(S, J->a + o, sa, N);
    scale_cols(S, J->w + o, N);
    add_outer(S, J->v + o, J->k + o, N);
    add_outer(S, sa, J->b + o, N);
}

static void *forward_worker(void *arg)
{
    job_t *J = (job_t *)arg;
    const int64_t N = J->N;
    double *S = (double *)malloc((size_t)(N * N) * sizeof(double));
    double *sa = (double *)malloc((size_t)N * sizeof(double));
    if (!S || !sa) { fail(J); free(S); free(sa); return NULL; }
    int64_t u;
    while (take_unit(J, &u)) {
        const int64_t b = u / J->H, h = u % J->H;
        copy_or_zero(S, J->s0 ? J->s0 + state_at(J, b, h) : NULL, N);
        for (int64_t t = 0; t < J->T; t++) {
            const size_t o = vec_at(J, b, t, h);
            step(J, o, S, sa);
            if (J->y) mat_vec(S, J->r + o, J->y + o, N);
        }
        if (J->sT) memcpy(J->sT + state_at(J, b, h), S, (size_t)(N * N) * sizeof(double));
    }
    free(S); free(sa);
    return NULL;
}

static void *backward_worker(void *arg)
{
    job_t *J = (job_t *)arg;
    const int64_t N = J->N, T = J->T, NN = N * N;
    const int64_t nkeep = (T + REPLAY - 1) / REPLAY;
    double *keep = (double *)malloc((size_t)((nkeep > 0 ? nkeep : 1) * NN) * sizeof(double));
    double *hist = (double *)malloc((size_t)((REPLAY + 1) * NN) * sizeof(double));
    double *G = (double *)malloc((size_t)NN * sizeof(double));
    double *u = (double *)malloc((size_t)N * sizeof(double));
    double *sa = (double *)malloc((size_t)N * sizeof(double));
    if (!keep || !hist || !G || !u || !sa) {
        fail(J);
        free(keep); free(hist); free(G); free(u); free(sa);
        return NULL;
    }
    int64_t unit;
    while (take_unit(J, &unit)) {
        const int64_t b = unit / J->H, h = unit % J->H;
        /* forward pass keeping the state before steps 0, REPLAY, 2 REPLAY, ... */
        double *S = hist;
        copy_or_zero(S, J->s0 ? J->s0 + state_at(J, b, h) : NULL, N);
        for (int64_t t = 0; t < T; t++) {
            if (t % REPLAY == 0) memcpy(keep + (t / REPLAY) * NN, S, (size_t)NN * sizeof(double));
            step(J, vec_at(J, b, t, h), S, sa);
        }
        /* G = dL/dS_{T-1} */
        copy_or_zero(G, J->dsT ? J->dsT + state_at(J, b, h) : NULL, N);
        for (int64_t c = nkeep - 1; c >= 0; c--) {
            const int64_t t0 = c * REPLAY, t1 = t0 + REPLAY < T ? t0 + REPLAY : T;
            /* hist[s] = S_{t0+s-1}: the state before step t0+s, s = 0 .. t1-t0 */
            memcpy(hist, keep + c * NN, (size_t)NN * sizeof(double));
            for (int64_t t = t0; t < t1; t++) {
                double *next = hist + (t - t0 + 1) * NN;
                memcpy(next, hist + (t - t0) * NN, (size_t)NN * sizeof(double));
                step(J, vec_at(J, b, t, h), next, sa);
            }
            for (int64_t t = t1 - 1; t >= t0; t--) {
                const size_t o = vec_at(J, b, t, h);
                const double *Sprev = hist + (t - t0) * NN;     /* S_{t-1} */
                const double *Scur = hist + (t - t0 + 1) * NN;  /* S_t */
                /* y_t = S_t r_t */
                mat_t_vec(Scur, J->dy + o, J->dr + o, N);
                add_outer(G, J->dy + o, J->r + o, N);
                /* v_t k_t^T */
                mat_vec(G, J->k + o, J->dv + o, N);
                mat_t_vec(G, J->v + o, J->dk + o, N);
                /* S_{t-1} M_t with M_t = W_t + a_t b_t^T */
                diag_t_prod(Sprev, G, J->dw + o, N);
                mat_vec(G, J->b + o, u, N);
                mat_t_vec(Sprev, u, J->da + o, N);
                mat_vec(Sprev, J->a + o, sa, N);
                mat_t_vec(G, sa, J->db + o, N);
                /* G <- G M_t^T = G W_t + (G b_t) a_t^T */
                scale_cols(G, J->w + o, N);
                add_outer(G, u, J->a + o, N);
            }
        }
        if (J->ds0) memcpy(J->ds0 + state_at(J, b, h), G, (size_t)NN * sizeof(double));
    }
    free(keep); free(hist); free(G); free(u); free(sa);
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
