/*
 * rwkv8_oracle.c -- plain fp64 CPU oracle of the RWKV-8 rho / rho_norm
 * recurrence with normalised pre-update readout, and of its exact gradient.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header or table with the
 * HIP library.
 *
 * What is computed (burn_dragon_kernel page src/sequence/rwkv8/backward.rs:
 * compute_chunk_traces forms delta = query (x) value and runs the "before"
 * recurrences of rho and rho_norm; backward_chunk_impl gives the readout
 * through its gradients), for one (batch b, head h), with state rho R in
 * R^{L x E} (row l = latent index, column e = embedding index), rho_norm
 * n in R^L, per-head decay d in R^L, EPS = 1e-6:
 *
 *   t = 0 .. T-1, R_0 = rho_state (zeros when absent), n_0 likewise:
 *     sigma_t = sum_l q_t[l] + EPS
 *     c_t[l]  = q_t[l] / sigma_t / (n_t[l] + EPS)
 *     y_t     = R_t^T c_t                 (the state before step t)
 *     R_{t+1} = diag(d) R_t + q_t v_t^T
 *     n_{t+1} = diag(d) n_t + q_t
 *   final states R_T, n_T.
 *
 *   backward: the gradient of L = sum_t <dy_t, y_t> + <dR_T, R_T> + <dn_T, n_T>
 *   (dR_T, dn_T zeros when absent: the page starts from zero boundary
 *   gradients) by reverse-mode through the lines above.  With
 *   GR = dL/dR_{t+1}, Gn = dL/dn_{t+1}, for t = T-1 .. 0:
 *     dv_t  = GR^T q_t
 *     dq_t  = GR v_t + Gn
 *     dd   += diag(GR R_t^T) + Gn * n_t       (summed over b and t)
 *     GR    = diag(d) GR,  Gn = d * Gn       (now dL/dR_t, dL/dn_t)
 *     gc    = R_t dy_t                        (dL/dc_t)
 *     GR   += c_t dy_t^T
 *     gw    = gc / (n_t + EPS)
 *     dq_t += (gw - <gw, q_t / sigma_t>) / sigma_t
 *     Gn   -= gw * c_t
 *   dR_0 = GR, dn_0 = Gn.  (The page's grad_query_weights is gw, its
 *   grad_rho_from_context c dy^T, its grad_rho_norm_from_context -gw c.)
 *
 * Layouts as on the page: query [B][H][T][L], value [B][Hv][T][E] with Hv 1
 * (one value shared by the heads) or H, output [B][H][T][E], rho
 * [B][H][L][E], rho_norm [B][H][L], decay [H][L].  The backward writes the
 * value gradient of each (b,h) to dv [B][H][T][E] and the decay gradient of
 * each (b,h) to dd [B][H][L]; the caller sums them (over heads when Hv = 1,
 * over b for the decay).  Memory: the backward keeps the states before every
 * REPLAY-th step and replays each stretch (same operations, same doubles).
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <pthread.h>

enum { REPLAY = 64 };
static const double EPS = 1e-6;

typedef struct {
    const double *q, *v, *d, *R0, *n0, *dy, *dRT, *dnT;
    double *y, *RT, *nT, *dq, *dv, *dd, *dR0, *dn0;
    int64_t B, T, H, Hv, L, E;
    int64_t next;
    int failed;
    pthread_mutex_t lock;
} job_t;

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

/* offsets of step t of (b,h) in the query / value / output tensors */
static size_t q_at(const job_t *J, int64_t b, int64_t h, int64_t t)
{
    return (size_t)(((b * J->H + h) * J->T + t) * J->L);
}
static size_t v_at(const job_t *J, int64_t b, int64_t h, int64_t t)
{
    const int64_t hv = J->Hv == 1 ? 0 : h;
    return (size_t)(((b * J->Hv + hv) * J->T + t) * J->E);
}
static size_t y_at(const job_t *J, int64_t b, int64_t h, int64_t t)
{
    return (size_t)(((b * J->H + h) * J->T + t) * J->E);
}

/* c = q / (sum q + EPS) / (n + EPS); returns sigma */
static double read_weights(const double *q, const double *n, double *c, int64_t L)
{
    double s = 0.0;
    for (int64_t l = 0; l < L; l++) s += q[l];
    const double sigma = s + EPS;
    for (int64_t l = 0; l < L; l++) c[l] = q[l] / sigma / (n[l] + EPS);
    return sigma;
}

/* y = R^T c */
static void readout(const double *R, const double *c, double *y, int64_t L, int64_t E)
{
    for (int64_t e = 0; e < E; e++) {
        double acc = 0.0;
        for (int64_t l = 0; l < L; l++) acc += R[l * E + e] * c[l];
        y[e] = acc;
    }
}

/* R = diag(d) R + q v^T;  n = diag(d) n + q */
static void update(double *R, double *n, const double *d, const double *q, const double *v,
                   int64_t L, int64_t E)
{
    for (int64_t l = 0; l < L; l++) {
        for (int64_t e = 0; e < E; e++) R[l * E + e] = d[l] * R[l * E + e] + q[l] * v[e];
        n[l] = d[l] * n[l] + q[l];
    }
}

static void load_state(const job_t *J, int64_t b, int64_t h, double *R, double *n)
{
    const int64_t L = J->L, E = J->E, u = b * J->H + h;
    if (J->R0) memcpy(R, J->R0 + u * L * E, (size_t)(L * E) * sizeof(double));
    else memset(R, 0, (size_t)(L * E) * sizeof(double));
    if (J->n0) memcpy(n, J->n0 + u * L, (size_t)L * sizeof(double));
    else memset(n, 0, (size_t)L * sizeof(double));
}

static void *forward_worker(void *arg)
{
    job_t *J = (job_t *)arg;
    const int64_t L = J->L, E = J->E;
    double *R = malloc((size_t)(L * E) * sizeof(double));
    double *n = malloc((size_t)L * sizeof(double));
    double *c = malloc((size_t)L * sizeof(double));
    if (!R || !n || !c) { fail(J); free(R); free(n); free(c); return NULL; }
    int64_t u;
    while (take_unit(J, &u)) {
        const int64_t b = u / J->H, h = u % J->H;
        const double *d = J->d + h * L;
        load_state(J, b, h, R, n);
        for (int64_t t = 0; t < J->T; t++) {
            const double *q = J->q + q_at(J, b, h, t), *v = J->v + v_at(J, b, h, t);
            read_weights(q, n, c, L);
            if (J->y) readout(R, c, J->y + y_at(J, b, h, t), L, E);
            update(R, n, d, q, v, L, E);
        }
        if (J->RT) memcpy(J->RT + u * L * E, R, (size_t)(L * E) * sizeof(double));
        if (J->nT) memcpy(J->nT + u * L, n, (size_t)L * sizeof(double));
    }
    free(R); free(n); free(c);
    return NULL;
}

static void *backward_worker(void *arg)
{
    job_t *J = (job_t *)arg;
    const int64_t L = J->L, E = J->E, T = J->T, LE = L * E;
    const int64_t nkeep = (T + REPLAY - 1) / REPLAY;
    const size_t keepn = (size_t)(nkeep > 0 ? nkeep : 1);
    double *kR = malloc(keepn * LE * sizeof(double)), *kn = malloc(keepn * L * sizeof(double));
    double *hR = malloc((size_t)(REPLAY + 1) * LE * sizeof(double));
    double *hn = malloc((size_t)(REPLAY + 1) * L * sizeof(double));
    double *GR = malloc((size_t)LE * sizeof(double)), *Gn = malloc((size_t)L * sizeof(double));
    double *c = malloc((size_t)L * sizeof(double)), *gc = malloc((size_t)L * sizeof(double));
    double *dd = malloc((size_t)L * sizeof(double));
    if (!kR || !kn || !hR || !hn || !GR || !Gn || !c || !gc || !dd) {
        fail(J);
        free(kR); free(kn); free(hR); free(hn); free(GR); free(Gn); free(c); free(gc); free(dd);
        return NULL;
    }
    int64_t u;
    while (take_unit(J, &u)) {
        const int64_t b = u / J->H, h = u % J->H;
        const double *d = J->d + h * L;
        /* forward, keeping the states before steps 0, REPLAY, ... */
        load_state(J, b, h, hR, hn);
        for (int64_t t = 0; t < T; t++) {
            if (t % REPLAY == 0) {
                memcpy(kR + (t / REPLAY) * LE, hR, (size_t)LE * sizeof(double));
                memcpy(kn + (t / REPLAY) * L, hn, (size_t)L * sizeof(double));
            }
            update(hR, hn, d, J->q + q_at(J, b, h, t), J->v + v_at(J, b, h, t), L, E);
        }
        if (J->dRT) memcpy(GR, J->dRT + u * LE, (size_t)LE * sizeof(double));
        else memset(GR, 0, (size_t)LE * sizeof(double));
        if (J->dnT) memcpy(Gn, J->dnT + u * L, (size_t)L * sizeof(double));
        else memset(Gn, 0, (size_t)L * sizeof(double));
        memset(dd, 0, (size_t)L * sizeof(double));
        for (int64_t k = nkeep - 1; k >= 0; k--) {
            const int64_t t0 = k * REPLAY, t1 = t0 + REPLAY < T ? t0 + REPLAY : T;
            /* hR[s], hn[s]: the state before step t0 + s */
            memcpy(hR, kR + k * LE, (size_t)LE * sizeof(double));
            memcpy(hn, kn + k * L, (size_t)L * sizeof(double));
            for (int64_t t = t0; t < t1; t++) {
                double *R1 = hR + (t - t0 + 1) * LE, *n1 = hn + (t - t0 + 1) * L;
                memcpy(R1, hR + (t - t0) * LE, (size_t)LE * sizeof(double));
                memcpy(n1, hn + (t - t0) * L, (size_t)L * sizeof(double));
                update(R1, n1, d, J->q + q_at(J, b, h, t), J->v + v_at(J, b, h, t), L, E);
            }
            for (int64_t t = t1 - 1; t >= t0; t--) {
                const double *Rt = hR + (t - t0) * LE, *nt = hn + (t - t0) * L;
                const double *q = J->q + q_at(J, b, h, t), *v = J->v + v_at(J, b, h, t);
                const double *dy = J->dy + y_at(J, b, h, t);
                double *dq = J->dq + q_at(J, b, h, t), *dv = J->dv + y_at(J, b, h, t);
                /* through R_{t+1} = diag(d) R_t + q v^T and n_{t+1} = d n_t + q */
                for (int64_t e = 0; e < E; e++) {
                    double acc = 0.0;
                    for (int64_t l = 0; l < L; l++) acc += GR[l * E + e] * q[l];
                    dv[e] = acc;
                }
                for (int64_t l = 0; l < L; l++) {
                    double acc = 0.0, dacc = 0.0;
                    for (int64_t e = 0; e < E; e++) {
                        acc += GR[l * E + e] * v[e];
                        dacc += GR[l * E + e] * Rt[l * E + e];
                    }
                    dq[l] = acc + Gn[l];
                    dd[l] += dacc + Gn[l] * nt[l];
                }
                for (int64_t l = 0; l < L; l++) {
                    for (int64_t e = 0; e < E; e++) GR[l * E + e] *= d[l];
                    Gn[l] *= d[l];
                }
                /* through y_t = R_t^T c_t, c_t = q / sigma / (n_t + EPS) */
                const double sigma = read_weights(q, nt, c, L);
                double wq = 0.0;
                for (int64_t l = 0; l < L; l++) {
                    double acc = 0.0;
                    for (int64_t e = 0; e < E; e++) acc += Rt[l * E + e] * dy[e];
                    gc[l] = acc / (nt[l] + EPS);          /* gw */
                    wq += gc[l] * (q[l] / sigma);
                }
                for (int64_t l = 0; l < L; l++) {
                    for (int64_t e = 0; e < E; e++) GR[l * E + e] += c[l] * dy[e];
                    dq[l] += (gc[l] - wq) / sigma;
                    Gn[l] -= gc[l] * c[l];
                }
            }
        }
        if (J->dR0) memcpy(J->dR0 + u * LE, GR, (size_t)LE * sizeof(double));
        if (J->dn0) memcpy(J->dn0 + u * L, Gn, (size_t)L * sizeof(double));
        memcpy(J->dd + u * L, dd, (size_t)L * sizeof(double));
    }
    free(kR); free(kn); free(hR); free(hn); free(GR); free(Gn); free(c); free(gc); free(dd);
    return NULL;
}

static int run(job_t *J, void *(*fn)(void *), int nthreads)
{
    if (J->B < 0 || J->T < 0 || J->H < 0 || J->L < 1 || J->E < 1 ||
        (J->Hv != 1 && J->Hv != J->H))
        return -2;
    J->next = 0;
    J->failed = 0;
    pthread_mutex_init(&J->lock, NULL);
    const int64_t units = J->B * J->H;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > units) nthreads = (int)(units > 0 ? units : 1);
    pthread_t *th = calloc((size_t)nthreads, sizeof(pthread_t));
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

/* y, RT, nT may be NULL (skipped); R0, n0 NULL mean zeros. */
int rwkv8_oracle_forward(const double *q, const double *v, const double *d, const double *R0,
                         const double *n0, double *y, double *RT, double *nT, int64_t B,
                         int64_t T, int64_t H, int64_t Hv, int64_t L, int64_t E, int nthreads)
{
    job_t J;
    memset(&J, 0, sizeof J);
    J.q = q; J.v = v; J.d = d; J.R0 = R0; J.n0 = n0;
    J.y = y; J.RT = RT; J.nT = nT;
    J.B = B; J.T = T; J.H = H; J.Hv = Hv; J.L = L; J.E = E;
    return run(&J, forward_worker, nthreads);
}

/* dRT, dnT, R0, n0 NULL mean zeros; dR0, dn0 may be NULL (skipped); dq
 * [B][H][T][L], dv [B][H][T][E] (per head) and dd [B][H][L] (per (b,h)) are
 * required. */
int rwkv8_oracle_backward(const double *q, const double *v, const double *d, const double *R0,
                          const double *n0, const double *dy, const double *dRT,
                          const double *dnT, double *dq, double *dv, double *dd, double *dR0,
                          double *dn0, int64_t B, int64_t T, int64_t H, int64_t Hv, int64_t L,
                          int64_t E, int nthreads)
{
    job_t J;
    memset(&J, 0, sizeof J);
    J.q = q; J.v = v; J.d = d; J.R0 = R0; J.n0 = n0; J.dy = dy; J.dRT = dRT; J.dnT = dnT;
    J.dq = dq; J.dv = dv; J.dd = dd; J.dR0 = dR0; J.dn0 = dn0;
    J.B = B; J.T = T; J.H = H; J.Hv = Hv; J.L = L; J.E = E;
    return run(&J, backward_worker, nthreads);
}
