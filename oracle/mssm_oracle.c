/*
 * Oracle for the selective scan: a plain, sequential, fp64 CPU reference.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call
 * this file; only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark use it.  It shares no code, header or constant with the GPU library.
 *
 * What it computes, in the notation of the pages it follows:
 *
 *   Discretisation ("Understanding Mamba", section 2.2, equation (2)):
 *       Abar = exp(Delta * A)                      (A diagonal, so one scalar exp
 *                                                   per state channel; see
 *                                                   "Mathematical Prerequisites
 *                                                   for Mamba", section 3,
 *                                                   diagonal case)
 *       Bbar = Delta * B                           first-order form, which
 *                                                   "Selective State Space Models"
 *                                                   (section "Selection") says
 *                                                   Mamba itself uses      [EULER]
 *       Bbar = (Abar - 1) / A * B                  exact zero-order hold,
 *                                                   equation (2) for diagonal A
 *                                                   ("Understanding Mamba" 2.3
 *                                                   and 10.1)              [ZOH]
 *   Recurrence and read-out ("Understanding Mamba", section 2.3, equation (3)):
 *       h_t = Abar_t * h_{t-1} + Bbar_t * x_t      (elementwise over n)
 *       y_t = sum_n C_t[n] * h_t[n]  (+ D * x_t)   (feedthrough optional; the
 *                                                   pages set it to zero,
 *                                                   section 2.1)
 *   Optional gate of the Mamba block ("Understanding Mamba", section 8.1,
 *   equation (9)): out_t = y_t * SiLU(z_t), SiLU(v) = v / (1 + exp(-v)).
 *
 * The batched shapes are those of the PyTorch listing in "Selective State Space
 * Models": x, delta, y, z are [batch, L, D] (d fastest), B and C are
 * [batch, L, N] (n fastest, shared by every channel d), A is [D, N].  The state
 * h is [batch, D, N]; it starts at h0 (zero when h0 is NULL) and its final
 * value is written to h_last when that pointer is not NULL.
 *
 * Every (b, d) chain is independent ("Understanding Mamba", section 10.2: a
 * real layer runs the same logic independently across channels), so chains
 * are split over threads; within a chain the loop runs strictly in time order
 * and, inside a step, in ascending n.  No blocking, reordering or fusion.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>

#define ORACLE_BBAR_EULER 0
#define ORACLE_BBAR_ZOH 1

typedef struct {
    const double *x, *delta, *A, *B, *C, *Dskip, *z, *h0;
    double *y, *h_last;
    int64_t batch, L, D, N;
    int bbar_mode;
    int64_t chain_begin, chain_end;
    int status;
} oracle_job;

static double oracle_silu(double v) { return v / (1.0 + exp(-v)); }

static void run_chain(const oracle_job *j, int64_t b, int64_t d, double *h) {
    const int64_t L = j->L, D = j->D, N = j->N;
    for (int64_t n = 0; n < N; ++n)
        h[n] = j->h0 ? j->h0[(b * D + d) * N + n] : 0.0;
    for (int64_t t = 0; t < L; ++t) {
        const int64_t i = (b * L + t) * D + d;   /* [batch, L, D] element   */
        const int64_t s = (b * L + t) * N;       /* [batch, L, N] row start */
        const double delta_t = j->delta[i];
        const double x_t = j->x[i];
        double y_t = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            const double a = j->A[d * N + n];
            const double Abar = exp(delta_t * a);
            double Bbar;
            if (j->bbar_mode == ORACLE_BBAR_ZOH)
                /* (Delta A)^-1 (exp(Delta A) - 1) Delta B; its A -> 0 limit is Delta B */
                Bbar = (a != 0.0) ? (Abar - 1.0) / a * j->B[s + n] : delta_t * j->B[s + n];
            else
                Bbar = delta_t * j->B[s + n];
            h[n] = Abar * h[n] + Bbar * x_t;
            y_t += j->C[s + n] * h[n];
        }
        if (j->Dskip) y_t += j->Dskip[d] * x_t;
        if (j->z) y_t *= oracle_silu(j->z[i]);
        j->y[i] = y_t;
    }
    if (j->h_last)
        for (int64_t n = 0; n < N; ++n) j->h_last[(b * D + d) * N + n] = h[n];
}

static void *run_range(void *arg) {
    oracle_job *j = (oracle_job *)arg;
    double *h = (double *)malloc((size_t)(j->N > 0 ? j->N : 1) * sizeof(double));
    if (!h) { j->status = 2; return NULL; }
    for (int64_t c = j->chain_begin; c < j->chain_end; ++c)
        run_chain(j, c / j->D, c % j->D, h);
    free(h);
    j->status = 0;
    return NULL;
}

/* Returns 0 on success, 1 on bad arguments, 2 on allocation/thread failure. */
int oracle_selective_scan(const double *x, const double *delta, const double *A,
                          const double *B, const double *C, const double *Dskip,
                          const double *z, const double *h0, double *y, double *h_last,
                          int64_t batch, int64_t L, int64_t D, int64_t N,
                          int bbar_mode, int nthreads) {
    if (batch < 0 || L < 0 || D < 0 || N < 0) return 1;
    if (bbar_mode != ORACLE_BBAR_EULER && bbar_mode != ORACLE_BBAR_ZOH) return 1;
    const int64_t chains = batch * D;
    if (chains == 0) return 0;
    if (L > 0 && (!x || !delta || !B || !C || !y)) return 1;
    if (N > 0 && !A) return 1;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > chains) nthreads = (int)chains;

    oracle_job *jobs = (oracle_job *)calloc((size_t)nthreads, sizeof(oracle_job));
    pthread_t *tids = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !tids) { free(jobs); free(tids); return 2; }
    int rc = 0;
    int started = 0;
    for (int k = 0; k < nthreads; ++k) {
        oracle_job *j = &jobs[k];
        j->x = x; j->delta = delta; j->A = A; j->B = B; j->C = C;
        j->Dskip = Dskip; j->z = z; j->h0 = h0; j->y = y; j->h_last = h_last;
        j->batch = batch; j->L = L; j->D = D; j->N = N; j->bbar_mode = bbar_mode;
        j->chain_begin = chains * k / nthreads;
        j->chain_end = chains * (k + 1) / nthreads;
        j->status = 2;
        if (nthreads == 1) { run_range(j); break; }
        if (pthread_create(&tids[k], NULL, run_range, j) != 0) { rc = 2; break; }
        ++started;
    }
    for (int k = 0; k < started; ++k) pthread_join(tids[k], NULL);
    if (rc == 0)
        for (int k = 0; k < nthreads; ++k) if (jobs[k].status != 0) rc = jobs[k].status;
    free(jobs);
    free(tids);
    return rc;
}
