/*
 * ssm_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, double-precision CPU reference for the selective state-space
 * layer that "The Mamba in the Llama: Distilling and Accelerating Hybrid Models"
 * puts in place of attention, and for its speculative verify / roll-back step.
 * Only the test suite, the smoke check and the bench's CPU-baseline leg may
 * load this file's library.  It shares no code, header or table with the GPU
 * library, and the GPU library never calls it.
 *
 * What it computes (one sequence b, one head h, group g = h / (H/G)):
 *   abar_t = exp(dt_t * A_h)                                  (discretised decay)
 *   h_t    = abar_t * h_{t-1} + (dt_t * B_t) x_t^T            (N x P state)
 *   y_t[p] = sum_n C_t[n] h_t[n][p]  +  D_h x_t[p]            (update, then read)
 * Sources:
 *   - abstract of the paper: attention is distilled into a linear RNN that
 *     reuses the attention projections (x from V, B from K, C from Q);
 *   - skycaiji.com summary, method paragraph: a continuous-time SSM, expanded
 *     hidden state, turned into a discrete-time linear RNN step by step (read
 *     here as a zero-order hold on A and an Euler step on B);
 *   - QbitAI article "Llama 3+Mamba 强强联手", speculative-decoding walkthrough:
 *     the Mamba layers take the K draft tokens one after another, the state
 *     moves forward only through accepted tokens, no intermediate state is
 *     kept, and a rejection rolls the state back to the last accepted token.
 *
 * Every loop runs in the order written above: tokens ascending, then n, then p;
 * the readout sums n ascending.  Compile with -O2 -fno-fast-math
 * -ffp-contract=off so that the compiler neither fuses nor reorders.
 * Parallelism is only over independent (sequence, head) pairs, each of which
 * runs the plain loop.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* One token for one (sequence, head): update the N x P state in place, then,
 * if y is not NULL, read out the P outputs.  The three passages cited in the
 * header define every term here. */
static void oracle_token(int P, int N, double dt, double A, double D,
                         const double *x, const double *b, const double *c,
                         double *h, double *y)
{
    const double abar = exp(dt * A);
    for (int n = 0; n < N; ++n) {
        const double bn = dt * b[n];
        double *row = h + (size_t)n * P;
        for (int p = 0; p < P; ++p)
            row[p] = abar * row[p] + bn * x[p];
    }
    if (!y)
        return;
    for (int p = 0; p < P; ++p) {
        double acc = 0.0;
        for (int n = 0; n < N; ++n)
            acc += c[n] * h[(size_t)n * P + p];
        y[p] = acc + D * x[p];
    }
}

typedef struct {
    int Bt, T, H, P, N, G;
    const double *x, *B, *C, *dt, *A, *D;
    const int *ntok;
    double *state, *y;
    int tid, nthreads;
} scan_job;

static void *scan_worker(void *arg)
{
    const scan_job *j = (const scan_job *)arg;
    const int heads_per_group = j->H / j->G;
    for (int bh = j->tid; bh < j->Bt * j->H; bh += j->nthreads) {
        const int b = bh / j->H, h = bh % j->H, g = h / heads_per_group;
        const int T = j->ntok ? j->ntok[b] : j->T;
        double *hs = j->state + (size_t)bh * j->N * j->P;
        for (int t = 0; t < T; ++t) {
            const size_t bt = (size_t)b * j->T + t;
            const double *x = j->x + (bt * j->H + h) * j->P;
            const double *bb = j->B + (bt * j->G + g) * j->N;
            const double *cc = j->C ? j->C + (bt * j->G + g) * j->N : NULL;
            double *y = j->y ? j->y + (bt * j->H + h) * j->P : NULL;
            oracle_token(j->P, j->N, j->dt[bt * j->H + h], j->A[h], j->D[h], x, bb, cc, hs, y);
        }
    }
    return NULL;
}

/*
 * Run the recurrence over tokens [0, ntok[b]) of each sequence b.
 *   x  [Bt][T][H][P], B and C [Bt][T][G][N], dt [Bt][T][H], A and D [H]
 *   state [Bt][H][N][P]: read as h_0, overwritten with h_{ntok[b]}
 *   y [Bt][T][H][P]: rows t < ntok[b] are written; NULL skips the readout
 *   C may be NULL only when y is NULL.  ntok NULL means T for every sequence.
 *   nthreads <= 1 runs on the calling thread.
 * Returns 0, or -1 for inconsistent arguments (nothing is touched then).
 */
int ssm_oracle_scan(int Bt, int T, int H, int P, int N, int G,
                    const double *x, const double *B, const double *C,
                    const double *dt, const double *A, const double *D,
                    const int *ntok, double *state, double *y, int nthreads)
{
    if (Bt < 0 || T < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G != 0)
        return -1;
    if (!state || !A || !D || (T > 0 && (!x || !B || !dt)) || (y && !C))
        return -1;
    if (ntok)
        for (int b = 0; b < Bt; ++b)
            if (ntok[b] < 0 || ntok[b] > T)
                return -1;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > Bt * H)
        nthreads = Bt * H > 0 ? Bt * H : 1;

    scan_job *jobs = (scan_job *)calloc((size_t)nthreads, sizeof(scan_job));
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !th) {
        free(jobs);
        free(th);
        return -1;
    }
    for (int i = 0; i < nthreads; ++i) {
        scan_job j = {Bt, T, H, P, N, G, x, B, C, dt, A, D, ntok, state, y, i, nthreads};
        jobs[i] = j;
    }
    int spawned = 0;
    for (int i = 1; i < nthreads; ++i)
        if (pthread_create(&th[i], NULL, scan_worker, &jobs[i]) == 0)
            spawned = i;
        else
            break;
    /* a worker that could not start is run here instead */
    for (int i = spawned + 1; i < nthreads; ++i)
        scan_worker(&jobs[i]);
    scan_worker(&jobs[0]);
    for (int i = 1; i <= spawned; ++i)
        pthread_join(th[i], NULL);
    free(jobs);
    free(th);
    return 0;
}
