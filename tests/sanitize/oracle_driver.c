/*
 * Drives the CPU oracle (oracle/ssm_oracle.c) under AddressSanitizer and
 * UndefinedBehaviorSanitizer: every argument shape the tests use (y and C present or
 * absent, per-sequence token counts including 0 and T, one and several threads, the
 * rejected argument sets), with two checks whose answers follow from the recurrence
 * alone: dt = 0 leaves the state unchanged, and a sequence given 0 tokens keeps h0.
 * Test infrastructure: built and run by tests/test_sanitizers.py on the CPU.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

int ssm_oracle_scan(int Bt, int T, int H, int P, int N, int G, const double *x, const double *B,
                    const double *C, const double *dt, const double *A, const double *D, const int *ntok,
                    double *state, double *y, int nthreads);

static double *filled(size_t n, double scale, unsigned *seed)
{
    double *p = (double *)malloc(n * sizeof(double));
    for (size_t i = 0; i < n; ++i) {
        *seed = *seed * 1103515245u + 12345u;
        p[i] = scale * ((double)((*seed >> 8) & 0xffff) / 65535.0 - 0.5);
    }
    return p;
}

int main(void)
{
    const int Bt = 3, T = 7, H = 4, P = 5, N = 6, G = 2;
    unsigned seed = 7;
    double *x = filled((size_t)Bt * T * H * P, 1.0, &seed);
    double *B = filled((size_t)Bt * T * G * N, 1.0, &seed);
    double *C = filled((size_t)Bt * T * G * N, 1.0, &seed);
    double *dt = filled((size_t)Bt * T * H, 1.0, &seed);
    double *A = filled(H, 1.0, &seed);
    double *D = filled(H, 1.0, &seed);
    double *h0 = filled((size_t)Bt * H * N * P, 1.0, &seed);
    double *st = (double *)malloc((size_t)Bt * H * N * P * sizeof(double));
    double *y = (double *)calloc((size_t)Bt * T * H * P, sizeof(double));
    for (int i = 0; i < Bt * T * H; ++i) dt[i] = fabs(dt[i]) + 0.1;
    for (int i = 0; i < H; ++i) A[i] = -fabs(A[i]) - 1.0;
    const int ntok[3] = {0, 3, 7};
    int fails = 0;
    for (int nth = 1; nth <= 5; nth += 4) {
        for (int i = 0; i < Bt * H * N * P; ++i) st[i] = h0[i];
        fails += ssm_oracle_scan(Bt, T, H, P, N, G, x, B, C, dt, A, D, NULL, st, y, nth) != 0;
        for (int i = 0; i < Bt * H * N * P; ++i) st[i] = h0[i];
        fails += ssm_oracle_scan(Bt, T, H, P, N, G, x, B, C, dt, A, D, ntok, st, y, nth) != 0;
        /* sequence 0 took no token: its state is h0 exactly */
        for (int i = 0; i < H * N * P; ++i) fails += st[i] != h0[i];
        fails += ssm_oracle_scan(Bt, T, H, P, N, G, x, B, NULL, dt, A, D, ntok, st, NULL, nth) != 0;
    }
    /* dt = 0: abar = 1 and no input, so the state does not move */
    double *z = (double *)calloc((size_t)Bt * T * H, sizeof(double));
    for (int i = 0; i < Bt * H * N * P; ++i) st[i] = h0[i];
    fails += ssm_oracle_scan(Bt, T, H, P, N, G, x, B, C, z, A, D, NULL, st, y, 2) != 0;
    for (int i = 0; i < Bt * H * N * P; ++i) fails += st[i] != h0[i];
    /* rejected argument sets touch nothing */
    const int bad_ntok[3] = {0, 8, 1};
    fails += ssm_oracle_scan(Bt, T, H, P, N, G, x, B, C, dt, A, D, bad_ntok, st, y, 1) != -1;
    fails += ssm_oracle_scan(Bt, T, 3, P, N, G, x, B, C, dt, A, D, NULL, st, y, 1) != -1;
    fails += ssm_oracle_scan(Bt, T, H, P, N, G, x, B, NULL, dt, A, D, NULL, st, y, 1) != -1;
    fails += ssm_oracle_scan(Bt, T, H, P, N, G, x, B, C, dt, A, D, NULL, NULL, y, 1) != -1;
    fails += ssm_oracle_scan(0, T, H, P, N, G, x, B, C, dt, A, D, NULL, st, y, 3) != 0;
    free(x); free(B); free(C); free(dt); free(A); free(D); free(h0); free(st); free(y); free(z);
    printf(fails ? "FAIL %d\n" : "OK\n", fails);
    return fails ? 1 : 0;
}
