/* Drives every entry point of oracle/oracle.c on small inputs, for a build
 * with AddressSanitizer and UndefinedBehaviorSanitizer (compiled and run by
 * tests/test_sanitizers.py).  Exits non-zero on any mismatch between the
 * brute force, the textbook network, the Kronecker form and the threaded
 * form on integer inputs, where all of them are exact. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double oracle_norm_constant_f64(int n);
float oracle_norm_constant_f32(int n);
void oracle_bruteforce_f64(const double* x, double* y, int64_t nvec, int n, int normalize);
void oracle_fwt_f64(double* x, int64_t nvec, int n, int normalize);
void oracle_fwt_f32(float* x, int64_t nvec, int n, int normalize);
int oracle_fwt_kron_f64(double* x, int64_t nvec, int n, int n1, int normalize);
int oracle_fwt_threaded_f32(float* x, int64_t nvec, int n, int normalize, int nthreads);
int oracle_fwt_threaded_f64(double* x, int64_t nvec, int n, int normalize, int nthreads);
int oracle_fwt_ld(const double* x, double* y, int64_t nvec, int n, int normalize);

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static int next_int(void)   /* xorshift64, values in [-8, 8] */
{
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (int)(rng % 17) - 8;
}

int main(void)
{
    int bad = 0;
    for (int n = 0; n <= 10; ++n) {
        const int64_t nvec = 3, N = (int64_t)1 << n, tot = nvec * N;
        double* x = malloc(sizeof(double) * tot);
        double* brute = malloc(sizeof(double) * tot);
        double* work = malloc(sizeof(double) * tot);
        float* wf = malloc(sizeof(float) * tot);
        for (int64_t i = 0; i < tot; ++i)
            x[i] = next_int();
        oracle_bruteforce_f64(x, brute, nvec, n, 0);
        memcpy(work, x, sizeof(double) * tot);
        oracle_fwt_f64(work, nvec, n, 0);
        bad += memcmp(work, brute, sizeof(double) * tot) != 0;
        for (int n1 = 0; n1 <= n; ++n1) {
            memcpy(work, x, sizeof(double) * tot);
            if (oracle_fwt_kron_f64(work, nvec, n, n1, 0) != 0)
                ++bad;
            bad += memcmp(work, brute, sizeof(double) * tot) != 0;
        }
        for (int64_t i = 0; i < tot; ++i)
            wf[i] = (float)x[i];
        oracle_fwt_f32(wf, nvec, n, 0);
        for (int64_t i = 0; i < tot; ++i)
            bad += (double)wf[i] != brute[i];
        for (int64_t i = 0; i < tot; ++i)
            wf[i] = (float)x[i];
        if (oracle_fwt_threaded_f32(wf, nvec, n, 0, 4) < 1)
            ++bad;
        for (int64_t i = 0; i < tot; ++i)
            bad += (double)wf[i] != brute[i];
        if (oracle_fwt_ld(x, work, nvec, n, 0) != 0)
            ++bad;
        bad += memcmp(work, brute, sizeof(double) * tot) != 0;
        memcpy(work, x, sizeof(double) * tot);
        if (oracle_fwt_threaded_f64(work, nvec, n, 1, 3) < 1)
            ++bad;
        oracle_fwt_f64(work, nvec, n, 1);   /* normalised twice: the input back */
        for (int64_t i = 0; i < tot; ++i)
            bad += fabs(work[i] - x[i]) > 1e-12 * (1 + fabs(x[i]));
        bad += !(oracle_norm_constant_f64(n) > 0) || !(oracle_norm_constant_f32(n) > 0);
        free(x);
        free(brute);
        free(work);
        free(wf);
    }
    {   /* a split outside [0, n] is rejected */
        double v[4] = {1, 2, 3, 4};
        bad += oracle_fwt_kron_f64(v, 1, 2, 3, 0) == 0;
        bad += oracle_fwt_kron_f64(v, 1, 2, -1, 0) == 0;
    }
    printf("oracle driver: %s\n", bad ? "MISMATCH" : "ok");
    return bad ? 1 : 0;
}
