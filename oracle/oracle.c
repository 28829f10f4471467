/*
 * CPU oracle for the batched Walsh-Hadamard transform.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: it exists so that tests, the smoke check and the CPU
 * baseline leg of the benchmark have an independent, obviously correct
 * reference.  It shares no code, header, table or constant with the HIP
 * library.
 *
 * What is computed (one real vector x of length N = 2^n; a complex planar
 * state is two such vectors, the real part and the imaginary part, since
 * every matrix entry is real):
 *
 *   y_k = c * sum_{i=0}^{N-1} (-1)^{popcount(k AND i)} * x_i
 *
 * with c = 1 (unnormalised) or c = 2^(-n/2) (normalised).  The entry
 * (-1)^{popcount(k AND i)} is the Walsh matrix entry that the Apache Mahout
 * pull request "[QDP] [feature] Pr4 kronecker fwt" (section "How", the
 * naive implicit Hadamard GEMM placeholder) generates on the fly from the
 * population count of k AND i.  Natural (Sylvester) order, no reordering.
 *
 * Functions:
 *   oracle_bruteforce_f64   the definition above, O(4^n) per vector
 *   oracle_fwt_f64 / _f32   textbook iterative butterfly network: for each
 *                           stage s = 0..n-1, every pair of indices that
 *                           differ only in bit s (stride 2^s) is replaced by
 *                           (sum, difference), lower index keeps the sum.
 *                           This is the stage list of the iThome "Day 18"
 *                           native-FWT article, section "Tensor Core wants
 *                           matrix multiplication" (stage 0 local pairs,
 *                           stage 1 stride 2, stage 2 stride 4, ...).  The
 *                           f32 variant is the timed CPU baseline; the f64
 *                           variant is the parity reference ("check mode").
 *   oracle_fwt_kron_f64     the Kronecker form H_n = H_{n1} (x) H_{n2}:
 *                           each vector viewed as a row-major 2^n1 x 2^n2
 *                           matrix; the n2-bit transform on every row, then
 *                           the n1-bit transform on every column.  Mahout
 *                           pull request, sections "Why" and the
 *                           deliverables table of "Why submit PR4"
 *                           (Y = (H_{n1} (x) I)(I (x) H_{n2}) X); iThome
 *                           article, section "Kronecker block GEMM idea".
 *   oracle_fwt_threaded_*   the textbook transform run over the batch by a
 *                           pool of POSIX threads (CPU baseline timing).
 *   oracle_fwt_ld           the same butterfly network in long double
 *                           (x86-64: 64-bit significand), rounded to double
 *                           once at the end: a higher-precision evaluation
 *                           that bounds the rounding of the fp64 check mode.
 *
 * Normalisation constant (the pages do not state one; the plain reading of
 * "1/sqrt(2^n)-normalised" is used): c = 2^(-n/2), computed as
 * ldexp(1, -n/2) for even n and ldexp(sqrt(0.5), -(n-1)/2) for odd n,
 * applied once after all stages.  The f32 variant rounds c to float once.
 *
 * Build: gcc -O2 -ffp-contract=off -shared -fPIC (no fast-math, no SIMD
 * intrinsics), so every add and subtract is a single IEEE operation.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Population count by the plain bit loop, so the definition can be read
 * without knowing any compiler builtin. */
static int popcount_u64(uint64_t v)
{
    int c = 0;
    while (v) {
        c += (int)(v & 1u);
        v >>= 1;
    }
    return c;
}

double oracle_norm_constant_f64(int n)
{
    if (n % 2 == 0)
        return ldexp(1.0, -(n / 2));
    return ldexp(sqrt(0.5), -((n - 1) / 2));
}

float oracle_norm_constant_f32(int n)
{
    return (float)oracle_norm_constant_f64(n);
}

/* y[b][k] = sum_i (-1)^popcount(k&i) x[b][i], accumulated in double,
 * then times c if normalize. x and y must not alias. */
void oracle_bruteforce_f64(const double* x, double* y, int64_t nvec, int n,
                           int normalize)
{
    const int64_t N = (int64_t)1 << n;
    const double c = normalize ? oracle_norm_constant_f64(n) : 1.0;
    for (int64_t b = 0; b < nvec; ++b) {
        const double* xb = x + b * N;
        double* yb = y + b * N;
        for (int64_t k = 0; k < N; ++k) {
            double acc = 0.0;
            for (int64_t i = 0; i < N; ++i) {
                if (popcount_u64((uint64_t)(k & i)) % 2 == 0)
                    acc += xb[i];
                else
                    acc -= xb[i];
            }
            yb[k] = normalize ? acc * c : acc;
        }
    }
}

/* One real vector, in place, textbook butterfly network, double. */
static void fwt_one_f64(double* v, int n)
{
    const int64_t N = (int64_t)1 << n;
    for (int64_t h = 1; h < N; h *= 2) {          /* stage s: h = 2^s */
        for (int64_t i = 0; i < N; i += 2 * h) {
            for (int64_t j = i; j < i + h; ++j) {
                const double a = v[j];
                const double b = v[j + h];
                v[j] = a + b;
                v[j + h] = a - b;
            }
        }
    }
}

static void fwt_one_f32(float* v, int n)
{
    const int64_t N = (int64_t)1 << n;
    for (int64_t h = 1; h < N; h *= 2) {
        for (int64_t i = 0; i < N; i += 2 * h) {
            for (int64_t j = i; j < i + h; ++j) {
                const float a = v[j];
                const float b = v[j + h];
                v[j] = a + b;
                v[j + h] = a - b;
            }
        }
    }
}

void oracle_fwt_f64(double* x, int64_t nvec, int n, int normalize)
{
    const int64_t N = (int64_t)1 << n;
    const double c = oracle_norm_constant_f64(n);
    for (int64_t b = 0; b < nvec; ++b) {
        double* v = x + b * N;
        fwt_one_f64(v, n);
        if (normalize)
            for (int64_t k = 0; k < N; ++k)
                v[k] *= c;
    }
}

void oracle_fwt_f32(float* x, int64_t nvec, int n, int normalize)
{
    const int64_t N = (int64_t)1 << n;
    const float c = oracle_norm_constant_f32(n);
    for (int64_t b = 0; b < nvec; ++b) {
        float* v = x + b * N;
        fwt_one_f32(v, n);
        if (normalize)
            for (int64_t k = 0; k < N; ++k)
                v[k] *= c;
    }
}

/* The textbook network in long double, one vector at a time, the result
 * (times c in long double if normalize) rounded to double once.  x and y
 * must not alias.  Returns 0, or -1 if the work vector cannot be
 * allocated. */
int oracle_fwt_ld(const double* x, double* y, int64_t nvec, int n, int normalize)
{
    const int64_t N = (int64_t)1 << n;
    const long double c = n % 2 == 0 ? ldexpl(1.0L, -(n / 2))
                                     : ldexpl(sqrtl(0.5L), -((n - 1) / 2));
    long double* v = (long double*)malloc((size_t)N * sizeof(long double));
    if (!v)
        return -1;
    for (int64_t b = 0; b < nvec; ++b) {
        for (int64_t k = 0; k < N; ++k)
            v[k] = (long double)x[b * N + k];
        for (int64_t h = 1; h < N; h *= 2) {
            for (int64_t i = 0; i < N; i += 2 * h) {
                for (int64_t j = i; j < i + h; ++j) {
                    const long double a = v[j];
                    const long double d = v[j + h];
                    v[j] = a + d;
                    v[j + h] = a - d;
                }
            }
        }
        for (int64_t k = 0; k < N; ++k)
            y[b * N + k] = (double)(normalize ? v[k] * c : v[k]);
    }
    free(v);
    return 0;
}

/* Kronecker-composed transform: rows (n2 = n - n1 low bits) first, then
 * columns (n1 high bits).  Returns 0, or -1 if n1 is out of range or the
 * column buffer cannot be allocated. */
int oracle_fwt_kron_f64(double* x, int64_t nvec, int n, int n1, int normalize)
{
    if (n1 < 0 || n1 > n)
        return -1;
    const int n2 = n - n1;
    const int64_t N = (int64_t)1 << n;
    const int64_t R = (int64_t)1 << n1;   /* number of rows    */
    const int64_t C = (int64_t)1 << n2;   /* number of columns */
    const double c = oracle_norm_constant_f64(n);
    double* col = (double*)malloc((size_t)R * sizeof(double));
    if (!col)
        return -1;
    for (int64_t b = 0; b < nvec; ++b) {
        double* m = x + b * N;            /* m[r*C + q] */
        for (int64_t r = 0; r < R; ++r)   /* (I (x) H_n2): every row */
            fwt_one_f64(m + r * C, n2);
        for (int64_t q = 0; q < C; ++q) { /* (H_n1 (x) I): every column */
            for (int64_t r = 0; r < R; ++r)
                col[r] = m[r * C + q];
            fwt_one_f64(col, n1);
            for (int64_t r = 0; r < R; ++r)
                m[r * C + q] = col[r];
        }
        if (normalize)
            for (int64_t k = 0; k < N; ++k)
                m[k] *= c;
    }
    free(col);
    return 0;
}

/* ---- threaded textbook transform (CPU baseline timing) ------------------ */

struct job {
    void* x;
    int64_t first, count;
    int n, normalize, is_f64;
};

static void* run_job(void* arg)
{
    const struct job* j = (const struct job*)arg;
    const int64_t N = (int64_t)1 << j->n;
    if (j->is_f64)
        oracle_fwt_f64((double*)j->x + j->first * N, j->count, j->n, j->normalize);
    else
        oracle_fwt_f32((float*)j->x + j->first * N, j->count, j->n, j->normalize);
    return NULL;
}

/* Splits the nvec real vectors into nthreads contiguous ranges, one POSIX
 * thread each.  Returns the number of threads actually used (>= 1), or -1. */
static int threaded(void* x, int64_t nvec, int n, int normalize, int nthreads,
                    int is_f64)
{
    if (nthreads < 1)
        nthreads = 1;
    if (nvec < nthreads)
        nthreads = nvec > 0 ? (int)nvec : 1;
    pthread_t* tid = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
    struct job* jobs = (struct job*)calloc((size_t)nthreads, sizeof(struct job));
    if (!tid || !jobs) {
        free(tid);
        free(jobs);
        return -1;
    }
    int64_t start = 0;
    for (int t = 0; t < nthreads; ++t) {
        const int64_t cnt = nvec / nthreads + (t < nvec % nthreads ? 1 : 0);
        jobs[t].x = x;
        jobs[t].first = start;
        jobs[t].count = cnt;
        jobs[t].n = n;
        jobs[t].normalize = normalize;
        jobs[t].is_f64 = is_f64;
        start += cnt;
    }
    int launched = 0;
    for (int t = 1; t < nthreads; ++t) {
        if (pthread_create(&tid[t], NULL, run_job, &jobs[t]) != 0)
            break;
        ++launched;
    }
    run_job(&jobs[0]);
    for (int t = 1; t <= launched; ++t)
        pthread_join(tid[t], NULL);
    /* Ranges whose thread could not be started run on the caller. */
    for (int t = launched + 1; t < nthreads; ++t)
        run_job(&jobs[t]);
    free(tid);
    free(jobs);
    return launched + 1;
}

int oracle_fwt_threaded_f32(float* x, int64_t nvec, int n, int normalize, int nthreads)
{
    return threaded(x, nvec, n, normalize, nthreads, 0);
}

int oracle_fwt_threaded_f64(double* x, int64_t nvec, int n, int normalize, int nthreads)
{
    return threaded(x, nvec, n, normalize, nthreads, 1);
}
