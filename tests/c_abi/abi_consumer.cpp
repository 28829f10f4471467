// A plain C++ consumer of the C ABI in include/fwt.h: device memory from
// hipMalloc, a stream of its own, no Python and no torch.  It checks closed
// forms of the transform (the entry (-1)^popcount(k AND i) of the Apache
// Mahout pull request "[QDP] [feature] Pr4 kronecker fwt", section "How"):
//   - the unit vector e_j maps to the sign pattern (-1)^popcount(j AND k);
//   - two unnormalised calls map x to 2^n x exactly (zero-mean small
//     integers: every partial sum stays an exact integer);
//   - e_0 maps to 2^(-n/2) times the all-ones vector when normalised;
// over one-, two- and three-pass default plans in fp32 and fp64; and the
// one-pass entry point (fwt_execute_ws) against fwt_execute at n = 20.
// Prints "abi consumer: ok" and exits 0 on success.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <vector>

#include "fwt.h"

#define HIP_OK(x)                                                                 \
    do {                                                                          \
        hipError_t e_ = (x);                                                      \
        if (e_ != hipSuccess) {                                                   \
            std::printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
            return 2;                                                             \
        }                                                                         \
    } while (0)

static int popcount64(uint64_t v)
{
    int c = 0;
    for (; v; v &= v - 1)
        ++c;
    return c;
}

template <typename T>
static int run_case(int n, fwt_dtype dtype, int64_t batch, hipStream_t stream, int* bad)
{
    const int64_t N = (int64_t)1 << n, tot = batch * N;
    std::vector<T> re(tot), im(tot), out_re(tot), out_im(tot);
    uint64_t s = 0x9E3779B97F4A7C15ull ^ (uint64_t)n;
    const int64_t j = (N * 5 / 7) & (N - 1);
    for (int64_t b = 0; b < batch; ++b)
        for (int64_t i = 0; i < N; ++i) {
            s = s * 6364136223846793005ull + 1442695040888963407ull;
            // zero-mean small integers: U{-8..8}, or {-1, 0, 1} above n = 20,
            // so that every partial sum stays an exact integer below 2^24
            const int v = n <= 20 ? (int)((s >> 33) % 17) - 8 : (int)((s >> 33) % 3) - 1;
            re[b * N + i] = (T)v;
            im[b * N + i] = (T)(b == 0 ? (i == j ? 1 : 0) : 0);  // e_j, then zeros
        }
    T *d_re = nullptr, *d_im = nullptr;
    HIP_OK(hipMalloc(&d_re, sizeof(T) * tot));
    HIP_OK(hipMalloc(&d_im, sizeof(T) * tot));
    HIP_OK(hipMemcpy(d_re, re.data(), sizeof(T) * tot, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_im, im.data(), sizeof(T) * tot, hipMemcpyHostToDevice));

    fwt_plan_t plan = nullptr;
    if (fwt_plan_create(&plan, n, dtype, FWT_PATH_AUTO) != FWT_OK) {
        ++*bad;
        return 0;
    }
    int passes = 0;
    fwt_plan_num_passes(plan, &passes);
    // one call: im[0] = e_j -> signs
    int st = fwt_execute(plan, batch, n, d_re, d_im, 0, stream);
    HIP_OK(hipStreamSynchronize(stream));
    HIP_OK(hipMemcpy(out_im.data(), d_im, sizeof(T) * tot, hipMemcpyDeviceToHost));
    if (st != FWT_OK)
        ++*bad;
    for (int64_t k = 0; k < N; ++k)
        *bad += out_im[k] != (T)(popcount64((uint64_t)(j & k)) & 1 ? -1 : 1);
    // second call: re back to 2^n x, exactly
    st = fwt_execute(plan, batch, n, d_re, d_im, 0, stream);
    HIP_OK(hipStreamSynchronize(stream));
    HIP_OK(hipMemcpy(out_re.data(), d_re, sizeof(T) * tot, hipMemcpyDeviceToHost));
    if (st != FWT_OK)
        ++*bad;
    for (int64_t i = 0; i < tot; ++i)
        *bad += out_re[i] != re[i] * (T)N;
    // normalised e_0 -> 2^(-n/2) (1, ..., 1)
    HIP_OK(hipMemset(d_re, 0, sizeof(T) * tot));
    const T one = 1;
    HIP_OK(hipMemcpy(d_re, &one, sizeof(T), hipMemcpyHostToDevice));
    st = fwt_execute(plan, 1, n, d_re, nullptr, 1, stream);
    HIP_OK(hipStreamSynchronize(stream));
    HIP_OK(hipMemcpy(out_re.data(), d_re, sizeof(T) * N, hipMemcpyDeviceToHost));
    if (st != FWT_OK)
        ++*bad;
    const double c = std::ldexp(1.0, -n / 2) * (n % 2 ? std::sqrt(0.5) : 1.0);
    for (int64_t k = 0; k < N; ++k)
        *bad += std::fabs((double)out_re[k] - c) > 1e-6 * c;
    fwt_plan_destroy(plan);
    HIP_OK(hipFree(d_re));
    HIP_OK(hipFree(d_im));
    std::printf("n=%d %s batch=%lld passes=%d\n", n, dtype == FWT_F32 ? "f32" : "f64",
                (long long)batch, passes);
    return 0;
}

// The one-pass entry point on the default fp32 n = 20 plan: the workspace
// query, then fwt_execute_ws against fwt_execute on the same small-integer
// input (both exact, so equal bit for bit), a zero error word, and a
// workspace one byte short rejected before anything runs.
static int run_workspace_case(hipStream_t stream, int* bad)
{
    const int n = 20;
    const int64_t batch = 3, N = (int64_t)1 << n, tot = batch * N;
    std::vector<float> x(tot), a(tot), b(tot);
    uint64_t s = 0x2545F4914F6CDD1Dull;
    for (int64_t i = 0; i < tot; ++i) {
        s = s * 6364136223846793005ull + 1442695040888963407ull;
        x[i] = (float)((int)((s >> 33) % 17) - 8);
    }
    fwt_plan_t plan = nullptr;
    if (fwt_plan_create(&plan, n, FWT_F32, FWT_PATH_AUTO) != FWT_OK) {
        ++*bad;
        return 0;
    }
    size_t need = 0;
    if (fwt_workspace_size(plan, batch, 1, &need) != FWT_OK || need == 0) {
        std::printf("one-pass kernel unavailable (workspace %zu)\n", need);
        ++*bad;
        fwt_plan_destroy(plan);
        return 0;
    }
    float *d_a = nullptr, *d_b = nullptr, *d_ai = nullptr, *d_bi = nullptr;
    void* ws = nullptr;
    HIP_OK(hipMalloc(&d_a, sizeof(float) * tot));
    HIP_OK(hipMalloc(&d_b, sizeof(float) * tot));
    HIP_OK(hipMalloc(&d_ai, sizeof(float) * tot));
    HIP_OK(hipMalloc(&d_bi, sizeof(float) * tot));
    HIP_OK(hipMalloc(&ws, need));
    for (float* d : {d_a, d_b, d_ai, d_bi})
        HIP_OK(hipMemcpy(d, x.data(), sizeof(float) * tot, hipMemcpyHostToDevice));
    *bad += fwt_execute_ws(plan, batch, n, d_a, d_ai, 1, ws, need - 1, stream) != FWT_EINVAL;
    *bad += fwt_execute(plan, batch, n, d_a, d_ai, 1, stream) != FWT_OK;
    *bad += fwt_execute_ws(plan, batch, n, d_b, d_bi, 1, ws, need, stream) != FWT_OK;
    HIP_OK(hipStreamSynchronize(stream));
    int bits = -1;
    *bad += fwt_workspace_status(ws, &bits) != FWT_OK || bits != 0;
    HIP_OK(hipMemcpy(a.data(), d_a, sizeof(float) * tot, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(b.data(), d_b, sizeof(float) * tot, hipMemcpyDeviceToHost));
    for (int64_t i = 0; i < tot; ++i)
        *bad += a[i] != b[i];
    HIP_OK(hipMemcpy(a.data(), d_ai, sizeof(float) * tot, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(b.data(), d_bi, sizeof(float) * tot, hipMemcpyDeviceToHost));
    for (int64_t i = 0; i < tot; ++i)
        *bad += a[i] != b[i];
    fwt_plan_destroy(plan);
    for (void* d : {(void*)d_a, (void*)d_b, (void*)d_ai, (void*)d_bi, ws})
        HIP_OK(hipFree(d));
    std::printf("one-pass n=20 f32 batch=%lld workspace=%zu bytes error bits=%d\n",
                (long long)batch, need, bits);
    return 0;
}

int main()
{
    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));
    int bad = 0;
    if (run_workspace_case(stream, &bad))
        return 2;
    const int nf[] = {1, 5, 10, 12, 15, 16, 20, 22, 27};
    for (int n : nf)
        if (run_case<float>(n, FWT_F32, n <= 20 ? 3 : 1, stream, &bad))
            return 2;
    const int nd[] = {1, 9, 14, 15, 20, 24, 26};
    for (int n : nd)
        if (run_case<double>(n, FWT_F64, n <= 20 ? 3 : 1, stream, &bad))
            return 2;
    HIP_OK(hipStreamDestroy(stream));
    std::printf("abi consumer: %s (%d mismatches)\n", bad ? "MISMATCH" : "ok", bad);
    return bad ? 1 : 0;
}
