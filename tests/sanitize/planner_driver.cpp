// Drives the host side of the C ABI (plan creation for random splits and
// tunings, every query, destruction, argument validation) for a build with
// AddressSanitizer, LeakSanitizer and UndefinedBehaviorSanitizer (compiled
// and run by tests/test_sanitizers.py).  No device is touched: the kernel
// entry points are stubs, and execute-side calls use arguments that fail
// validation before any HIP call.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "fwt.h"

static uint64_t state = 0x2545F4914F6CDD1Dull;
static int rnd(int lo, int hi)   // inclusive, xorshift64
{
    state ^= state << 13;
    state ^= state >> 7;
    state ^= state << 17;
    return lo + (int)(state % (uint64_t)(hi - lo + 1));
}

int main()
{
    int bad = 0, ok = 0;
    // Default plans over every n, dtype and path, plus out-of-range ones.
    for (int n = -2; n <= 32; ++n)
        for (int d = 0; d <= 2; ++d)
            for (int path = 0; path <= 4; ++path) {
                fwt_plan_t p = nullptr;
                const int st = fwt_plan_create(&p, n, (fwt_dtype)d, (fwt_path)path);
                if (st == FWT_OK) {
                    int np = 0;
                    // n = 0 is the identity: no passes
                    bad += fwt_plan_num_passes(p, &np) != FWT_OK || np < (n > 0) || np > 4;
                    int sum = 0;
                    for (int i = 0; i < np; ++i) {
                        int b = 0, cfg[12];
                        bad += fwt_plan_pass_bits(p, i, &b) != FWT_OK;
                        bad += fwt_plan_pass_config(p, i, cfg) != FWT_OK;
                        for (int64_t batch : {(int64_t)0, (int64_t)64, (int64_t)1 << 40})
                            for (int w = 0; w <= 1; ++w)
                                bad += fwt_plan_call_pass_config(p, i, batch, w, cfg) != FWT_OK;
                        bad += fwt_plan_call_pass_config(p, i, -1, 1, cfg) != FWT_EINVAL;
                        sum += b;
                    }
                    bad += np > 0 && n > 0 && sum != n;
                    int64_t cv = -1;
                    bad += fwt_plan_chunk_vectors(p, 1 << 10, 1, &cv) != FWT_OK || cv < 0;
                    for (int64_t batch : {(int64_t)0, (int64_t)3, (int64_t)1 << 12})
                        for (int w = 0; w <= 1; ++w) {
                            int cp = -1, bb = -1;
                            int64_t bl = -1;
                            bad += fwt_plan_call_schedule(p, batch, w, &cp, &bb, &bl) != FWT_OK ||
                                   cp < 0 || cp > np || bb < 0 || bb > n || bl < 0;
                        }
                    {
                        int cp, bb;
                        int64_t bl;
                        bad += fwt_plan_call_schedule(p, -1, 1, &cp, &bb, &bl) != FWT_EINVAL;
                        bad += fwt_plan_call_schedule(p, 1, 1, nullptr, &bb, &bl) != FWT_EINVAL;
                    }
                    bad += fwt_plan_pass_bits(p, np, nullptr) == FWT_OK;
                    bad += fwt_plan_destroy(p) != FWT_OK;
                    ++ok;
                } else if (p != nullptr) {
                    ++bad;   // a failed create leaves no plan
                }
            }
    // Random splits and tunings, valid or not.
    for (int it = 0; it < 20000; ++it) {
        const int n = rnd(1, 30), d = rnd(0, 1), np = rnd(1, 5);
        int bits[5] = {0, 0, 0, 0, 0}, left = n;
        for (int i = 0; i < np - 1; ++i) {
            bits[i] = rnd(0, left);
            left -= bits[i];
        }
        bits[np - 1] = left;
        fwt_pass_tuning t[5];
        for (int i = 0; i < 5; ++i)
            t[i] = fwt_pass_tuning{rnd(-1, 6), rnd(-1, 5), rnd(-1, 3), rnd(-1, 2), rnd(-1, 3)};
        fwt_plan_t p = nullptr;
        const int st = fwt_plan_create_tuned(&p, n, (fwt_dtype)d, np, bits, rnd(0, 3) ? t : nullptr);
        if (st == FWT_OK) {
            int cfg[12], np2 = 0;
            fwt_plan_num_passes(p, &np2);
            for (int i = 0; i < np2; ++i) {
                bad += fwt_plan_pass_config(p, i, cfg) != FWT_OK;
                bad += fwt_plan_call_pass_config(p, i, rnd(0, 1 << 20), rnd(0, 1), cfg) != FWT_OK;
            }
            fwt_plan_destroy(p);
            ++ok;
        } else if (st != FWT_EINVAL && st != FWT_EUNSUPPORTED) {
            ++bad;
        }
    }
    // Validation that returns before any HIP call.
    fwt_plan_t p = nullptr;
    bad += fwt_plan_create(&p, 10, FWT_F32, FWT_PATH_AUTO) != FWT_OK;
    char buf[64];
    void* a = (void*)(((uintptr_t)buf + 15) & ~(uintptr_t)15);
    bad += fwt_execute(p, 1, 10, nullptr, nullptr, 1, nullptr) != FWT_EINVAL;
    bad += fwt_execute(p, -1, 10, a, nullptr, 1, nullptr) != FWT_EINVAL;
    bad += fwt_execute(p, 1, 9, a, nullptr, 1, nullptr) != FWT_EINVAL;
    bad += fwt_execute(p, 1, 10, (char*)a + 4, nullptr, 1, nullptr) != FWT_EALIGN;
    bad += fwt_execute(p, 1, 10, a, a, 1, nullptr) != FWT_EINVAL;
    bad += fwt_execute_check(nullptr, 1, 10, a, nullptr) != FWT_EINVAL;
    bad += fwt_execute(p, 0, 10, a, nullptr, 1, nullptr) != FWT_OK;   // batch 0: no-op
    bad += fwt_plan_destroy(nullptr) != FWT_OK;
    bad += fwt_plan_destroy(p) != FWT_OK;
    for (int s = -10; s <= 2; ++s)
        bad += fwt_strerror(s) == nullptr || std::strlen(fwt_strerror(s)) == 0;
    std::printf("planner driver: %d plans built, %s\n", ok, bad ? "MISMATCH" : "ok");
    return bad ? 1 : 0;
}
