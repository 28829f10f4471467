// Host-only check of the launch schedule of fwt_execute, with the kernels
// stubbed (kernel_stubs.cpp) and a fake HIP runtime below, so it runs on a
// machine without a GPU.  For every plan and batch tried, the recorded
// tile-pass launches must:
//  * cover, pass by pass, every tile of the whole state exactly once (the
//    tile origins of all launches of a pass, taken relative to the state,
//    are exactly those of one launch over the whole state);
//  * keep each launch of a chunked pass inside its chunk of blocks, and
//    every launch inside the buffers;
//  * come in the order fwt_plan_call_schedule states (per chunk, the
//    chunked passes in order; then the other passes over the whole state);
//  * scale only in the last pass, and use nontemporal loads only in the
//    first pass and nontemporal stores only in the last one of a
//    multi-pass plan;
//  * put re and im at the same offset of their buffers;
//  * place workgroups by XCD only on launches over less than the 256 MiB
//    Infinity Cache, through a permutation of the launch's workgroups
//    that keeps every vector component on one XCD.
// Nothing is dereferenced: the buffers are address ranges only.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <vector>

#include "../../include/fwt.h"
#include "stub_hooks.h"

// ---- a fake HIP runtime: one device, allocations from a registry --------

namespace {
struct Range {
    uintptr_t base;
    size_t size;
};
std::vector<Range> g_ranges;
}  // namespace

hipError_t hipGetDevice(int* d)
{
    *d = 0;
    return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t, int)
{
    *v = 256;
    return hipSuccess;
}
hipError_t hipStreamGetDevice(hipStream_t, hipDevice_t* d)
{
    *d = 0;
    return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }
hipError_t hipGetLastError(void) { return hipSuccess; }
hipError_t hipMemcpy(void*, const void*, size_t, hipMemcpyKind) { return hipErrorNotSupported; }
hipError_t hipMemGetAddressRange(hipDeviceptr_t* base, size_t* size, hipDeviceptr_t p)
{
    const uintptr_t a = (uintptr_t)p;
    for (const Range& r : g_ranges)
        if (a >= r.base && a - r.base < r.size) {
            *base = (hipDeviceptr_t)r.base;
            *size = r.size;
            return hipSuccess;
        }
    return hipErrorInvalidValue;
}

// ---- recorded launches ----------------------------------------------------

namespace {

struct Launch {
    qse::KernelKey key;
    uintptr_t re, im;
    int ncomp;
    qse::TileArgs a;
};
std::vector<Launch> g_launches;

hipError_t record(const qse::KernelKey& key, void* re, void* im, int ncomp,
                  const qse::TileArgs& a, unsigned, size_t)
{
    g_launches.push_back(Launch{key, (uintptr_t)re, (uintptr_t)im, ncomp, a});
    return hipSuccess;
}

int g_bad = 0;
int g_vector_chunked = 0, g_block_chunked = 0;   // cases of each schedule kind
int g_xcd_launches = 0;                           // launches with XCD-affine placement
int g_wt_launches = 0;                            // launches with device-scope stores
int g_nt_launches = 0;                            // launches with nontemporal stores
#define EXPECT(c, ...)                                                           \
    do {                                                                         \
        if (!(c)) {                                                              \
            if (g_bad < 20) {                                                    \
                std::printf("FAIL line %d: %s | ", __LINE__, #c);                \
                std::printf(__VA_ARGS__);                                        \
                std::printf("\n");                                               \
            }                                                                    \
            ++g_bad;                                                             \
        }                                                                        \
    } while (0)

struct PassInfo {
    int lo, k, row, kr, gbits;
};

// Element origin (within a component) of tile t of a pass, and its last
// element + 1, relative to the launch's base pointer.
void tile_span(const PassInfo& p, int vb, int nblk, int64_t t, int64_t* first, int64_t* end)
{
    if (p.row) {
        *first = t << p.k;
        *end = *first + ((int64_t)1 << p.k);
        return;
    }
    const int64_t o = t >> nblk, c = t & (((int64_t)1 << nblk) - 1);
    *first = (o << (p.lo + p.kr)) + (c << (p.gbits + vb));
    *end = *first + ((((int64_t)1 << p.kr) - 1) << p.lo) + ((int64_t)1 << (p.gbits + vb));
}

void check_case(fwt_plan_t plan, int n, fwt_dtype dt, int64_t batch, bool with_im, int normalize)
{
    const int vb = dt == FWT_F64 ? 1 : 2;
    const size_t esize = dt == FWT_F64 ? 8 : 4;
    const int64_t N = (int64_t)1 << n;
    const size_t bytes = (size_t)batch * (size_t)N * esize;
    const uintptr_t A = (uintptr_t)1 << 44, B = A + ((bytes + 4095) & ~(size_t)4095) + 4096;
    g_ranges.assign({Range{A, bytes}, Range{B, bytes}});
    g_launches.clear();
    const int rc = fwt_execute(plan, batch, n, (void*)A, with_im ? (void*)B : nullptr, normalize,
                               nullptr);
    EXPECT(rc == FWT_OK, "n=%d batch=%lld rc=%d", n, (long long)batch, rc);
    if (rc != FWT_OK)
        return;
    int np = 0;
    fwt_plan_num_passes(plan, &np);
    std::vector<PassInfo> pi(np);
    for (int i = 0; i < np; ++i) {
        int c[12];
        fwt_plan_call_pass_config(plan, i, batch, with_im, c);
        pi[i] = PassInfo{c[0], c[1], c[2] == 0, c[3], c[5]};
    }
    int chunked = 0, bbits = 0;
    int64_t blocks = 0;
    fwt_plan_call_schedule(plan, batch, with_im, &chunked, &bbits, &blocks);
    if (chunked)
        ++(bbits == n ? g_vector_chunked : g_block_chunked);
    // The expected sequence of pass indices.
    std::vector<int> want;
    if (chunked == 0) {
        for (int i = 0; i < np; ++i)
            want.push_back(i);
    } else {
        const int64_t nblocks = batch << (n - bbits);
        for (int64_t b0 = 0; b0 < nblocks; b0 += blocks)
            for (int i = 0; i < chunked; ++i)
                want.push_back(i);
        for (int i = chunked; i < np; ++i)
            want.push_back(i);
    }
    EXPECT(g_launches.size() == want.size(), "n=%d batch=%lld launches %zu want %zu", n,
           (long long)batch, g_launches.size(), want.size());
    if (g_launches.size() != want.size())
        return;
    std::vector<std::vector<int64_t>> got(np);
    std::vector<int64_t> total(np);   // tiles of each pass over the whole state
    for (int i = 0; i < np; ++i) {
        const int nblk = pi[i].row ? 0 : pi[i].lo - vb - pi[i].gbits;
        total[i] = batch * (pi[i].row ? ((int64_t)1 << (n - pi[i].k))
                                      : ((int64_t)1 << (n - pi[i].lo - pi[i].k + nblk)));
    }
    const int64_t chunk_elems = chunked ? blocks << bbits : batch * N;
    for (size_t j = 0; j < g_launches.size(); ++j) {
        const Launch& L = g_launches[j];
        const int i = want[j];
        const PassInfo& p = pi[i];
        EXPECT(L.a.lo == p.lo && L.key.row == p.row && L.key.kr == p.kr, "pass %d order", i);
        EXPECT(L.ncomp == (with_im ? 2 : 1), "ncomp");
        EXPECT(!with_im || L.im - B == L.re - A, "im offset");
        EXPECT(L.re >= A && (L.re - A) % esize == 0, "re base");
        const int64_t e0 = (int64_t)((L.re - A) / esize);
        const bool last = i == np - 1;
        EXPECT(L.a.do_scale == (last && normalize ? 1 : 0), "scale flag, pass %d", i);
        if (L.a.do_scale) {
            const double c = std::ldexp(1.0, -(n / 2)) * (n % 2 ? std::sqrt(0.5) : 1.0);
            const double want_c = dt == FWT_F64 ? c : (double)(float)c;
            EXPECT(L.a.scale == want_c, "scale value n=%d", n);
        }
        EXPECT(L.a.ld_nt == (np > 1 && i == 0 ? 1 : 0), "nontemporal loads, pass %d", i);
        // Stores of a multi-pass plan: the last pass nontemporal in chunked
        // schedules (states past 256 MiB); earlier passes with device scope
        // once the state exceeds 32 MiB, if their tiles have at most 2^10
        // slots.
        const size_t bytes = (size_t)batch * (size_t)N * esize * (with_im ? 2 : 1);
        EXPECT(np < 2 || (chunked != 0) == (bytes > ((size_t)256 << 20)),
               "multi-pass calls chunked past 256 MiB");
        const int want_st =
            np < 2 ? qse::kStorePlain
            : last ? (chunked ? qse::kStoreNontemporal : qse::kStorePlain)
                   : (bytes > ((size_t)32 << 20) && p.kr + p.gbits <= 10 ? qse::kStoreWriteThrough
                                                                        : qse::kStorePlain);
        EXPECT(L.a.st_policy == want_st, "store policy %d, want %d, pass %d", L.a.st_policy,
               want_st, i);
        g_wt_launches += L.a.st_policy == qse::kStoreWriteThrough;
        g_nt_launches += L.a.st_policy == qse::kStoreNontemporal;
        EXPECT(L.a.tile0 == 0 && L.a.tiles > 0, "tiles");
        EXPECT(L.a.wg_count == (L.a.tiles + ((int64_t)1 << L.a.tpw_bits) - 1) >> L.a.tpw_bits,
               "workgroups");
        // XCD-affine placement: only on states that fit the L2s, with whole
        // vector components per workgroup group, and a permutation of the
        // launch's workgroups that keeps each component on one XCD.
        if (L.a.xcd_bits >= 0) {
            ++g_xcd_launches;
            const int xb = L.a.xcd_bits;
            // the launch's own vectors, below the Infinity Cache's 256 MiB
            const int64_t lb = L.a.tiles / (total[i] / batch);
            EXPECT((size_t)lb * (size_t)N * esize * (with_im ? 2 : 1) < ((size_t)256 << 20),
                   "xcd placement on a launch of %lld vectors", (long long)lb);
            EXPECT(!L.key.pipe && xb < 30 && L.a.wg_count >= ((int64_t)8 << xb) &&
                       ((L.a.tiles >> L.a.tpw_bits) << L.a.tpw_bits) == L.a.tiles,
                   "xcd placement shape");
            if (L.a.wg_count <= ((int64_t)1 << 22)) {
                const int64_t tpv = total[i] / batch;   // tiles per vector component
                const int64_t span = L.a.wg_count & ~(((int64_t)8 << xb) - 1);
                std::vector<char> seen((size_t)L.a.wg_count, 0);
                for (int64_t w = 0; w < L.a.wg_count; ++w) {
                    const int64_t g = qse::xcd_group(w, xb, L.a.wg_count);
                    EXPECT(g >= 0 && g < L.a.wg_count && !seen[(size_t)g], "xcd map w=%lld",
                           (long long)w);
                    if (g >= 0 && g < L.a.wg_count)
                        seen[(size_t)g] = 1;
                    const int64_t v = (g << L.a.tpw_bits) / tpv;   // its vector component
                    EXPECT(w >= span || w % 8 == v % 8, "xcd map: w=%lld holds component %lld",
                           (long long)w, (long long)v);
                    EXPECT(w < span || g == w, "xcd map: tail w=%lld moved", (long long)w);
                }
            }
        }
        // the chunk this launch may touch
        int64_t lo_e = 0, hi_e = batch * N;
        if (i < chunked) {
            EXPECT(e0 % chunk_elems == 0, "chunk start");
            lo_e = e0;
            hi_e = std::min(batch * N, e0 + chunk_elems);
        } else {
            EXPECT(e0 == 0, "whole-state pass starts at the state");
        }
        EXPECT(L.a.tiles <= total[i], "pass %d launch of %lld tiles, the state has %lld", i,
               (long long)L.a.tiles, (long long)total[i]);
        if (L.a.tiles > total[i] || (int64_t)got[i].size() + L.a.tiles > total[i])
            continue;   // too many tiles: already wrong, do not enumerate them
        for (int64_t t = 0; t < L.a.tiles; ++t) {
            int64_t f, e;
            tile_span(p, vb, L.a.nblk_bits, t, &f, &e);
            EXPECT(e0 + f >= lo_e && e0 + e <= hi_e, "pass %d tile %lld outside [%lld, %lld)", i,
                   (long long)t, (long long)lo_e, (long long)hi_e);
            got[i].push_back(e0 + f);
        }
    }
    // Every tile of the whole state exactly once per pass.
    for (int i = 0; i < np; ++i) {
        const PassInfo& p = pi[i];
        const int nblk = p.row ? 0 : p.lo - vb - p.gbits;
        std::vector<int64_t> exp;
        exp.reserve((size_t)total[i]);
        for (int64_t t = 0; t < total[i]; ++t) {
            int64_t f, e;
            tile_span(p, vb, nblk, t, &f, &e);
            exp.push_back(f);
        }
        std::sort(got[i].begin(), got[i].end());
        EXPECT(got[i] == exp, "pass %d of n=%d batch=%lld: %zu tiles, want %zu", i, n,
               (long long)batch, got[i].size(), exp.size());
    }
}

// The cache hints of single-pass calls: fwt_execute's, with a state of
// 256 MiB or more taken as one chunk of a chunked call.
void check_pass_hints()
{
    fwt_plan_t plan = nullptr;
    EXPECT(fwt_plan_create(&plan, 20, FWT_F32, FWT_PATH_AUTO) == FWT_OK, "plan n=20");
    int np = 0;
    fwt_plan_num_passes(plan, &np);
    EXPECT(np == 2, "n=20 passes %d", np);
    const size_t vec = (size_t)4 << 20;   // one fp32 component of 2^20
    const uintptr_t A = (uintptr_t)1 << 44, B = A + 32 * vec + 4096;
    g_ranges.assign({Range{A, 32 * vec}, Range{B, 32 * vec}});
    hipEvent_t ev = reinterpret_cast<hipEvent_t>(&g_bad);   // never dereferenced
    struct Want {
        int pass;
        int64_t batch;
        bool timed;
        int policy;
    } const wants[] = {
        {1, 32, false, qse::kStoreNontemporal},   // 256 MiB: a chunk of a larger call
        {1, 32, true, qse::kStoreNontemporal},
        {1, 31, false, qse::kStorePlain},
        {0, 32, true, qse::kStoreWriteThrough},   // 12-bit row tiles of 2^10 slots
        {0, 2, false, qse::kStorePlain},          // 16 MiB: within the L2s
    };
    for (const Want& w : wants) {
        g_launches.clear();
        const int rc = w.timed ? fwt_execute_pass_timed(plan, w.pass, w.batch, 20, (void*)A,
                                                        (void*)B, 1, nullptr, ev, ev)
                               : fwt_execute_pass(plan, w.pass, w.batch, 20, (void*)A, (void*)B,
                                                  1, nullptr);
        EXPECT(rc == FWT_OK && g_launches.size() == 1, "pass %d batch %lld rc %d", w.pass,
               (long long)w.batch, rc);
        if (rc == FWT_OK && g_launches.size() == 1)
            EXPECT(g_launches[0].a.st_policy == w.policy, "pass %d batch %lld policy %d, want %d",
                   w.pass, (long long)w.batch, g_launches[0].a.st_policy, w.policy);
    }
    // the whole 256 MiB call is not chunked: its last pass stores plainly
    g_launches.clear();
    EXPECT(fwt_execute(plan, 32, 20, (void*)A, (void*)B, 1, nullptr) == FWT_OK &&
               g_launches.size() == 2 && g_launches[1].a.st_policy == qse::kStorePlain &&
               g_launches[0].a.st_policy == qse::kStoreWriteThrough,
           "fwt_execute on 256 MiB");
    fwt_plan_destroy(plan);
}

}  // namespace

int main()
{
    qse::g_tile_launch_hook = record;
    check_pass_hints();
    int cases = 0;
    const size_t cache = (size_t)256 << 20;
    for (int d = 0; d <= 1; ++d) {
        const fwt_dtype dt = (fwt_dtype)d;
        const size_t esize = d ? 8 : 4;
        const int nmax = 30;
        for (int n = 2; n <= nmax; ++n) {
            std::vector<std::vector<int>> splits = {{}};   // {} = the default plan
            if (n % 5 == 2 && n >= 12) {
                splits.push_back({n / 3, n / 3, n - 2 * (n / 3)});
                splits.push_back({n / 4, n / 4, n / 4, n - 3 * (n / 4)});
            }
            for (const auto& sp : splits) {
                fwt_plan_t plan = nullptr;
                const int rc = sp.empty()
                                   ? fwt_plan_create(&plan, n, dt, FWT_PATH_AUTO)
                                   : fwt_plan_create_split(&plan, n, dt, (int)sp.size(), sp.data());
                if (rc != FWT_OK)
                    continue;   // a split outside the per-pass limits
                const size_t vec = ((size_t)1 << n) * esize * 2;
                // small, ragged, past the cache (when the tile count stays
                // small), and for states below the cache a multiple of the 8
                // XCDs and a batch just past one
                std::vector<int64_t> batches = {1, 3};
                if (vec * 11 < ((size_t)256 << 20)) {
                    batches.push_back(8);
                    batches.push_back(11);
                }
                const int64_t big = (int64_t)(2 * cache / vec) + 3;
                if (big > 3 && big <= ((int64_t)1 << 12))
                    batches.push_back(big);
                if (vec > cache && n <= 28)
                    batches.push_back(2);
                for (int64_t batch : batches)
                    for (int w = 0; w <= 1; ++w) {
                        check_case(plan, n, dt, batch, w == 1, (int)(batch + n + w) % 2);
                        ++cases;
                    }
                fwt_plan_destroy(plan);
            }
        }
    }
    // both kinds of chunking must have been exercised
    EXPECT(g_vector_chunked >= 10 && g_block_chunked >= 10, "chunked cases: %d by vectors, %d by "
           "blocks", g_vector_chunked, g_block_chunked);
    EXPECT(g_xcd_launches >= 10, "XCD-affine launches: %d", g_xcd_launches);
    EXPECT(g_wt_launches >= 10 && g_nt_launches >= 10,
           "device-scope store launches: %d, nontemporal: %d", g_wt_launches, g_nt_launches);
    std::printf("schedule driver: %d cases (%d chunked by vectors, %d by blocks, %d launches "
                "placed by XCD, %d with device-scope and %d with nontemporal stores), %d "
                "failures%s\n", cases, g_vector_chunked, g_block_chunked, g_xcd_launches,
                g_wt_launches, g_nt_launches, g_bad, g_bad ? "" : " ok");
    return g_bad ? 1 : 0;
}
