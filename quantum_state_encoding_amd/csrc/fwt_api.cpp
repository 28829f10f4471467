// C ABI and planner for the batched in-place Walsh-Hadamard transform.
//
// The planner maps (n, dtype, path) to a list of passes over disjoint
// index-bit ranges whose union is [0, n): the Kronecker factorisation
// H_n = H_{n_p} (x) ... (x) H_{n_1} (Apache Mahout pull request
// "[QDP] [feature] Pr4 kronecker fwt", sections "Why" and "How", where the
// launcher splits n into two factors and dispatches by size; iThome
// "Day 18" native-FWT article, introduction: a single on-chip block while
// the state fits, a Kronecker split into several passes beyond).  The
// factors commute, so the order of the passes does not change the result;
// the lowest bits go first.  Every pass is an in-place streaming tile pass
// (fwt_kernels.hip); no pass transposes or needs a temporary buffer.
#include "../../include/fwt.h"

#include <hip/hip_runtime_api.h>

#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>

#include "fwt_internal.h"

using qse::KernelKey;
using qse::TileArgs;

namespace {

constexpr uint64_t kPlanMagic = 0x46575450'4c414e31ull;  // "FWTPLAN1"
constexpr int kMaxPasses = 4;
constexpr int kRowKrMax = 13;          // rows bits of a row pass (vectors)
constexpr int kColKrMax = 12;          // rows bits of a column pass
constexpr size_t kLdsMax = 160 * 1024; // per workgroup on gfx950
constexpr size_t kColLdsBudget = 128 * 1024;
constexpr int kTargetThreads = 256;    // workgroup size aimed for when packing tiles

struct Pass {
    int lo = 0;          // first index bit
    int k = 0;           // number of index bits
    int pair = 0;        // fp32 n = 1: two-element kernel
    KernelKey key{};
    int gbits = 0;       // log2 column groups per tile
    int nblk_bits = 0;   // log2 column blocks per outer index
    int tt_bits = 0;     // log2 threads per tile
    int tpw_bits = 0;    // log2 tiles per workgroup
    int store_back = 0;
    unsigned block = 0;
    size_t lds = 0;
    int tiles_bits = 0;  // log2 tiles per vector (per component)
};

}  // namespace

struct fwt_plan_s {
    uint64_t magic;
    int n;
    fwt_dtype dtype;
    int npasses;
    Pass passes[kMaxPasses];
};

namespace {

thread_local int t_last_hip = hipSuccess;

int hip_fail(hipError_t e)
{
    t_last_hip = (int)e;
    return FWT_EHIP;
}

int ilog2(int64_t v)
{
    int r = 0;
    while (((int64_t)1 << (r + 1)) <= v)
        ++r;
    return r;
}

int vec_bits(fwt_dtype d) { return d == FWT_F64 ? 1 : 2; }

int max_threads(int eb) { return eb >= 5 ? 512 : 1024; }

// Default register-round width for a pass of kr row bits.
int default_eb(int kr) { return kr < 4 ? kr : 4; }

bool log_enabled()
{
    const char* s = std::getenv("FWT_LOG");
    return s && s[0] && s[0] != '0';
}

// Fill in the tiling of a pass over bits [lo, lo + k) of a 2^n vector.
// eb_req / gbits_req < 0 select defaults.  Returns FWT_OK or an error.
int build_pass(Pass& p, int n, fwt_dtype dtype, int lo, int k, int eb_req, int gbits_req)
{
    const int vb = vec_bits(dtype);
    p = Pass{};
    p.lo = lo;
    p.k = k;
    if (dtype == FWT_F32 && n == 1) {
        p.pair = 1;
        return FWT_OK;
    }
    const bool row = (lo == 0);
    int kr, gbits;
    if (row) {
        if (k < vb)
            return FWT_EINVAL;
        kr = k - vb;
        if (kr > kRowKrMax)
            return FWT_EINVAL;
        gbits = 0;
        if (gbits_req > 0)
            return FWT_EINVAL;
    } else {
        if (lo < vb)
            return FWT_EINVAL;
        kr = k;
        if (kr < 1 || kr > kColKrMax)
            return FWT_EINVAL;
    }
    int eb = eb_req < 0 ? default_eb(kr) : eb_req;
    if (eb > kr || eb < 0)
        return FWT_EINVAL;
    if (!row) {
        const int gmax_cols = lo - vb;  // log2 16-byte groups in a row
        if (gbits_req >= 0) {
            gbits = gbits_req;
            if (gbits > gmax_cols)
                return FWT_EINVAL;
        } else {
            gbits = 0;
            while (gbits < 4 && gbits < gmax_cols &&
                   ((size_t)16 << (kr + gbits + 1)) <= kColLdsBudget &&
                   (kr - eb) + gbits + 1 <= ilog2(max_threads(eb)))
                ++gbits;
        }
        p.nblk_bits = gmax_cols - gbits;
    }
    p.key = KernelKey{dtype == FWT_F64 ? 1 : 0, kr, eb, gbits, row ? 1 : 0};
    p.gbits = gbits;
    p.tt_bits = (kr - eb) + gbits;
    if (p.tt_bits > ilog2(max_threads(eb)))
        return FWT_EINVAL;
    const int nr = qse::rounds_of(kr, eb);
    // LDS of one tile: 2^(kr + gbits) 16-byte slots plus one pad slot per
    // 2^(eb + gbits) slots.
    const size_t slots = (size_t)1 << (kr + gbits);
    const size_t tile_lds = 16 * (slots + (slots >> (eb + gbits)));
    // Pack tiles into a workgroup of about kTargetThreads threads.
    int tpw_bits = 0;
    while (p.tt_bits + tpw_bits < ilog2(kTargetThreads))
        ++tpw_bits;
    p.store_back = qse::store_back(kr, eb, gbits) ? 1 : 0;
    const bool needs_lds = nr > 1;
    if (needs_lds) {
        if (tile_lds > kLdsMax)
            return FWT_EINVAL;
        while (tpw_bits > 0 && (tile_lds << tpw_bits) > kLdsMax)
            --tpw_bits;
    }
    if (!row) {
        // Tiles of one workgroup stay inside one outer index unless there
        // are fewer column blocks than tiles per workgroup.
        if (tpw_bits > p.nblk_bits && p.nblk_bits < 0)
            return FWT_EINVAL;
    }
    // Lanes address from the workgroup's first tile with 32-bit byte
    // offsets; the largest one must fit.
    {
        const int esize_bits = dtype == FWT_F64 ? 3 : 2;
        const uint64_t tmax = ((uint64_t)1 << tpw_bits) - 1;
        uint64_t max_el;
        if (row) {
            max_el = ((tmax + 1) << k) - 1;
        } else {
            const uint64_t mask = ((uint64_t)1 << p.nblk_bits) - 1;
            max_el = ((tmax >> p.nblk_bits) << (lo + kr)) + ((tmax & mask) << (gbits + vb)) +
                     ((((uint64_t)1 << kr) - 1) << lo) + ((uint64_t)1 << (gbits + vb)) - 1;
        }
        if ((max_el << esize_bits) + ((uint64_t)1 << esize_bits) - 1 > 0xFFFFFFFFull)
            return FWT_EUNSUPPORTED;
    }
    if (!qse::kernel_available(p.key))
        return FWT_EUNSUPPORTED;
    p.tpw_bits = tpw_bits;
    p.block = 1u << (p.tt_bits + tpw_bits);
    p.lds = needs_lds ? (tile_lds << tpw_bits) : 0;
    p.tiles_bits = row ? (n - k) : (n - lo - k) + p.nblk_bits;
    return FWT_OK;
}

// Default Kronecker split (bit counts, lowest bits first).
int default_split(int n, fwt_dtype dtype, fwt_path path, int* bits)
{
    const int vb = vec_bits(dtype);
    const int single_max = kRowKrMax - 1 + vb;   // 64 KiB tiles: 14 fp32, 13 fp64
    if (path == FWT_PATH_SINGLE_BLOCK) {
        if (n > single_max + 1)
            return -1;
        bits[0] = n;
        return 1;
    }
    if (n <= 1 || (path == FWT_PATH_AUTO && n <= single_max) ||
        (path == FWT_PATH_MULTIPASS && n < 2 + vb)) {
        bits[0] = n;
        return 1;
    }
    if (path == FWT_PATH_MULTIPASS && n <= single_max) {
        bits[1] = n / 2 < n - vb ? n / 2 : n - vb;   // column factor
        bits[0] = n - bits[1];
        return 2;
    }
    if (n <= 12 + kColKrMax) {
        // Two passes: a 12-bit row pass on the contiguous low bits, then
        // one column pass on the rest.
        bits[0] = 12;
        bits[1] = n - 12;
        return 2;
    }
    // Three passes: 10 row bits, the rest split evenly (n <= 30).
    const int rest = n - 10;
    bits[0] = 10;
    bits[1] = rest - rest / 2;
    bits[2] = rest / 2;
    return 3;
}

int make_plan(fwt_plan_t* out, int n, fwt_dtype dtype, int npasses, const int* bits,
              const int* ebs, const int* gbits)
{
    if (!out)
        return FWT_EINVAL;
    *out = nullptr;
    if (n < 0 || n > FWT_MAX_N || (dtype != FWT_F32 && dtype != FWT_F64))
        return FWT_EINVAL;
    if (npasses < 1 || npasses > kMaxPasses || !bits)
        return FWT_EINVAL;
    int sum = 0;
    for (int i = 0; i < npasses; ++i) {
        if (bits[i] < (n == 0 ? 0 : 1))
            return FWT_EINVAL;
        sum += bits[i];
    }
    if (sum != n)
        return FWT_EINVAL;
    fwt_plan_s* p = new (std::nothrow) fwt_plan_s;
    if (!p)
        return FWT_ENOMEM;
    p->magic = kPlanMagic;
    p->n = n;
    p->dtype = dtype;
    p->npasses = n == 0 ? 0 : npasses;
    int lo = 0;
    for (int i = 0; i < p->npasses; ++i) {
        const int rc = build_pass(p->passes[i], n, dtype, lo, bits[i], ebs ? ebs[i] : -1,
                                  gbits ? gbits[i] : -1);
        if (rc != FWT_OK) {
            delete p;
            return rc;
        }
        lo += bits[i];
    }
    if (log_enabled()) {
        std::fprintf(stderr, "[fwt] plan n=%d dtype=%s passes=%d\n", n,
                     dtype == FWT_F64 ? "f64" : "f32", p->npasses);
        for (int i = 0; i < p->npasses; ++i) {
            const Pass& q = p->passes[i];
            std::fprintf(stderr,
                         "[fwt]   pass %d: bits [%d,%d) %s kr=%d eb=%d G=%d threads/tile=%d "
                         "block=%u lds=%zu store_back=%d tiles/vec=2^%d\n",
                         i, q.lo, q.lo + q.k, q.pair ? "pair" : (q.key.row ? "row" : "col"),
                         q.key.kr, q.key.eb, 1 << q.gbits, 1 << q.tt_bits, q.block, q.lds,
                         q.store_back, q.tiles_bits);
        }
    }
    *out = p;
    return FWT_OK;
}

bool valid_plan(fwt_plan_t p) { return p && p->magic == kPlanMagic; }

std::mutex g_init_mutex;
std::atomic<uint64_t> g_init_devices{0};

int ensure_device_init()
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e);
    if (dev < 64 && (g_init_devices.load(std::memory_order_acquire) >> dev) & 1)
        return FWT_OK;
    std::lock_guard<std::mutex> lock(g_init_mutex);
    if (dev < 64 && (g_init_devices.load() >> dev) & 1)
        return FWT_OK;
    e = qse::kernels_init_device();
    if (e != hipSuccess)
        return hip_fail(e);
    if (dev < 64)
        g_init_devices.fetch_or((uint64_t)1 << dev);
    return FWT_OK;
}

// The buffer must be device-visible memory holding [ptr, ptr + bytes).
int check_range(const void* ptr, size_t bytes)
{
    hipDeviceptr_t base = nullptr;
    size_t size = 0;
    hipError_t e = hipMemGetAddressRange(&base, &size, (hipDeviceptr_t)ptr);
    if (e != hipSuccess) {
        t_last_hip = (int)e;
        (void)hipGetLastError();  // do not leave the lookup's error behind
        if (e == hipErrorNoDevice || e == hipErrorNotInitialized ||
            e == hipErrorInsufficientDriver)
            return FWT_EHIP;
        return FWT_EINVAL;
    }
    const uintptr_t b = (uintptr_t)base, p = (uintptr_t)ptr;
    if (p < b || p - b > size || size - (p - b) < bytes)
        return FWT_EINVAL;
    return FWT_OK;
}

double norm_constant(int n)
{
    if (n % 2 == 0)
        return std::ldexp(1.0, -(n / 2));
    return std::ldexp(std::sqrt(0.5), -((n - 1) / 2));
}

// Host-side validation shared by fwt_execute and fwt_execute_check.  Sets
// *nothing_to_do for batch == 0 or n == 0.
int validate(fwt_plan_t plan, int64_t batch, int n, const void* re, const void* im,
             bool* nothing_to_do)
{
    *nothing_to_do = false;
    if (!valid_plan(plan) || !re)
        return FWT_EINVAL;
    if (batch < 0 || n != plan->n)
        return FWT_EINVAL;
    if (((uintptr_t)re & 15u) || ((uintptr_t)im & 15u))
        return FWT_EALIGN;
    if (re == im)
        return FWT_EINVAL;
    const size_t esize = plan->dtype == FWT_F64 ? 8 : 4;
    const int64_t N = (int64_t)1 << n;
    if (batch > INT64_MAX / N / (int64_t)esize)
        return FWT_EINVAL;
    const size_t bytes = (size_t)batch * (size_t)N * esize;
    if (im) {
        const uintptr_t a = (uintptr_t)re, b = (uintptr_t)im;
        if ((a < b && b - a < bytes) || (b < a && a - b < bytes))
            return FWT_EINVAL;
    }
    if (batch == 0 || plan->npasses == 0) {
        *nothing_to_do = true;
        return FWT_OK;
    }
    int rc = check_range(re, bytes);
    if (rc == FWT_OK && im)
        rc = check_range(im, bytes);
    return rc;
}

}  // namespace

extern "C" {

int fwt_plan_create(fwt_plan_t* out, int n, fwt_dtype dtype, fwt_path path)
{
    if (!out)
        return FWT_EINVAL;
    *out = nullptr;
    if (n < 0 || n > FWT_MAX_N || (dtype != FWT_F32 && dtype != FWT_F64))
        return FWT_EINVAL;
    if (path == FWT_PATH_MFMA_ABLATION)
        return FWT_EUNSUPPORTED;
    if (path != FWT_PATH_AUTO && path != FWT_PATH_SINGLE_BLOCK && path != FWT_PATH_MULTIPASS)
        return FWT_EINVAL;
    int bits[kMaxPasses] = {0, 0, 0, 0};
    const int np = default_split(n, dtype, path, bits);
    if (np < 0)
        return FWT_EUNSUPPORTED;
    return make_plan(out, n, dtype, np, bits, nullptr, nullptr);
}

int fwt_plan_create_split(fwt_plan_t* out, int n, fwt_dtype dtype, int npasses, const int* bits)
{
    return make_plan(out, n, dtype, npasses, bits, nullptr, nullptr);
}

int fwt_plan_create_tuned(fwt_plan_t* out, int n, fwt_dtype dtype, int npasses, const int* bits,
                          const int* eb, const int* gbits)
{
    return make_plan(out, n, dtype, npasses, bits, eb, gbits);
}

int fwt_execute_check(fwt_plan_t plan, int64_t batch, int n, const void* re, const void* im)
{
    bool nothing = false;
    return validate(plan, batch, n, re, im, &nothing);
}

namespace {

// Enqueue passes [first, last) of a validated call.
int launch_passes(fwt_plan_t plan, int first, int last, int64_t batch, int n, void* re, void* im,
                  int normalize, hipStream_t stream)
{
    int rc = ensure_device_init();
    if (rc != FWT_OK)
        return rc;
    const int ncomp = im ? 2 : 1;
    const double c = norm_constant(n);
    for (int i = first; i < last; ++i) {
        const Pass& p = plan->passes[i];
        const bool final_pass = (i == plan->npasses - 1);
        const int do_scale = (normalize && final_pass) ? 1 : 0;
        hipError_t e;
        if (p.pair) {
            e = qse::launch_pair_f32((float*)re, (float*)im, batch, do_scale, (float)c, stream);
        } else {
            TileArgs a{};
            a.tiles = batch << p.tiles_bits;
            a.wg_count = (a.tiles + ((int64_t)1 << p.tpw_bits) - 1) >> p.tpw_bits;
            a.lo = p.lo;
            a.nblk_bits = p.nblk_bits;
            a.tpw_bits = p.tpw_bits;
            a.tt_bits = p.tt_bits;
            a.do_scale = do_scale;
            a.scale = plan->dtype == FWT_F64 ? c : (double)(float)c;
            e = qse::launch_tile_pass(p.key, re, im, ncomp, a, p.block, p.lds, stream);
        }
        if (e != hipSuccess)
            return hip_fail(e);
    }
    return FWT_OK;
}

}  // namespace

int fwt_execute(fwt_plan_t plan, int64_t batch, int n, void* re, void* im, int normalize,
                hipStream_t stream)
{
    bool nothing = false;
    const int rc = validate(plan, batch, n, re, im, &nothing);
    if (rc != FWT_OK || nothing)
        return rc;
    return launch_passes(plan, 0, plan->npasses, batch, n, re, im, normalize, stream);
}

int fwt_execute_pass(fwt_plan_t plan, int pass, int64_t batch, int n, void* re, void* im,
                     int normalize, hipStream_t stream)
{
    if (!valid_plan(plan) || pass < 0 || pass >= (plan->npasses > 0 ? plan->npasses : 1))
        return FWT_EINVAL;
    bool nothing = false;
    const int rc = validate(plan, batch, n, re, im, &nothing);
    if (rc != FWT_OK || nothing)
        return rc;
    return launch_passes(plan, pass, pass + 1, batch, n, re, im, normalize, stream);
}

int fwt_plan_num_passes(fwt_plan_t plan, int* out_passes)
{
    if (!valid_plan(plan) || !out_passes)
        return FWT_EINVAL;
    *out_passes = plan->npasses;
    return FWT_OK;
}

int fwt_plan_pass_bits(fwt_plan_t plan, int i, int* out_bits)
{
    if (!valid_plan(plan) || !out_bits || i < 0 || i >= plan->npasses)
        return FWT_EINVAL;
    *out_bits = plan->passes[i].k;
    return FWT_OK;
}

int fwt_plan_destroy(fwt_plan_t plan)
{
    if (!plan)
        return FWT_OK;
    if (!valid_plan(plan))
        return FWT_EINVAL;
    plan->magic = 0;
    delete plan;
    return FWT_OK;
}

const char* fwt_strerror(int status)
{
    switch (status) {
    case FWT_OK: return "success";
    case FWT_EINVAL: return "invalid argument";
    case FWT_EALIGN: return "buffer not 16-byte aligned";
    case FWT_EUNSUPPORTED: return "unsupported configuration";
    case FWT_EHIP: return "HIP runtime error";
    case FWT_ENOMEM: return "out of host memory";
    default: return "unknown status";
    }
}

int fwt_last_hip_error(void) { return t_last_hip; }

int fwt_stream_copy(void* dst, const void* src, int64_t bytes, hipStream_t stream)
{
    if (!dst || !src || bytes < 0 || (bytes & 15))
        return FWT_EINVAL;
    if (((uintptr_t)dst & 15u) || ((uintptr_t)src & 15u))
        return FWT_EALIGN;
    const uintptr_t a = (uintptr_t)dst, b = (uintptr_t)src;
    if ((a <= b && b - a < (uint64_t)bytes) || (b < a && a - b < (uint64_t)bytes))
        return FWT_EINVAL;
    if (bytes == 0)
        return FWT_OK;
    int rc = check_range(dst, (size_t)bytes);
    if (rc == FWT_OK)
        rc = check_range(src, (size_t)bytes);
    if (rc != FWT_OK)
        return rc;
    const hipError_t e = qse::launch_stream_copy(dst, src, bytes, stream);
    return e == hipSuccess ? FWT_OK : hip_fail(e);
}

}  // extern "C"
