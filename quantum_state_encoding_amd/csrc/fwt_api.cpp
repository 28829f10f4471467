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
// One-pass plans of this range of n use the wave-tile kernel by default.
constexpr int kWaveDefaultMin = 3;
constexpr int kWaveDefaultMax = 10;
// Row bits of the matrix-core ablation's block-Hadamard kernel: at least
// 8, at most what one padded tile in LDS holds.
constexpr int kMfmaRowMin = 8;
int mfma_row_max(fwt_dtype dtype) { return dtype == FWT_F64 ? 14 : 15; }
constexpr int kRowKrMax = 13;          // rows bits of a row pass (vectors)
constexpr int kLxDefaultMin = 8;       // lane-exchange kernel by default from here
constexpr int kColKrMax = 12;          // rows bits of a column pass
constexpr int kColPref = 9;            // column factor of the default two-pass split
constexpr int kColTwoPassMax = 11;     // widest column factor of a default two-pass plan
constexpr size_t kLdsMax = 160 * 1024; // per workgroup on gfx950
constexpr size_t kPhaseLdsTarget = 68 * 1024;  // two tiles per CU
constexpr size_t kChunkBytes = (size_t)256 << 20;  // Infinity Cache capacity
constexpr size_t kL2Bytes = (size_t)32 << 20;      // eight XCDs' L2s together
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
    int phb = 0;         // log2 exchange phases
    unsigned block = 0;
    size_t lds = 0;
    int tiles_bits = 0;  // log2 tiles per vector (per component)
    int mfma = 0;        // matrix-core block-Hadamard row pass (lo = 0)
};

}  // namespace

struct fwt_plan_s {
    uint64_t magic;
    int n;
    fwt_dtype dtype;
    int npasses;
    Pass passes[kMaxPasses];
    // One-pass plans only: the pass launched instead of passes[0] when the
    // call's state fits the Infinity Cache (has_small != 0).
    int has_small;
    Pass small;
    // Default fp32 n = 20 plans: fwt_execute_ws may run the whole transform
    // as one HBM pass (the group-of-workgroups kernel) on a workspace.
    int onepass;
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

// Default register-round width for a pass of kr row bits (measured on
// MI355X): 8 vectors per thread (more threads per tile: lower latency for
// single passes, more memory parallelism for streaming passes); 16 for
// fp64 rows of 12+ bits (32 in a single pass of 13) and fp64 column tiles
// of 9+ bits, and for any column tile of 11+ bits, where 8 per thread
// would exceed the thread limits of the pipelined or phased kernels.
int default_eb(int kr, fwt_dtype dtype, bool multipass, bool row)
{
    if (kr < 3)
        return kr;
    if (dtype == FWT_F64) {
        if (row && kr >= 13)
            return multipass ? 4 : 5;
        if (row && kr == 12)
            return 4;
        if (!row && kr >= 9)
            return 4;
    }
    if (!row && kr >= 11)
        return 4;   // keeps 8 column groups (128-byte segments) within 1024 threads
    return 3;
}

bool log_enabled()
{
    const char* s = std::getenv("FWT_LOG");
    return s && s[0] && s[0] != '0';
}

// LDS bytes of one exchange phase of a tile: 2^(kr + gbits - phb) 16-byte
// slots plus one pad slot per 2^(eb + gbits - phb) slots.
size_t phase_lds(int kr, int eb, int gbits, int phb)
{
    const size_t slots = (size_t)1 << (kr + gbits - phb);
    return 16 * (slots + (slots >> (eb + gbits - phb)));
}

// Whether a column-pass variant with phased exchange exists (mirrors the
// instantiation rule in fwt_kernels.hip).
bool phases_allowed(int kr, int eb, int gbits, int phb)
{
    return phb == 0 || (kr >= 9 && gbits >= 3 && kr > eb && phb <= 2);
}

// Fill in the tiling of a pass over bits [lo, lo + k) of a 2^n vector.
// eb_req / gbits_req / phb_req < 0 select defaults.  Returns FWT_OK or an
// error.
int build_wave_pass(Pass& p, int n, fwt_dtype dtype, int lo, int k, int kr, bool row,
                    const fwt_pass_tuning& t);
int build_lx_pass(Pass& p, int n, fwt_dtype dtype, int lo, int k, int kr, bool row,
                  const fwt_pass_tuning& t, bool multipass);

// Largest 32-bit lane offset of a pass's tile group must fit (lanes address
// from the workgroup's first tile).  `split`: the kernel addresses the top
// half of each tile's rows from a second base (lane-exchange tiles whose
// top row bit stays a register bit), so offsets span half the rows.
// Returns FWT_OK or FWT_EUNSUPPORTED.
int check_offsets(const Pass& p, fwt_dtype dtype, bool row, int kr, int vb, bool split = false)
{
    const int esize_bits = dtype == FWT_F64 ? 3 : 2;
    const uint64_t tmax = ((uint64_t)1 << p.tpw_bits) - 1;
    const int krs = split ? kr - 1 : kr;   // row bits the lane offsets span
    uint64_t max_el;
    if (row) {
        max_el = split ? (((uint64_t)1 << (krs + vb)) - 1) : ((tmax + 1) << p.k) - 1;
    } else {
        const uint64_t mask = ((uint64_t)1 << p.nblk_bits) - 1;
        max_el = ((tmax >> p.nblk_bits) << (p.lo + kr)) + ((tmax & mask) << (p.gbits + vb)) +
                 ((((uint64_t)1 << krs) - 1) << p.lo) + ((uint64_t)1 << (p.gbits + vb)) - 1;
    }
    if ((max_el << esize_bits) + ((uint64_t)1 << esize_bits) - 1 > 0xFFFFFFFFull)
        return FWT_EUNSUPPORTED;
    return FWT_OK;
}

int build_pass(Pass& p, int n, fwt_dtype dtype, int lo, int k, const fwt_pass_tuning& t,
               bool multipass)
{
    const int eb_req = t.eb, gbits_req = t.gbits, phb_req = t.phases, pipe_req = t.pipe;
    const int vb = vec_bits(dtype);
    p = Pass{};
    p.lo = lo;
    p.k = k;
    if (dtype == FWT_F32 && n == 1) {
        p.pair = 1;
        return FWT_OK;
    }
    const bool row = (lo == 0);
    int kr;
    if (row) {
        if (k < vb)
            return FWT_EINVAL;
        kr = k - vb;
        // exchange phases of a row pass: the lane-exchange kernel only
        if (kr > kRowKrMax || gbits_req > 0 || (phb_req > 0 && t.wave != 2))
            return FWT_EINVAL;
    } else {
        if (lo < vb)
            return FWT_EINVAL;
        kr = k;
        if (kr < 1 || kr > kColKrMax)
            return FWT_EINVAL;
    }
    if (t.wave > 2 || t.pipe > 1)
        return FWT_EINVAL;
    if (t.wave == 1)
        return build_wave_pass(p, n, dtype, lo, k, kr, row, t);
    if (t.wave == 2)
        return build_lx_pass(p, n, dtype, lo, k, kr, row, t, multipass);
    // One-pass plans of 3 <= n <= 10 default to the wave-tile kernel: on
    // 512 MiB states it ran at 6.0 TB/s against 5.0-5.4 for the LDS tiles
    // (both dtypes), and on cache-resident batches 2-12 % faster.  From 11
    // bits its register tiles cost more than the LDS exchanges save.  (As
    // the row pass of a two-pass plan it gained 3-5 % on HBM-bound states
    // but lost up to 20 % on cache-resident ones, so it is not the default
    // there.)
    const bool all_default =
        t.eb < 0 && t.gbits < 0 && t.phases < 0 && t.pipe < 0 && t.wave < 0;
    if (all_default && row && !multipass && k >= kWaveDefaultMin && k <= kWaveDefaultMax) {
        const int rc = build_wave_pass(p, n, dtype, lo, k, kr, row, t);
        if (rc == FWT_OK)
            return rc;
        p = Pass{};
        p.lo = lo;
        p.k = k;
    }
    // Other row passes of 8..13 vector bits default to the lane-exchange
    // kernel: against the LDS tiles it took one-pass plans 4-22 % faster
    // (n = 11..15, cache-resident and 512 MiB states) and fp64 two-pass row
    // passes 1-5 % faster (n = 17..24).  Two-pass row passes of 11 vector
    // bits (fp32 n = 20..24, fp64 n = 20) measured 0.3-0.8 % slower in it
    // and stay on the LDS tiles.
    if (all_default && row && kr >= kLxDefaultMin && kr <= kRowKrMax &&
        !(multipass && kr == 11)) {
        const int rc = build_lx_pass(p, n, dtype, lo, k, kr, row, t, multipass);
        if (rc == FWT_OK)
            return rc;
        p = Pass{};
        p.lo = lo;
        p.k = k;
    }
    // Column passes of 8..11 bits with rows of at least 8 groups default to
    // it as well: measured 0.2-5.5 % faster per call (fp32 n = 19..25, fp64
    // n = 23..24; the n = 24 fp64 workload 2.9 %), and within 0.4 % at fp64
    // n = 20.  The 11-bit column factor (fp32 n = 26, fp64 n = 25, 2 GiB
    // states) took a call 13 % less time than on the LDS tiles.
    if (all_default && !row && kr >= 8 && kr <= 11 && lo - vec_bits(dtype) >= 3) {
        const int rc = build_lx_pass(p, n, dtype, lo, k, kr, row, t, multipass);
        if (rc == FWT_OK)
            return rc;
        p = Pass{};
        p.lo = lo;
        p.k = k;
    }
    // 7-bit column passes with rows of at least 16 groups: the lane-exchange
    // tile of 16 groups with eb = 2 (512 threads, one exchange) measured
    // 0.1-3.7 % faster than the LDS tiles on every state tried (fp32 n = 14
    // as 7|7 at 8-512 MiB, n = 17 at 16 MiB and 2 GiB, fp64 n = 16 at 16 MiB
    // and 1 GiB).  (At 6 bits it was mixed: up to 11 % slower.)
    if (all_default && !row && kr == 7 && lo - vec_bits(dtype) >= 4) {
        fwt_pass_tuning t7 = t;
        t7.eb = 2;
        t7.gbits = 4;
        t7.phases = 0;
        const int rc = build_lx_pass(p, n, dtype, lo, k, kr, row, t7, multipass);
        if (rc == FWT_OK)
            return rc;
        p = Pass{};
        p.lo = lo;
        p.k = k;
    }
    const int eb = eb_req < 0 ? default_eb(kr, dtype, multipass, row) : eb_req;
    // A round of LDS tiles butterflies eb register bits, so a tile with row
    // bits needs eb >= 1 (rounds_of divides by eb).
    if (eb > kr || eb < 0 || eb > 5 || (eb == 0 && kr > 0))
        return FWT_EINVAL;
    const int tt_max = ilog2(max_threads(eb));
    const int nr = qse::rounds_of(kr, eb);
    const bool needs_lds = nr > 1;
    int gbits = 0, phb = 0;
    if (!row) {
        const int gmax_cols = lo - vb;  // log2 16-byte groups in a row
        if (gbits_req > 4 || gbits_req > gmax_cols || phb_req > 2)
            return FWT_EINVAL;
        // Defaults: row segments of at least 128 bytes (8 groups) where the
        // rows allow it, then the fewest exchange phases, then the most
        // groups (up to 256-byte segments), such that one phase's LDS stays
        // near 64 KiB (two tiles per CU); failing that, up to the 160 KiB
        // limit; failing that, shorter segments.
        const int gb_top = gbits_req >= 0 ? gbits_req : (gmax_cols < 4 ? gmax_cols : 4);
        const int gb_min = gmax_cols < 3 ? gmax_cols : 3;
        const int ph_lo = phb_req >= 0 ? phb_req : 0;
        const int ph_hi = phb_req >= 0 ? phb_req : 2;
        bool found = false;
        for (int attempt = 0; attempt < 3 && !found; ++attempt) {
            const size_t limit = attempt == 0 ? kPhaseLdsTarget : kLdsMax;
            const int gb_lo = gbits_req >= 0 ? gbits_req : (attempt < 2 ? gb_min : 0);
            for (int ph = ph_lo; ph <= ph_hi && !found; ++ph) {
                for (int gb = gb_top; gb >= gb_lo && !found; --gb) {
                    if ((kr - eb) + gb > tt_max)
                        continue;
                    if (ph > gb || !phases_allowed(kr, eb, gb, ph))
                        continue;
                    if (needs_lds && phase_lds(kr, eb, gb, ph) > limit)
                        continue;
                    gbits = gb;
                    phb = needs_lds ? ph : 0;
                    found = true;
                }
            }
        }
        if (!found)
            return FWT_EINVAL;
        p.nblk_bits = gmax_cols - gbits;
    }
    if (pipe_req > 1)
        return FWT_EINVAL;
    p.key = KernelKey{dtype == FWT_F64 ? 1 : 0, kr, eb, gbits, phb, row ? 1 : 0, 0, 0};
    p.gbits = gbits;
    p.phb = phb;
    p.tt_bits = (kr - eb) + gbits;
    if (p.tt_bits > tt_max)
        return FWT_EINVAL;
    const size_t tile_lds = phase_lds(kr, eb, gbits, phb);
    // Pack tiles into a workgroup of about kTargetThreads threads.
    int tpw_bits = 0;
    while (p.tt_bits + tpw_bits < ilog2(kTargetThreads))
        ++tpw_bits;
    p.store_back = qse::store_back(kr, eb, gbits) ? 1 : 0;
    if (needs_lds) {
        if (tile_lds > kLdsMax)
            return FWT_EINVAL;
        while (tpw_bits > 0 && (tile_lds << tpw_bits) > kLdsMax)
            --tpw_bits;
    }
    // Lanes address from the workgroup's first tile with 32-bit byte
    // offsets; the largest one must fit.
    p.tpw_bits = tpw_bits;
    if (check_offsets(p, dtype, row, kr, vb) != FWT_OK)
        return FWT_EUNSUPPORTED;
    if (!qse::kernel_available(p.key))
        return FWT_EUNSUPPORTED;
    // Tiles so large that a CU holds one workgroup run in the persistent
    // software-pipelined kernel, which streams the next tile group in while
    // the current one is exchanged.
    {
        KernelKey pk = p.key;
        pk.pipe = 1;
        const bool one_per_cu = needs_lds && (tile_lds << tpw_bits) > kLdsMax / 2;
        const bool want = pipe_req >= 0 ? pipe_req == 1 : one_per_cu;
        const bool can = (1 << (p.tt_bits + tpw_bits)) <= 512 && qse::kernel_available(pk);
        if (want && can)
            p.key = pk;
        else if (want && pipe_req == 1)
            return FWT_EUNSUPPORTED;
    }
    p.tpw_bits = tpw_bits;
    p.block = 1u << (p.tt_bits + tpw_bits);
    p.lds = needs_lds ? (tile_lds << tpw_bits) : 0;
    p.tiles_bits = row ? (n - k) : (n - lo - k) + p.nblk_bits;
    return FWT_OK;
}

// A pass in the wave-tile kernel: each wave holds whole tiles, register bits
// [LB, kr) in registers and row bits [0, LB) in lanes (above the column-group
// lane bits), with lane stages instead of LDS exchanges; LB <= 6 - gbits.
int build_wave_pass(Pass& p, int n, fwt_dtype dtype, int lo, int k, int kr, bool row,
                    const fwt_pass_tuning& t)
{
    const int vb = vec_bits(dtype);
    if (t.phases > 0 || t.pipe > 0)
        return FWT_EINVAL;
    int gbits = 0;
    if (!row) {
        const int gmax_cols = lo - vb;
        if (t.gbits > 4 || t.gbits > gmax_cols)
            return FWT_EINVAL;
        // Default: 8 groups (128-byte segments) where the rows allow, else
        // as many as there are.
        gbits = t.gbits >= 0 ? t.gbits : (gmax_cols < 3 ? gmax_cols : 3);
        p.nblk_bits = gmax_cols - gbits;
    } else if (t.gbits > 0) {
        return FWT_EINVAL;
    }
    const int lane_room = 6 - gbits;
    int eb = t.eb >= 0 ? t.eb : (kr - lane_room > 0 ? kr - lane_room : 0);
    if (t.eb < 0 && eb == 0 && kr + gbits >= 5)
        eb = 1;   // lane bits 4 and 5 are swapped through register pairs
    const int lb = kr - eb;
    if (eb < 0 || eb > 5 || eb > kr || lb < 0 || lb > lane_room)
        return FWT_EINVAL;
    p.key = KernelKey{dtype == FWT_F64 ? 1 : 0, kr, eb, gbits, 0, row ? 1 : 0, 0, 1};
    if (!qse::kernel_available(p.key))
        return FWT_EUNSUPPORTED;
    p.gbits = gbits;
    p.phb = 0;
    p.tt_bits = gbits + lb;
    p.tpw_bits = 2 + (lane_room - lb);   // 4 waves of 2^(6 - gbits - lb) tiles
    p.block = 256;
    p.lds = 0;
    p.store_back = 0;
    p.tiles_bits = row ? (n - k) : (n - lo - k) + p.nblk_bits;
    return check_offsets(p, dtype, row, kr, vb);
}

// A pass in the lane-exchange kernel.  Row pass: a tile of 2^kr 16-byte
// vectors in a workgroup of 2^(6 + W) threads holding 2^eb vectors each,
// kr = eb + 6 + W, with 1 <= W <= 4 and 2 <= eb <= 5 (or eb = W = 1): lane
// stages for the 6 lowest row bits and ceil(W / eb) LDS exchanges.
// Default: the most threads with eb >= 2, W = min(4, kr - 8), and W = 1
// below 10 row bits (measured: best, or within 4 % of the best variant, at
// every n and batch tried); except the row pass of a multi-pass plan with a
// 128 KiB tile (kr = 13, fp64 n = 22..24): W = 3, eb = 4, one exchange in
// two phases through 64 KiB of LDS, so that two tiles share a CU (3.3 %
// faster there).  Column pass: 2^kr rows x 2^gbits 16-byte groups (gbits 3
// or 4: 128- or 256-byte row segments); lanes hold the groups and 6 - gbits
// row bits, kr = eb + (6 - gbits) + W.  Default (measured best for 7..10
// column bits): 16 groups while the tile fits 128 KiB of LDS, else 8;
// eb = 4 (W = 2 or 3); one exchange in two phases, so that a tile takes
// 64 KiB of LDS (32 KiB at 8 row bits) and two or more share a CU.  At 11
// column bits (8 groups, 128 KiB of slots) the two phases need W < eb:
// eb = 5, W = 3.
int build_lx_pass(Pass& p, int n, fwt_dtype dtype, int lo, int k, int kr, bool row,
                  const fwt_pass_tuning& t, bool multipass)
{
    const int vb = vec_bits(dtype);
    if (t.phases > 1 || t.pipe > 0)
        return FWT_EINVAL;
    int gbits = 0;
    if (row) {
        if (t.gbits > 0)
            return FWT_EINVAL;
    } else {
        const int gmax_cols = lo - vb;   // log2 16-byte groups in a row
        gbits = t.gbits >= 0 ? t.gbits : (kr + 4 <= 13 && gmax_cols >= 4 ? 4 : 3);
        if (gbits < 3 || gbits > 4 || gbits > gmax_cols)
            return FWT_EINVAL;
        p.nblk_bits = gmax_cols - gbits;
    }
    const int lr = 6 - gbits;   // row bits held by lanes
    const bool two_tiles = row && multipass && kr == 13;
    int eb;
    if (t.eb >= 0)
        eb = t.eb;
    else if (two_tiles)
        eb = 4;
    else if (row)
        eb = kr - 6 - (kr >= 10 ? (kr - 8 < 4 ? kr - 8 : 4) : 1);
    else if (kr + gbits > 13)
        eb = (kr - lr + 2) / 2;   // two phases: w < eb
    else
        eb = kr - lr - 1 < 4 ? kr - lr - 1 : 4;
    const int w = kr - lr - eb;
    if (w < 1 || w > 4 || eb > 5 || eb < 1 || (eb == 1 && w != 1))
        return FWT_EINVAL;
    // Two exchange phases need one exchange (w < eb) whose top register bit
    // stays put.
    // Two phases by default for fp64-sized row tiles of two-pass plans and
    // for column tiles of 2^11+ slots (compiled from there on), and where
    // the tile would exceed 128 KiB of LDS.
    const bool col_phased = !row && kr + gbits >= 11;
    const int phb = t.phases >= 0 ? t.phases
                                  : ((two_tiles || col_phased || kr + gbits > 13) && w < eb ? 1 : 0);
    if (phb && w >= eb)
        return FWT_EINVAL;
    p.key = KernelKey{dtype == FWT_F64 ? 1 : 0, kr, eb, gbits, phb, row ? 1 : 0, 0, 2};
    if (!qse::kernel_available(p.key))
        return FWT_EUNSUPPORTED;
    p.gbits = gbits;
    p.phb = phb;
    p.tt_bits = 6 + w;
    p.tpw_bits = 0;
    p.block = 64u << w;
    p.lds = (size_t)16 << (kr + gbits - phb);
    p.store_back = 0;
    p.tiles_bits = row ? n - k : (n - lo - k) + p.nblk_bits;
    return check_offsets(p, dtype, row, kr, vb, w < eb);
}

// Default Kronecker split (bit counts, lowest bits first), from sweeps of
// every two-pass split on MI355X (2 GiB states, n = 15..26):
//  - one pass while a vector fits one tile: n <= 15 (fp32), 14 (fp64);
//  - two passes while the column factor stays within 11 bits: the row pass
//    takes n - 9 bits (a 9-bit column factor: tiles of 512 rows x 128 B),
//    but at least 8 vector bits (its lane-exchange tile of 8 vector bits
//    was the fastest row pass for n = 15..19), never exactly 9 vector bits
//    (10 measured faster there: n = 20 fp32 as 12|8, n = 19 fp64 as 11|8),
//    and at most what one tile holds (15 fp32, 14 fp64 bits), the column
//    factor taking the rest (10-11 bits at n = 25-26 fp32, 24-25 fp64);
//  - three passes above: 10 row bits, the rest split evenly.
int default_split(int n, fwt_dtype dtype, fwt_path path, int* bits)
{
    const int vb = vec_bits(dtype);
    const int single_max = kRowKrMax + vb;   // 15 fp32, 14 fp64
    if (path == FWT_PATH_SINGLE_BLOCK) {
        if (n > single_max)
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
    if (n - single_max <= kColTwoPassMax) {
        int row = n - kColPref;
        if (row - vb < 8)
            row = 8 + vb;
        if (row - vb == 9)
            row = 10 + vb;
        if (row > single_max)
            row = single_max;
        bits[0] = row;
        bits[1] = n - row;
        return 2;
    }
    const int rest = n - 10;
    bits[0] = 10;
    bits[1] = rest - rest / 2;
    bits[2] = rest / 2;
    return 3;
}

int make_plan(fwt_plan_t* out, int n, fwt_dtype dtype, int npasses, const int* bits,
              const fwt_pass_tuning* tuning, bool mfma_row = false)
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
        if (i == 0 && mfma_row) {
            if (bits[0] < kMfmaRowMin || bits[0] > mfma_row_max(dtype)) {
                delete p;
                return FWT_EUNSUPPORTED;
            }
            p->passes[0] = Pass{};
            p->passes[0].k = bits[0];
            p->passes[0].mfma = 1;
            lo += bits[0];
            continue;
        }
        const fwt_pass_tuning dflt{-1, -1, -1, -1, -1};
        const int rc = build_pass(p->passes[i], n, dtype, lo, bits[i], tuning ? tuning[i] : dflt,
                                  p->npasses > 1);
        if (rc != FWT_OK) {
            delete p;
            return rc;
        }
        lo += bits[i];
    }
    // A one-pass plan of 12 vector bits on the lane-exchange kernel keeps a
    // second tiling for states that fit the Infinity Cache: 512 threads of
    // 8 vectors and one LDS exchange (eb = 3) instead of 1024 threads of 4
    // and two (eb = 2).  Measured on MI355X (fp32 n = 14, fp64 n = 13): 3-10 %
    // faster per call on states of 4-192 MiB (n = 14, batch 64: 6.05 against
    // 6.28 us), equal at 256 MiB, and 4-5 % slower at 384-512 MiB, where the
    // extra threads keep more HBM reads in flight.
    p->has_small = 0;
    p->onepass = 0;
    const bool pass0_default =
        !tuning || (tuning[0].eb < 0 && tuning[0].gbits < 0 && tuning[0].phases < 0 &&
                    tuning[0].pipe < 0 && tuning[0].wave < 0);
    if (p->npasses == 1 && !mfma_row && pass0_default && p->passes[0].key.wave == 2 &&
        p->passes[0].key.row && p->passes[0].key.kr == 12 && p->passes[0].key.eb == 2) {
        const fwt_pass_tuning t3{3, -1, -1, -1, 2};
        p->small = Pass{};
        p->small.lo = 0;
        p->small.k = n;
        if (build_lx_pass(p->small, n, dtype, 0, n, 12, true, t3, false) == FWT_OK)
            p->has_small = 1;
    }
    if (log_enabled()) {
        std::fprintf(stderr, "[fwt] plan n=%d dtype=%s passes=%d\n", n,
                     dtype == FWT_F64 ? "f64" : "f32", p->npasses);
        for (int i = 0; i < p->npasses; ++i) {
            const Pass& q = p->passes[i];
            std::fprintf(stderr,
                         "[fwt]   pass %d: bits [%d,%d) %s kr=%d eb=%d G=%d phases=%d pipe=%d "
                         "wave=%d threads/tile=%d block=%u lds=%zu store_back=%d tiles/vec=2^%d\n",
                         i, q.lo, q.lo + q.k,
                         q.mfma ? "mfma" : (q.pair ? "pair" : (q.key.row ? "row" : "col")),
                         q.key.kr, q.key.eb, 1 << q.gbits, 1 << q.phb, q.key.pipe, q.key.wave,
                         1 << q.tt_bits, q.block, q.lds, q.store_back, q.tiles_bits);
        }
    }
    *out = p;
    return FWT_OK;
}

bool valid_plan(fwt_plan_t p) { return p && p->magic == kPlanMagic; }

constexpr int kMaxDevices = 64;
std::mutex g_init_mutex;
std::atomic<uint64_t> g_init_devices{0};
int g_cu_count[kMaxDevices];
int g_onepass_ok[kMaxDevices];

// Once per device: kernel attributes and the compute-unit count.  Returns
// the CU count of the current device in *cus.
int ensure_device_init(int* cus)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e);
    if (dev < 0 || dev >= kMaxDevices)
        return FWT_EUNSUPPORTED;
    if (!((g_init_devices.load(std::memory_order_acquire) >> dev) & 1)) {
        std::lock_guard<std::mutex> lock(g_init_mutex);
        if (!((g_init_devices.load() >> dev) & 1)) {
            e = qse::kernels_init_device();
            if (e != hipSuccess)
                return hip_fail(e);
            int n = 0;
            e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
            if (e != hipSuccess)
                return hip_fail(e);
            g_cu_count[dev] = n > 0 ? n : 1;
            // The one-pass kernel needs all kOpGroups * kOpMembers workgroups
            // resident at once: 8 XCDs of 32 CUs, two workgroups per CU.
            int per_cu = 0;
            e = qse::onepass_occupancy(&per_cu);
            if (e != hipSuccess)
                return hip_fail(e);
            g_onepass_ok[dev] = (n == qse::kOpXcds * qse::kOpMembers &&
                                 per_cu >= qse::kOpGroupsPerXcd) ? 1 : 0;
            g_init_devices.fetch_or((uint64_t)1 << dev, std::memory_order_release);
        }
    }
    *cus = g_cu_count[dev];
    return FWT_OK;
}

// Whether the one-pass kernel can run on the current device (after
// ensure_device_init).
bool onepass_device_ok()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return false;
    return g_onepass_ok[dev] != 0;
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

// The chunk schedule of a call.  A multi-pass call whose state exceeds the
// Infinity Cache runs its leading passes on one chunk of about kChunkBytes
// before the next chunk starts, so that the later passes re-read what the
// earlier ones left in the cache.  A chunk is `blocks` consecutive blocks
// of 2^block_bits elements of each component.  Normally a block is a whole
// vector (block_bits = n) and every pass runs per chunk.  When one vector
// alone exceeds the cache, the leading passes whose bits all lie below
// block_bits < n touch each block of 2^block_bits elements on its own, so
// they run per chunk of such blocks, and the remaining passes then run
// over the whole state (fp32 n = 27, [10, 9, 8]: passes 0 and 1 per chunk
// of 64 blocks of 2^19 elements, then pass 2; 14 % faster than whole
// vectors per chunk).  chunked = 0: no chunking.
struct Schedule {
    int chunked;        // leading passes run chunk by chunk
    int block_bits;     // log2 elements per block
    int64_t blocks;     // blocks per chunk
};

Schedule call_schedule(const fwt_plan_s* plan, int64_t batch, int ncomp)
{
    Schedule s{0, plan->n, 0};
    const int np = plan->npasses;
    if (np < 2)
        return s;
    const size_t esize = plan->dtype == FWT_F64 ? 8 : 4;
    const size_t vec_bytes = ((size_t)1 << plan->n) * esize * (size_t)ncomp;
    if ((size_t)batch * vec_bytes <= kChunkBytes)
        return s;
    if (vec_bytes <= kChunkBytes) {
        s.chunked = np;
        s.blocks = (int64_t)(kChunkBytes / vec_bytes);
        return s;
    }
    // The longest run of leading passes (not the last, none on the matrix
    // cores) whose bits fit one cached block.
    int lead = 0, lead_bits = 0, bits = 0;
    for (int j = 0; j < np - 1 && !plan->passes[j].mfma; ++j) {
        bits += plan->passes[j].k;
        if (((size_t)1 << bits) * esize * (size_t)ncomp > kChunkBytes)
            break;
        lead = j + 1;
        lead_bits = bits;
    }
    if (lead >= 2) {
        s.chunked = lead;
        s.block_bits = lead_bits;
        s.blocks = (int64_t)(kChunkBytes / (((size_t)1 << lead_bits) * esize * (size_t)ncomp));
        return s;
    }
    s.chunked = np;   // one vector per chunk
    s.blocks = 1;
    return s;
}

// Vectors per chunk when the chunks hold whole vectors, else 0.
int64_t chunk_vectors(const fwt_plan_s* plan, int64_t batch, int ncomp)
{
    const Schedule s = call_schedule(plan, batch, ncomp);
    return s.chunked && s.block_bits == plan->n ? s.blocks : 0;
}

// Whether a call on `batch` vectors of ncomp components launches the plan's
// cache-resident tiling: a one-pass plan that has one, on a state of at
// most the Infinity Cache's 256 MiB.
bool use_small(const fwt_plan_s* plan, int64_t batch, int ncomp)
{
    if (!plan->has_small)
        return false;
    const size_t esize = plan->dtype == FWT_F64 ? 8 : 4;
    const size_t vec_bytes = ((size_t)1 << plan->n) * esize * (size_t)ncomp;
    return (size_t)batch <= kChunkBytes / vec_bytes;
}

// Bytes of the state of a call on `batch` vectors of ncomp components.
size_t state_bytes(const fwt_plan_s* plan, int64_t batch, int ncomp)
{
    return (size_t)batch * ((size_t)1 << plan->n) * (plan->dtype == FWT_F64 ? 8 : 4) *
           (size_t)ncomp;
}

// Cache policy of the stores of pass p, in a call on a state of `bytes`
// whose schedule is chunked or not.  Multi-pass plans only (one-pass plans
// store plainly).  From A/B timings of the four combinations on 26
// workloads from 8 MiB to 4 GiB:
//  - the last pass stores nontemporally in chunked schedules (states past
//    the Infinity Cache), so that a chunk's results leave room for the
//    next chunk: -0.1 to -3.8 % per call; on smaller states the plain
//    stores leave the results cached for the next call, and nontemporal
//    ones cost 2-5 %;
//  - an earlier pass stores with device scope once the state exceeds the
//    L2s, when its tiles are at most 2^10 16-byte slots (the small row
//    tiles, several per CU): 64-256 MiB states -0.8 to -8.7 %, 2 GiB
//    states with such row tiles a further -1.1 to -1.6 %.  Within the L2s
//    it costs 4-12 %, and with larger tiles (one or two per CU) it is
//    0.5-2.5 % slower than plain stores.
int store_policy(const Pass& p, bool multi, bool final_pass, size_t bytes, bool chunked)
{
    if (!multi)
        return qse::kStorePlain;
    if (final_pass)
        return chunked ? qse::kStoreNontemporal : qse::kStorePlain;
    return bytes > kL2Bytes && p.key.kr + p.gbits <= 10 ? qse::kStoreWriteThrough
                                                        : qse::kStorePlain;
}

// Enqueue passes [first, last) over `batch` vectors starting at re/im, or,
// with sub_bits > 0, over `batch` blocks of 2^(n - sub_bits) elements (for
// passes whose bits all lie below n - sub_bits).  In a multi-pass plan the
// first pass reads and the last pass writes with nontemporal hints: their
// data is not reused by this call, while the intermediate data between
// passes should stay in the caches.  The stores follow store_policy for
// the call's whole state of call_bytes, in a chunked schedule or not.
int launch_passes(fwt_plan_t plan, int first, int last, int64_t batch, int n, void* re, void* im,
                  int normalize, size_t call_bytes, bool chunked, hipStream_t stream,
                  hipEvent_t start = nullptr, hipEvent_t stop = nullptr, int sub_bits = 0)
{
    int cus = 1;
    int rc = ensure_device_init(&cus);
    if (rc != FWT_OK)
        return rc;
    if (stream) {
        // Kernel attributes and the grid sizes are set up for the current
        // device: the stream must belong to it.
        int cur = 0;
        hipDevice_t sdev = 0;
        hipError_t e = hipGetDevice(&cur);
        if (e == hipSuccess)
            e = hipStreamGetDevice(stream, &sdev);
        if (e != hipSuccess)
            return hip_fail(e);
        if ((int)sdev != cur)
            return FWT_EINVAL;
    }
    const int ncomp = im ? 2 : 1;
    const double c = norm_constant(n);
    const bool multi = plan->npasses >= 2;
    const bool small = sub_bits == 0 && use_small(plan, batch, ncomp);
    for (int i = first; i < last; ++i) {
        const Pass& p = small ? plan->small : plan->passes[i];
        const bool final_pass = (i == plan->npasses - 1);
        const int do_scale = (normalize && final_pass) ? 1 : 0;
        if (sub_bits && (p.mfma || p.pair || p.lo + p.k > n - sub_bits))
            return FWT_EINVAL;   // a block schedule covers low-bit tile passes only
        hipError_t e;
        if (p.mfma) {
            e = hipSuccess;
            if (i == first && start)
                e = hipEventRecord(start, stream);
            if (e == hipSuccess)
                e = qse::ablation_mfma_row(plan->dtype == FWT_F64 ? 1 : 0, re, im, batch, n, p.k,
                                           do_scale, c, stream);
            if (e == hipSuccess && i == last - 1 && stop)
                e = hipEventRecord(stop, stream);
        } else if (p.pair) {
            e = qse::launch_pair_f32((float*)re, (float*)im, batch, do_scale, (float)c, stream,
                                     i == first ? start : nullptr,
                                     i == last - 1 ? stop : nullptr);
        } else {
            TileArgs a{};
            a.tiles = batch << (p.tiles_bits - sub_bits);
            a.wg_count = (a.tiles + ((int64_t)1 << p.tpw_bits) - 1) >> p.tpw_bits;
            a.lo = p.lo;
            a.nblk_bits = p.nblk_bits;
            a.tpw_bits = p.tpw_bits;
            a.tt_bits = p.tt_bits;
            a.do_scale = do_scale;
            a.ld_nt = (multi && i == 0) ? 1 : 0;
            a.st_policy = store_policy(p, multi, final_pass, call_bytes, chunked);
            a.scale = plan->dtype == FWT_F64 ? c : (double)(float)c;
            // Persistent kernels: as many workgroups as the CUs hold at once.
            const int64_t per_cu = p.lds ? (int64_t)(kLdsMax / p.lds) : 1;
            const int64_t total = (int64_t)cus * (per_cu > 0 ? per_cu : 1);
            a.grid = total / ncomp > 0 ? total / ncomp : 1;
            // States below the Infinity Cache's size: each vector
            // component's workgroups on one XCD, the same in every pass and
            // call (xcd_group), so that a pass finds the previous launch's
            // output of a component in that XCD's L2.  Measured per call:
            // 32 MiB states 27 % faster, 64-256 MiB states 0.5-3.7 %, the
            // configured n = 14 7|7 split 22 %.  The 256 MiB chunks of larger
            // states stay in launch order (placed, n = 20 and 21 at 2 GiB were
            // 3-6 % slower).
            const int kb = p.tiles_bits - p.tpw_bits;   // log2 workgroups per component
            a.xcd_bits = -1;
            if (!p.key.pipe && sub_bits == 0 && kb >= 1 && kb < 30 &&
                (size_t)batch * ((size_t)1 << n) * (plan->dtype == FWT_F64 ? 8 : 4) *
                        (size_t)ncomp < kChunkBytes &&
                a.wg_count >= ((int64_t)8 << kb) && a.wg_count <= ((int64_t)1 << 30))
                a.xcd_bits = kb;
            e = qse::launch_tile_pass(p.key, re, im, ncomp, a, p.block, p.lds, stream,
                                      i == first ? start : nullptr,
                                      i == last - 1 ? stop : nullptr);
        }
        if (e != hipSuccess)
            return hip_fail(e);
    }
    return FWT_OK;
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
    if (path == FWT_PATH_MFMA_ABLATION) {
        // the default split, with the row pass on the matrix-core kernel
        // (measured and tested up to n = 29 for fp64)
        if (n < kMfmaRowMin || (dtype == FWT_F64 && n > 29))
            return FWT_EUNSUPPORTED;
        int bits[kMaxPasses] = {0, 0, 0, 0};
        const int np = default_split(n, dtype, FWT_PATH_AUTO, bits);
        if (np < 0)
            return FWT_EUNSUPPORTED;
        return make_plan(out, n, dtype, np, bits, nullptr, true);
    }
    if (path != FWT_PATH_AUTO && path != FWT_PATH_SINGLE_BLOCK && path != FWT_PATH_MULTIPASS)
        return FWT_EINVAL;
    int bits[kMaxPasses] = {0, 0, 0, 0};
    const int np = default_split(n, dtype, path, bits);
    if (np < 0)
        return FWT_EUNSUPPORTED;
    const int rc = make_plan(out, n, dtype, np, bits, nullptr);
    if (rc == FWT_OK && path == FWT_PATH_AUTO && n == qse::kOpN && dtype == FWT_F32)
        (*out)->onepass = 1;
    return rc;
}

int fwt_plan_create_split(fwt_plan_t* out, int n, fwt_dtype dtype, int npasses, const int* bits)
{
    return make_plan(out, n, dtype, npasses, bits, nullptr);
}

int fwt_plan_create_tuned(fwt_plan_t* out, int n, fwt_dtype dtype, int npasses, const int* bits,
                          const fwt_pass_tuning* tuning)
{
    return make_plan(out, n, dtype, npasses, bits, tuning);
}

int fwt_execute_check(fwt_plan_t plan, int64_t batch, int n, const void* re, const void* im)
{
    bool nothing = false;
    return validate(plan, batch, n, re, im, &nothing);
}

int fwt_execute(fwt_plan_t plan, int64_t batch, int n, void* re, void* im, int normalize,
                hipStream_t stream)
{
    bool nothing = false;
    const int rc = validate(plan, batch, n, re, im, &nothing);
    if (rc != FWT_OK || nothing)
        return rc;
    const Schedule s = call_schedule(plan, batch, im ? 2 : 1);
    const size_t bytes = state_bytes(plan, batch, im ? 2 : 1);
    if (s.chunked == 0)
        return launch_passes(plan, 0, plan->npasses, batch, n, re, im, normalize, bytes, false,
                             stream);
    const int sub = n - s.block_bits;
    const int64_t blocks = batch << sub;
    const size_t block_bytes = ((size_t)1 << s.block_bits) * (plan->dtype == FWT_F64 ? 8 : 4);
    for (int64_t b0 = 0; b0 < blocks; b0 += s.blocks) {
        const int64_t nb = blocks - b0 < s.blocks ? blocks - b0 : s.blocks;
        void* cre = (char*)re + (size_t)b0 * block_bytes;
        void* cim = im ? (char*)im + (size_t)b0 * block_bytes : nullptr;
        const int r = launch_passes(plan, 0, s.chunked, nb, n, cre, cim, normalize, bytes, true,
                                    stream, nullptr, nullptr, sub);
        if (r != FWT_OK)
            return r;
    }
    if (s.chunked < plan->npasses)
        return launch_passes(plan, s.chunked, plan->npasses, batch, n, re, im, normalize, bytes,
                             true, stream);
    return FWT_OK;
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
    const size_t bytes = state_bytes(plan, batch, im ? 2 : 1);
    return launch_passes(plan, pass, pass + 1, batch, n, re, im, normalize, bytes,
                         bytes >= kChunkBytes, stream);
}

int fwt_execute_pass_timed(fwt_plan_t plan, int pass, int64_t batch, int n, void* re, void* im,
                           int normalize, hipStream_t stream, hipEvent_t start, hipEvent_t stop)
{
    if (!valid_plan(plan) || pass < 0 || pass >= plan->npasses || !start || !stop)
        return FWT_EINVAL;
    bool nothing = false;
    const int rc = validate(plan, batch, n, re, im, &nothing);
    if (rc != FWT_OK || nothing)
        return rc == FWT_OK ? FWT_EINVAL : rc;   // nothing to time
    const size_t bytes = state_bytes(plan, batch, im ? 2 : 1);
    return launch_passes(plan, pass, pass + 1, batch, n, re, im, normalize, bytes,
                         bytes >= kChunkBytes, stream, start, stop);
}

// ---- one HBM pass on a workspace (fp32 n = 20) -------------------------------

namespace {

// Workspace bytes a call of `plan` on `batch` vectors needs for the one-pass
// kernel, or 0 when the call runs fwt_execute's passes.  *rc receives an
// FWT_* status (FWT_EHIP when the device cannot be queried).
size_t onepass_bytes(fwt_plan_t plan, int64_t batch, int with_im, int* rc)
{
    *rc = FWT_OK;
    if (!plan->onepass || batch <= 0)
        return 0;
    const int64_t ncomp = batch * (with_im ? 2 : 1);
    if (ncomp >= ((int64_t)1 << 30))
        return 0;
    int cus = 0;
    *rc = ensure_device_init(&cus);
    if (*rc != FWT_OK || !onepass_device_ok())
        return 0;
    return qse::kOpWorkspaceBytes;
}

int execute_ws(fwt_plan_t plan, int64_t batch, int n, void* re, void* im, int normalize,
               void* ws, size_t ws_bytes, hipStream_t stream, hipEvent_t start,
               hipEvent_t stop)
{
    bool nothing = false;
    int rc = validate(plan, batch, n, re, im, &nothing);
    if (rc != FWT_OK || nothing)
        return rc;
    const size_t need = onepass_bytes(plan, batch, im != nullptr, &rc);
    if (rc != FWT_OK)
        return rc;
    if (need == 0)
        return fwt_execute(plan, batch, n, re, im, normalize, stream);
    if (!ws || ws_bytes < need)
        return FWT_EINVAL;
    if ((uintptr_t)ws & 255u)
        return FWT_EALIGN;
    const size_t bytes = (size_t)batch << (n + 2);
    const uintptr_t w = (uintptr_t)ws;
    for (const void* b : {(const void*)re, (const void*)im}) {
        const uintptr_t a = (uintptr_t)b;
        if (b && ((a <= w && w - a < bytes) || (w < a && a - w < need)))
            return FWT_EINVAL;
    }
    rc = check_range(ws, need);
    if (rc != FWT_OK)
        return rc;
    const int ncomp = (int)(batch * (im ? 2 : 1));
    const float scale = normalize ? (float)norm_constant(n) : 1.0f;
    const hipError_t e = qse::launch_onepass((float*)re, (float*)im, ncomp, ws, scale, stream,
                                             start, stop);
    return e == hipSuccess ? FWT_OK : hip_fail(e);
}

}  // namespace

int fwt_workspace_size(fwt_plan_t plan, int64_t batch, int with_im, size_t* bytes)
{
    if (!valid_plan(plan) || !bytes || batch < 0)
        return FWT_EINVAL;
    *bytes = 0;
    int rc = FWT_OK;
    *bytes = onepass_bytes(plan, batch, with_im, &rc);
    return rc;
}

int fwt_execute_ws(fwt_plan_t plan, int64_t batch, int n, void* re, void* im, int normalize,
                   void* ws, size_t ws_bytes, hipStream_t stream)
{
    return execute_ws(plan, batch, n, re, im, normalize, ws, ws_bytes, stream, nullptr,
                      nullptr);
}

int fwt_execute_ws_timed(fwt_plan_t plan, int64_t batch, int n, void* re, void* im,
                         int normalize, void* ws, size_t ws_bytes, hipStream_t stream,
                         hipEvent_t start, hipEvent_t stop)
{
    if (!start || !stop || !valid_plan(plan))
        return FWT_EINVAL;
    int rc = FWT_OK;
    const size_t need = onepass_bytes(plan, batch, im != nullptr, &rc);
    if (rc != FWT_OK)
        return rc;
    if (need == 0)
        return FWT_EINVAL;   // only the one-pass kernel is timed here
    return execute_ws(plan, batch, n, re, im, normalize, ws, ws_bytes, stream, start, stop);
}

int fwt_workspace_status(const void* ws, int* bits)
{
    if (!ws || !bits)
        return FWT_EINVAL;
    *bits = 0;
    const hipError_t e = hipMemcpy(bits, (const unsigned char*)ws + qse::kOpErrOff, sizeof(int),
                                   hipMemcpyDeviceToHost);
    return e == hipSuccess ? FWT_OK : hip_fail(e);
}

int fwt_plan_chunk_vectors(fwt_plan_t plan, int64_t batch, int with_im, int64_t* out)
{
    if (!valid_plan(plan) || !out || batch < 0)
        return FWT_EINVAL;
    *out = chunk_vectors(plan, batch, with_im ? 2 : 1);
    return FWT_OK;
}

int fwt_plan_call_schedule(fwt_plan_t plan, int64_t batch, int with_im, int* chunked_passes,
                           int* block_bits, int64_t* blocks_per_chunk)
{
    if (!valid_plan(plan) || !chunked_passes || !block_bits || !blocks_per_chunk || batch < 0)
        return FWT_EINVAL;
    const Schedule s = call_schedule(plan, batch, with_im ? 2 : 1);
    *chunked_passes = s.chunked;
    *block_bits = s.block_bits;
    *blocks_per_chunk = s.blocks;
    return FWT_OK;
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

// ---- ablations ---------------------------------------------------------------

namespace {

size_t ablation_workspace_bytes(int kind, int64_t batch, int n, fwt_dtype dtype, int with_im)
{
    if (kind == FWT_ABLATION_OZAKI) {
        if (n < qse::kOzMinN || n > qse::kOzMaxN)
            return 0;
        size_t a, b;
        return qse::oz_workspace_layout(batch, n, with_im ? 2 : 1, &a, &b);
    }
    if (kind != FWT_ABLATION_POPC_GEMM && kind != FWT_ABLATION_MFMA_TRANSPOSE)
        return 0;
    const size_t esize = dtype == FWT_F64 ? 8 : 4;
    return (size_t)batch * ((size_t)1 << n) * esize * (with_im ? 2 : 1);
}

// Argument checks of an ablation call.  `ws_owned`: the workspace is the
// library's own static scratch (256-byte aligned, never inside a caller's
// buffer), so it is not checked at all; its size is checked by the caller.
int ablation_check(int kind, int64_t batch, int n, fwt_dtype dtype, const void* re,
                   const void* im, const void* ws, size_t ws_bytes, bool ws_owned)
{
    if (dtype != FWT_F32 && dtype != FWT_F64)
        return FWT_EINVAL;
    const int vb = vec_bits(dtype);
    if (kind == FWT_ABLATION_STAGEWISE) {
        if (n < vb || n > FWT_MAX_N)
            return n < 0 || n > FWT_MAX_N ? FWT_EINVAL : FWT_EUNSUPPORTED;
    } else if (kind == FWT_ABLATION_POPC_GEMM) {
        if (n < 2 || n > 26)
            return n < 0 || n > FWT_MAX_N ? FWT_EINVAL : FWT_EUNSUPPORTED;
    } else if (kind == FWT_ABLATION_MFMA) {
        if (n < kMfmaRowMin || n > (dtype == FWT_F64 ? 29 : FWT_MAX_N))
            return n < 0 || n > FWT_MAX_N ? FWT_EINVAL : FWT_EUNSUPPORTED;
    } else if (kind == FWT_ABLATION_OZAKI) {
        if (n < 0 || n > FWT_MAX_N)
            return FWT_EINVAL;
        if (dtype != FWT_F64 || n < qse::kOzMinN || n > qse::kOzMaxN)
            return FWT_EUNSUPPORTED;
    } else if (kind == FWT_ABLATION_MFMA_TRANSPOSE) {
        // both factors n / 2 and n - n / 2 within the matrix-core row kernel
        if (n < 2 * kMfmaRowMin || n > 2 * mfma_row_max(dtype))
            return n < 0 || n > FWT_MAX_N ? FWT_EINVAL : FWT_EUNSUPPORTED;
    } else {
        return FWT_EINVAL;
    }
    if (!re || batch < 0)
        return FWT_EINVAL;
    if (((uintptr_t)re & 15u) || ((uintptr_t)im & 15u) || (!ws_owned && ((uintptr_t)ws & 15u)))
        return FWT_EALIGN;
    if (re == im)
        return FWT_EINVAL;
    const size_t esize = dtype == FWT_F64 ? 8 : 4;
    if (batch > INT64_MAX / ((int64_t)1 << n) / (int64_t)esize)
        return FWT_EINVAL;
    const size_t bytes = (size_t)batch * ((size_t)1 << n) * esize;
    auto overlap = [](const void* a, size_t na, const void* b, size_t nb) {
        const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
        return x < y + nb && y < x + na;
    };
    if (im && overlap(re, bytes, im, bytes))
        return FWT_EINVAL;
    const size_t need = ablation_workspace_bytes(kind, batch, n, dtype, im != nullptr);
    if (need && !ws_owned) {
        if (!ws || ws_bytes < need)
            return FWT_EINVAL;
        if (overlap(ws, need, re, bytes) || (im && overlap(ws, need, im, bytes)))
            return FWT_EINVAL;
    }
    if (batch == 0)
        return FWT_OK;
    int rc = check_range(re, bytes);
    if (rc == FWT_OK && im)
        rc = check_range(im, bytes);
    if (rc == FWT_OK && need && !ws_owned)
        rc = check_range(ws, need);
    return rc;
}

// Matrix-core ablation: an FWT_PATH_MFMA_ABLATION plan, made once per
// (dtype, n) and kept for the life of the process.
fwt_plan_t g_mfma_plans[2][FWT_MAX_N + 1];
std::mutex g_mfma_mutex;

int ablation_mfma(int64_t batch, int n, fwt_dtype dtype, void* re, void* im, int normalize,
                  hipStream_t stream)
{
    fwt_plan_t plan = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_mfma_mutex);
        fwt_plan_t& slot = g_mfma_plans[dtype == FWT_F64 ? 1 : 0][n];
        if (!slot) {
            const int rc = fwt_plan_create(&slot, n, dtype, FWT_PATH_MFMA_ABLATION);
            if (rc != FWT_OK)
                return rc;
        }
        plan = slot;
    }
    return fwt_execute(plan, batch, n, re, im, normalize, stream);
}

}  // namespace

int fwt_ablation_workspace(int kind, int64_t batch, int n, fwt_dtype dtype, int with_im,
                           size_t* out)
{
    if (!out || batch < 0 || n < 0 || n > FWT_MAX_N)
        return FWT_EINVAL;
    if (kind < FWT_ABLATION_STAGEWISE || kind > FWT_ABLATION_MFMA_TRANSPOSE)
        return FWT_EINVAL;
    *out = ablation_workspace_bytes(kind, batch, n, dtype, with_im);
    return FWT_OK;
}

int fwt_ablation_execute(int kind, int64_t batch, int n, fwt_dtype dtype, void* re, void* im,
                         int normalize, void* workspace, size_t workspace_bytes,
                         hipStream_t stream)
{
    return qse::ablation_run(kind, batch, n, (int)dtype, re, im, normalize, workspace,
                             workspace_bytes, false, stream);
}

}  // extern "C"

int qse::ablation_validate(int kind, int64_t batch, int n, int dtype, const void* re,
                           const void* im)
{
    return ablation_check(kind, batch, n, (fwt_dtype)dtype, re, im, nullptr, 0, true);
}

int qse::hip_status(hipError_t e)
{
    return hip_fail(e);
}

size_t qse::ablation_workspace_size(int kind, int64_t batch, int n, int dtype, int with_im)
{
    return ablation_workspace_bytes(kind, batch, n, (fwt_dtype)dtype, with_im);
}

int qse::ablation_run(int kind, int64_t batch, int n, int dtype_, void* re, void* im,
                      int normalize, void* workspace, size_t workspace_bytes, bool ws_owned,
                      hipStream_t stream)
{
    const fwt_dtype dtype = (fwt_dtype)dtype_;
    int rc = ablation_check(kind, batch, n, dtype, re, im, workspace, workspace_bytes, ws_owned);
    if (rc != FWT_OK || batch == 0)
        return rc;
    int cus = 1;
    rc = ensure_device_init(&cus);
    if (rc != FWT_OK)
        return rc;
    const double c = dtype == FWT_F64 ? norm_constant(n) : (double)(float)norm_constant(n);
    const int f64 = dtype == FWT_F64 ? 1 : 0;
    hipError_t e;
    if (kind == FWT_ABLATION_MFMA)
        return ablation_mfma(batch, n, dtype, re, im, normalize, stream);
    if (kind == FWT_ABLATION_OZAKI) {
        e = qse::ablation_ozaki((double*)re, (double*)im, batch, n, normalize ? c : 1.0,
                                workspace, stream);
        return e == hipSuccess ? FWT_OK : hip_fail(e);
    }
    if (kind == FWT_ABLATION_STAGEWISE) {
        e = qse::ablation_stagewise(f64, re, im, batch, n, normalize, c, stream);
    } else {
        const size_t esize = f64 ? 8 : 4;
        void* ws_im = im ? (char*)workspace + (size_t)batch * ((size_t)1 << n) * esize : nullptr;
        if (kind == FWT_ABLATION_MFMA_TRANSPOSE)
            e = qse::ablation_mfma_transpose(f64, re, im, workspace, ws_im, batch, n, normalize,
                                             c, stream);
        else
            e = qse::ablation_popc_gemm(f64, re, im, workspace, ws_im, batch, n, normalize, c,
                                        stream);
    }
    return e == hipSuccess ? FWT_OK : hip_fail(e);
}

extern "C" {

namespace {

void pass_config(const Pass& p, int* out)
{
    out[0] = p.lo;
    out[1] = p.k;
    out[2] = p.mfma ? 3 : (p.pair ? 2 : (p.key.row ? 0 : 1));
    out[3] = p.key.kr;
    out[4] = p.key.eb;
    out[5] = p.gbits;
    out[6] = p.phb;
    out[7] = (int)p.block;
    out[8] = (int)p.lds;
    out[9] = p.tpw_bits;
    out[10] = p.key.pipe;
    out[11] = p.key.wave;
}

}  // namespace

int fwt_plan_pass_config(fwt_plan_t plan, int i, int* out)
{
    if (!valid_plan(plan) || !out || i < 0 || i >= plan->npasses)
        return FWT_EINVAL;
    pass_config(plan->passes[i], out);
    return FWT_OK;
}

int fwt_plan_call_pass_config(fwt_plan_t plan, int i, int64_t batch, int with_im, int* out)
{
    if (!valid_plan(plan) || !out || i < 0 || i >= plan->npasses || batch < 0)
        return FWT_EINVAL;
    pass_config(use_small(plan, batch, with_im ? 2 : 1) ? plan->small : plan->passes[i], out);
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
    case FWT_ESCRATCH: return "workspace larger than the static scratch array";
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
