// gfx950 kernels for the batched in-place Walsh-Hadamard transform.
//
// Every pass is one launch of one of three kernel families, all built on
// the tiles described here: tile_kernel (and its persistent pipelined form
// tile_kernel_pipe) exchanges through padded LDS tiles; wave_kernel holds a
// whole tile in one wave and crosses lanes without LDS; lx_kernel keeps the
// lowest row bits in lanes and moves only the wave bits through unpadded
// LDS.  The planner picks one per pass.  A pass owns the index bits
// [lo, lo + k) of each real vector (the Kronecker factor H_{2^k} acting on
// those bits, Apache Mahout pull request "[QDP] [feature] Pr4 kronecker
// fwt", sections "Why" and "How"; iThome "Day 18" native-FWT article,
// section "Kronecker block GEMM idea").  Its work is cut into tiles: all
// 2^k "rows" (the values of the pass's bits) times G 16-byte column
// groups.  A tile is read from HBM once, transformed on chip, and written
// back to the same place, so a pass costs exactly one read and one write of
// the state, and tiles are disjoint, so in-place passes are race-free.
//
// On chip, each thread holds E = 2^EB 16-byte vectors (rows of one column
// group).  The add/subtract stages (one per index bit, iThome article,
// section "Tensor Core wants matrix multiplication") whose bits are
// currently "register bits" run as butterflies on those registers; then
// the tile is exchanged through LDS so that the next EB row bits become
// register bits (the shared-memory swizzle of the article's introduction,
// done here by padding the 16-byte slots, see LdsLayout).  Column groups never
// mix, so an exchange moves whole 16-byte vectors.  Row passes (lo = 0) see
// the 2^k contiguous elements as 2^(k - vb) rows of a single vector and do
// the vb in-vector bits in registers as well.
//
// Global accesses are 16-byte vector loads and stores in which consecutive
// lanes touch consecutive 16-byte chunks (consecutive rows of a row pass,
// or the G column groups of a row of a column pass).
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <type_traits>
#include <vector>

#include "fwt_internal.h"
#include "fwt_device.h"

namespace qse {
namespace {

// Vector types, butterflies and lane stages: fwt_device.h.

// Row held by thread tau in register j when the register bits are the EB
// row bits starting at A: the low A row bits come from tau's low bits, the
// row bits above A + EB from tau's high bits.  Split into the part that
// depends on the thread and the part that depends on the register.
template <int A, int EB>
__device__ __forceinline__ int row_thread_part(int tau)
{
    return (tau & ((1 << A) - 1)) | ((tau >> A) << (A + EB));
}

// First row bit held in registers in round r.
__host__ __device__ constexpr int round_lo(int kr, int eb, int r)
{
    return kr - eb * (r + 1) > 0 ? kr - eb * (r + 1) : 0;
}

// LDS layout of one exchange phase of a tile.  A tile's 2^GB column
// groups never mix, so an exchange may run in 2^PHB phases, each moving the
// 2^GL (GL = GB - PHB) column groups of one phase through an LDS region
// 2^PHB times smaller than the tile; threads of the other groups wait at
// the phase's barriers.  Within a phase, 16-byte slot s = (row << GL) | gl
// (gl = the group within the phase) is stored at s + (s >> P) with
// P = EB + GL, i.e. one pad slot after every 2^P slots.  For every layout
// of the kernel, the 8 (or 16) lanes that the LDS serves together then
// fall on distinct bank groups: lanes holding consecutive slots stay
// consecutive, and lanes whose slots are 2^P apart are shifted by one slot
// each.  Because the thread part and the register part of a slot are
// disjoint bit fields, s + (s >> P) splits into a per-thread base plus a
// per-register constant, so each access is one address register plus an
// immediate offset.
template <int A, int EB, int GL>
struct LdsLayout {
    static constexpr int P = EB + GL;
    int base;  // padded slot of register 0 for this thread
    __device__ __forceinline__ LdsLayout(int tau, int gl)
    {
        const int s = (row_thread_part<A, EB>(tau) << GL) | gl;
        base = s + (s >> P);
    }
    // Padded offset of register j from register 0 (a compile-time constant
    // once j is unrolled).
    __device__ __forceinline__ static constexpr int offset(int j)
    {
        return ((j << A) << GL) + (((j << A) << GL) >> P);
    }
};

template <typename V, int AF, int AT, int EB, int GB, int PHB>
__device__ __forceinline__ void exchange(V* x, V* L, int tau, int g)
{
    constexpr int E = 1 << EB;
    constexpr int GL = GB - PHB;
    const int gl = g & ((1 << GL) - 1);
    const int my_phase = g >> GL;
    const LdsLayout<AF, EB, GL> from(tau, gl);
    const LdsLayout<AT, EB, GL> to(tau, gl);
#pragma unroll
    for (int ph = 0; ph < (1 << PHB); ++ph) {
        if (PHB == 0 || my_phase == ph) {
#pragma unroll
            for (int j = 0; j < E; ++j)
                L[from.base + LdsLayout<AF, EB, GL>::offset(j)] = x[j];
        }
        __syncthreads();
        if (PHB == 0 || my_phase == ph) {
#pragma unroll
            for (int j = 0; j < E; ++j)
                x[j] = L[to.base + LdsLayout<AT, EB, GL>::offset(j)];
        }
        __syncthreads();
    }
}

// Rounds 1 .. NR-1: exchange into round R's layout, then the stages on the
// row bits [round_lo(R), round_lo(R-1)) that no earlier round did.
template <typename V, int KR, int EB, int GB, int PHB, int R, int NR>
struct Rounds {
    __device__ __forceinline__ static void run(V* x, V* L, int tau, int g)
    {
        constexpr int AP = round_lo(KR, EB, R - 1);
        constexpr int AC = round_lo(KR, EB, R);
        exchange<V, AP, AC, EB, GB, PHB>(x, L, tau, g);
        register_stages<AP - AC, (1 << EB)>(x);
        Rounds<V, KR, EB, GB, PHB, R + 1, NR>::run(x, L, tau, g);
    }
};
template <typename V, int KR, int EB, int GB, int PHB, int NR>
struct Rounds<V, KR, EB, GB, PHB, NR, NR> {
    __device__ __forceinline__ static void run(V*, V*, int, int) {}
};

// Global element offset (relative to the workgroup's base) of register j
// in the layout whose register bits start at row bit A.
template <int A, int EB>
struct GlobalLayout {
    uint32_t base;     // bytes, thread part
    uint32_t jstride;  // bytes between consecutive registers
    __device__ __forceinline__ GlobalLayout(uint32_t lane_bytes, int tau, uint32_t row_bytes)
        : base(lane_bytes + (uint32_t)row_thread_part<A, EB>(tau) * row_bytes),
          jstride(row_bytes << A)
    {
    }
};

// 16-byte global accesses; the nontemporal forms mark data that this
// pass will not touch again (a first pass's input, a last pass's output),
// so that the caches keep the intermediate data between passes.
template <typename V>
__device__ __forceinline__ V load16(const unsigned char* p, uint32_t off)
{
    return *reinterpret_cast<const V*>(p + off);
}
template <typename V>
__device__ __forceinline__ V load16_nt(const unsigned char* p, uint32_t off)
{
    return __builtin_nontemporal_load(reinterpret_cast<const V*>(p + off));
}
// A 16-byte store with cache policy POL (StorePolicy).  The write-through
// form is a buffer store with the device-scope bit (sc1) set: the resource
// spans 2^32 bytes from the workgroup-uniform base p (its third word is
// gfx9's 32-bit data format), so it lives in scalar registers and the lane
// offset is the store's 32-bit VGPR offset.
template <int POL, typename V>
__device__ __forceinline__ void store16(unsigned char* p, uint32_t off, const V& v)
{
    if constexpr (POL == kStoreNontemporal) {
        __builtin_nontemporal_store(v, reinterpret_cast<V*>(p + off));
    } else if constexpr (POL == kStoreWriteThrough) {
        typedef unsigned int u4 __attribute__((ext_vector_type(4)));
        constexpr int kFormatWord = 0x00020000;
        constexpr int kScopeDevice = 16;   // the sc1 bit of the cache-policy operand
        const __amdgpu_buffer_rsrc_t r =
            __builtin_amdgcn_make_buffer_rsrc(p, (short)0, -1, kFormatWord);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, v), r, (int)off, 0,
                                               kScopeDevice);
    } else {
        *reinterpret_cast<V*>(p + off) = v;
    }
}

// Runs f(std::integral_constant<int, POL>) for the run-time policy pol, so
// that each policy's stores are unrolled with a compile-time form.
template <typename F>
__device__ __forceinline__ void with_store_policy(int pol, F&& f)
{
    if (__builtin_expect(pol == kStorePlain, 1))
        f(std::integral_constant<int, kStorePlain>{});
    else if (pol == kStoreNontemporal)
        f(std::integral_constant<int, kStoreNontemporal>{});
    else
        f(std::integral_constant<int, kStoreWriteThrough>{});
}

// The arguments a tile uses only after its stages, read together with the
// ones it uses first.  Left to the scheduler, their scalar load can still
// be in flight during the lane stages, and since LDS operations and scalar
// loads share one wait counter, every ds_swizzle wait then drains to zero
// (up to 4 % per pass).  The asm pins the values in scalar registers here.
struct LateArgs {
    int do_scale;
    int st_policy;
    double scale;
};
__device__ __forceinline__ LateArgs late_args(const TileArgs& a)
{
    LateArgs r{a.do_scale, a.st_policy, a.scale};
    asm volatile("" : "+s"(r.do_scale), "+s"(r.st_policy), "+s"(r.scale));
    return r;
}

// Compile-time shape of a tile kernel.
template <typename T, int KR_, int EB_, int GB_, int PHB_, bool ROW_>
struct Shape {
    using Elem = T;
    using V = typename Vec<T>::type;
    static constexpr int KR = KR_, EB = EB_, GB = GB_, PHB = PHB_;
    static constexpr bool ROW = ROW_;
    static constexpr int WB = Vec<T>::WB;
    static constexpr int E = 1 << EB;
    static constexpr int NR = rounds_of(KR, EB);
    static constexpr int A0 = round_lo(KR, EB, 0);
    static constexpr int AL = round_lo(KR, EB, NR - 1);
    // Store from the load layout (one more exchange) when the last round's
    // layout would give consecutive lanes runs shorter than 128 bytes.
    static constexpr bool STORE_BACK = store_back(KR, EB, GB);
    static constexpr int AF = STORE_BACK ? A0 : AL;   // layout of the final store
    static constexpr int PHASE_SLOTS = 1 << (KR + GB - PHB);
    static constexpr int TILE_LDS = PHASE_SLOTS + (PHASE_SLOTS >> (EB + GB - PHB));
    static_assert(EB <= KR || (KR == 0 && EB == 0), "EB must not exceed KR");
    static_assert(!ROW || GB == 0, "row passes have one column group");
    static_assert(PHB <= GB, "at most one phase per column group");
};

// Where the lanes of one tile group (2^tpw_bits tiles) read and write:
// a workgroup-uniform base pointer plus 32-bit lane offsets (a pass's tile
// span is below 4 GiB).
struct TileAddr {
    unsigned char* p;
    uint32_t lane_bytes;
    uint32_t row_bytes;
    bool active;
};

template <typename S, typename T>
__device__ __forceinline__ TileAddr tile_addr(T* buf, const TileArgs& a, int64_t w, int tl, int g)
{
    const int64_t t0 = a.tile0 + (w << a.tpw_bits);
    int64_t base;
    TileAddr r;
    if (S::ROW) {
        base = t0 << (S::KR + S::WB);
        r.lane_bytes = (uint32_t)tl << (S::KR + S::WB + (sizeof(T) == 8 ? 3 : 2));
        r.row_bytes = 16;
    } else {
        const int64_t blk_mask = ((int64_t)1 << a.nblk_bits) - 1;
        base = ((t0 >> a.nblk_bits) << (a.lo + S::KR)) + ((t0 & blk_mask) << (S::GB + S::WB));
        const uint32_t tlo = (uint32_t)tl >> a.nblk_bits;
        const uint32_t tlb = (uint32_t)tl & (uint32_t)blk_mask;
        r.lane_bytes = ((tlo << (a.lo + S::KR)) + (tlb << (S::GB + S::WB))) * (uint32_t)sizeof(T) +
                       ((uint32_t)g << 4);
        r.row_bytes = (uint32_t)sizeof(T) << a.lo;
    }
    r.p = reinterpret_cast<unsigned char*>(buf + base);
    r.active = t0 + tl < a.tiles;
    return r;
}

template <typename S>
__device__ __forceinline__ void load_tile(typename S::V* x, const TileAddr& ta, int tau, int nt)
{
    using V = typename S::V;
    const GlobalLayout<S::A0, S::EB> gl(ta.lane_bytes, tau, ta.row_bytes);
    if (ta.active && nt) {
#pragma unroll
        for (int j = 0; j < S::E; ++j)
            x[j] = load16_nt<V>(ta.p, gl.base + (uint32_t)j * gl.jstride);
    } else if (ta.active) {
#pragma unroll
        for (int j = 0; j < S::E; ++j)
            x[j] = load16<V>(ta.p, gl.base + (uint32_t)j * gl.jstride);
    } else {
#pragma unroll
        for (int j = 0; j < S::E; ++j)
            x[j] = V{};
    }
}

// All stages of the tile: in-vector bits (row passes), the register bits of
// the load layout, then the remaining rounds through LDS; then the scale
// and, where the final layout differs from the last round's, one more
// exchange.  Every exchange ends with a barrier, so LDS is free again when
// this returns.
template <typename S>
__device__ __forceinline__ void process_tile(typename S::V* x, typename S::V* L, int tau, int g,
                                             int do_scale, double scale)
{
    using V = typename S::V;
    if (S::ROW) {
#pragma unroll
        for (int j = 0; j < S::E; ++j)
            in_vector(x[j]);
    }
    register_stages<S::EB, S::E>(x);
    Rounds<V, S::KR, S::EB, S::GB, S::PHB, 1, S::NR>::run(x, L, tau, g);
    if (do_scale) {
        const typename S::Elem c = (typename S::Elem)scale;
#pragma unroll
        for (int j = 0; j < S::E; ++j)
            x[j] *= c;
    }
    if constexpr (S::STORE_BACK)
        exchange<V, S::AL, S::A0, S::EB, S::GB, S::PHB>(x, L, tau, g);
}

template <typename S>
__device__ __forceinline__ void store_tile(const typename S::V* x, const TileAddr& ta, int tau,
                                           int pol)
{
    using V = typename S::V;
    const GlobalLayout<S::AF, S::EB> gl(ta.lane_bytes, tau, ta.row_bytes);
    if (!ta.active)
        return;
    with_store_policy(pol, [&](auto P) {
#pragma unroll
        for (int j = 0; j < S::E; ++j)
            store16<decltype(P)::value, V>(ta.p, gl.base + (uint32_t)j * gl.jstride, x[j]);
    });
}

// One workgroup per tile group: load, transform, store.
template <typename T, int KR, int EB, int GB, int PHB, bool ROW>
__global__ void __launch_bounds__(EB >= 5 ? 512 : 1024)
    tile_kernel(T* __restrict__ re, T* __restrict__ im, TileArgs a)
{
    using S = Shape<T, KR, EB, GB, PHB, ROW>;
    using V = typename S::V;
    extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
    const int tid = threadIdx.x;
    const int tl = tid >> a.tt_bits;                  // tile within the workgroup
    const int tt = tid & ((1 << a.tt_bits) - 1);      // thread within the tile
    const int g = tt & ((1 << GB) - 1);               // column group
    const int tau = tt >> GB;                         // row-thread index
    V* const L = reinterpret_cast<V*>(lds_raw) + tl * S::TILE_LDS;

    const TileAddr ta =
        tile_addr<S>(blockIdx.y ? im : re, a, xcd_group(blockIdx.x, a.xcd_bits, a.wg_count), tl,
                     g);
    const LateArgs la = late_args(a);
    V x[S::E];
    load_tile<S>(x, ta, tau, a.ld_nt);
    process_tile<S>(x, L, tau, g, la.do_scale, la.scale);
    store_tile<S>(x, ta, tau, la.st_policy);
}

// Persistent, software-pipelined form for tiles so large that a CU holds
// only one: each workgroup walks tile groups blockIdx.x, blockIdx.x +
// gridDim.x, ... and issues the next group's loads into a second register
// set before transforming the current one, so the CU keeps HBM busy while
// its tile goes through the LDS exchanges (barriers wait on LDS only).
template <typename T, int KR, int EB, int GB, int PHB, bool ROW>
__global__ void __launch_bounds__(512)
    tile_kernel_pipe(T* __restrict__ re, T* __restrict__ im, TileArgs a)
{
    using S = Shape<T, KR, EB, GB, PHB, ROW>;
    using V = typename S::V;
    extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
    const int tid = threadIdx.x;
    const int tl = tid >> a.tt_bits;
    const int tt = tid & ((1 << a.tt_bits) - 1);
    const int g = tt & ((1 << GB) - 1);
    const int tau = tt >> GB;
    V* const L = reinterpret_cast<V*>(lds_raw) + tl * S::TILE_LDS;
    T* const buf = blockIdx.y ? im : re;

    int64_t w = blockIdx.x;
    if (w >= a.wg_count)
        return;   // uniform across the workgroup
    const LateArgs la = late_args(a);
    V nx[S::E];
    TileAddr na = tile_addr<S>(buf, a, w, tl, g);
    load_tile<S>(nx, na, tau, a.ld_nt);
    while (true) {
        V x[S::E];
#pragma unroll
        for (int j = 0; j < S::E; ++j)
            x[j] = nx[j];
        const TileAddr ca = na;
        const int64_t wn = w + gridDim.x;
        const bool more = wn < a.wg_count;   // uniform across the workgroup
        if (more) {
            na = tile_addr<S>(buf, a, wn, tl, g);
            load_tile<S>(nx, na, tau, a.ld_nt);
        }
        process_tile<S>(x, L, tau, g, la.do_scale, la.scale);
        store_tile<S>(x, ca, tau, la.st_policy);
        if (!more)
            break;
        w = wn;
    }
}

// ---- wave tiles: a whole tile in one wave, lane stages, no LDS ----------
//
// A wave holds 2^(6 - GB - LB) tiles of 2^KR rows x 2^GB column groups: lane
// l holds column group l mod 2^GB and row bits [0, LB) = the next LB lane
// bits; its E = 2^EB registers hold row bits [LB, KR).  Register bits are
// butterflied in registers; lane bits cross lanes (the single-block design
// of the iThome article's introduction, registers plus warp shuffle, on
// wave64): lane bits 0 and 1 with DPP quad permutes, 2 and 3 with
// ds_swizzle (bit 3 with a DPP row rotation instead, and bit 2 with a DPP
// row half-mirror in mirrored row tiles), and 4 and 5 with
// v_permlane16/32_swap, which exchange a lane
// bit with a register bit so the stage becomes a register butterfly (and
// a second swap restores the layout).  Lanes keep their own half of each
// pair with y = partner + s * x, s = +1 for the lower index and -1 for the
// upper: one rounding, exactly the sum or difference.  (fp32 stages on lane
// bits 0, 1 and 3 keep x + s * partner instead, the difference negated,
// and the kernel's final scaling removes the sign: fmac_dpp_regs.)


template <typename T, int KR, int EB, int GB, bool ROW>
__global__ void __launch_bounds__(256)
    wave_kernel(T* __restrict__ re, T* __restrict__ im, TileArgs a)
{
    using S = Shape<T, KR, EB, GB, 0, ROW>;
    using V = typename S::V;
    constexpr int LB = KR - EB;           // row bits held by lanes
    constexpr int E = 1 << EB;
    constexpr int SUB = 6 - GB - LB;      // log2 tiles per wave
    static_assert(LB >= 0 && SUB >= 0, "a wave tile spans at most 64 lanes");
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int g = lane & ((1 << GB) - 1);
    const int rl = (lane >> GB) & ((1 << LB) - 1);
    const int tl = (wave << SUB) | (lane >> (GB + LB));

    const TileAddr ta =
        tile_addr<S>(blockIdx.y ? im : re, a, xcd_group(blockIdx.x, a.xcd_bits, a.wg_count), tl,
                     g);
    const LateArgs la = late_args(a);
    const GlobalLayout<LB, EB> gl(ta.lane_bytes, rl, ta.row_bytes);
    V x[E];
    if (ta.active && a.ld_nt) {
#pragma unroll
        for (int j = 0; j < E; ++j)
            x[j] = load16_nt<V>(ta.p, gl.base + (uint32_t)j * gl.jstride);
    } else if (ta.active) {
#pragma unroll
        for (int j = 0; j < E; ++j)
            x[j] = load16<V>(ta.p, gl.base + (uint32_t)j * gl.jstride);
    } else {
#pragma unroll
        for (int j = 0; j < E; ++j)
            x[j] = V{};
    }
    if (ROW) {
#pragma unroll
        for (int j = 0; j < E; ++j)
            in_vector(x[j]);
    }
    register_stages<EB, E>(x);
    LaneStages<0, LB, GB, E, V, T>::run(x, lane);
    // The scale, times the sign the fp32 DPP lane stages leave.
    constexpr unsigned SM = (sizeof(T) == 4 && E >= 2) ? dpp_sign_lanes(GB, LB) : 0u;
    if (SM || la.do_scale) {
        T c = la.do_scale ? (T)la.scale : T(1);
        if (SM && (__popc((unsigned)lane & SM) & 1))
            c = -c;
#pragma unroll
        for (int j = 0; j < E; ++j)
            x[j] *= c;
    }
    if (ta.active) {
        with_store_policy(la.st_policy, [&](auto P) {
#pragma unroll
            for (int j = 0; j < E; ++j)
                store16<decltype(P)::value, V>(ta.p, gl.base + (uint32_t)j * gl.jstride, x[j]);
        });
    }
}

// ---- lane-exchange tiles: lane stages plus LDS exchanges of wave bits ---
//
// A tile of 2^KR rows x 2^GB 16-byte column groups (row passes: GB = 0, a
// row is one 16-byte vector) in one workgroup of 2^(6 + W) threads, each
// holding E = 2^EB vectors, KR = LR + W + EB with LR = 6 - GB.  A lane
// holds column group lane mod 2^GB and the LR lowest row bits, whose stages
// cross lanes as in wave_kernel.  In the load layout the W wave bits are
// row bits [LR, LR + W) and the register bits the top EB row bits.  After
// the register, lane and (row passes) in-vector stages, each exchange
// through LDS swaps the next min(EB, bits left) wave bits with the low
// register bits, whose stages then run in registers: ceil(W / EB)
// exchanges in all.  Lane bits keep their rows, so the lanes of a wave
// touch 64 consecutive 16-byte LDS slots (slot = row * 2^GB + group): the
// exchanges need no padding.  (With EB >= 2 + PHB, lane bits 4 and 5 stay
// exchanged with register bits 0 and 1 after their stages, lane_stage_nr;
// the first exchange's writes then cover four runs of 16 consecutive slots
// per wave, still conflict-free, and its reads restore the plain layout.)
// In memory a wave covers 2^LR rows of 2^GB consecutive 16-byte groups
// (1 KiB for row passes).
//
// With PHB > 0 (one exchange, W < EB) the exchange runs in 2^PHB phases:
// the top PHB register bits do not move, they are the top row bits in both
// layouts, so phase ph moves the registers whose top bits are ph through
// an LDS region 2^PHB times smaller than the tile, and two tiles of 128 KiB
// fit one CU.

// Row bit held by wave bit i (register bit i when REG) after X exchanges.
template <int W, int EB, int LR>
__host__ __device__ constexpr int lx_pos(int x, int i, bool reg)
{
    int wp[4] = {LR, LR + 1, LR + 2, LR + 3};
    int rp[5] = {LR + W, LR + W + 1, LR + W + 2, LR + W + 3, LR + W + 4};
    for (int e = 0; e < x; ++e) {
        const int c = W - e * EB < EB ? W - e * EB : EB;
        for (int q = 0; q < c; ++q) {
            const int t = wp[e * EB + q];
            wp[e * EB + q] = rp[q];
            rp[q] = t;
        }
    }
    return reg ? rp[i] : wp[i];
}

// Row bits of register j in layout X: a compile-time constant once j is
// unrolled.
template <int W, int EB, int LR, int X>
__device__ __forceinline__ constexpr uint32_t lx_reg_row(int j)
{
    uint32_t r = 0;
    for (int i = 0; i < EB; ++i)
        r |= (uint32_t)((j >> i) & 1) << lx_pos<W, EB, LR>(X, i, true);
    return r;
}

// Row bits held by the thread (lane row bits and wave bits) in layout X.
template <int W, int EB, int LR, int X>
__device__ __forceinline__ uint32_t lx_thread_row(int lane_row, int wave)
{
    uint32_t r = (uint32_t)lane_row;
#pragma unroll
    for (int i = 0; i < W; ++i)
        r |= (uint32_t)((wave >> i) & 1) << lx_pos<W, EB, LR>(X, i, false);
    return r;
}

// The load layout after lane_stage_nr on lane bits 4 and 5 (both are
// lane row bits, GB <= 4): lane bits 4, 5 hold the row bits of register
// bits 0, 1 (LR + W, LR + W + 1), and register bits 0, 1 hold rows 4 - GB
// and 5 - GB.
template <int W, int EB, int LR, int GB>
__device__ __forceinline__ constexpr uint32_t lx_reg_row_rl(int j)
{
    return lx_reg_row<W, EB, LR, 0>(j & ~3) | ((uint32_t)(j & 1) << (4 - GB)) |
           ((uint32_t)((j >> 1) & 1) << (5 - GB));
}
template <int W, int EB, int LR, int GB>
__device__ __forceinline__ uint32_t lx_thread_row_rl(int lane_row, int wave)
{
    const uint32_t lr = (uint32_t)lane_row;
    const uint32_t keep = lr & ~((1u << (4 - GB)) | (1u << (5 - GB)));
    return lx_thread_row<W, EB, LR, 0>((int)keep, wave) | (((lr >> (4 - GB)) & 1u) << (LR + W)) |
           (((lr >> (5 - GB)) & 1u) << (LR + W + 1));
}

// Exchanges X + 1 .. NX: move the next wave bits into the low register
// bits through LDS, then their stages.  RL: the data arrive in the
// relabelled load layout of lane_stage_nr, which the first exchange's
// writes undo (its reads, and everything after, use the plain layouts).
// The stage on the top register bit the last exchange moves is left to the
// caller (lx_last_bit), which fuses it with the scale.
template <typename V, int KR, int GB, int W, int EB, int PHB, int X, int NX, bool RL>
struct LxRounds {
    __device__ __forceinline__ static void run(V* x, V* L, int lane_row, int g, int wave)
    {
        constexpr int LR = 6 - GB;
        constexpr int E = 1 << EB;
        constexpr int C = W - X * EB < EB ? W - X * EB : EB;   // wave bits moved
        constexpr int EP = E >> PHB;                           // registers per phase
        constexpr uint32_t MASK = (1u << (KR + GB - PHB)) - 1; // slot within a phase
        constexpr bool R = RL && X == 0;
        static_assert(PHB == 0 || (NX == 1 && EB - C >= PHB), "phases keep their bits");
        static_assert(!RL || EB >= 2 + PHB, "relabelled register bits lie below the phase bits");
        const uint32_t from = ((R ? lx_thread_row_rl<W, EB, LR, GB>(lane_row, wave)
                                  : lx_thread_row<W, EB, LR, X>(lane_row, wave)) << GB) |
                              (uint32_t)g;
        const uint32_t to = (lx_thread_row<W, EB, LR, X + 1>(lane_row, wave) << GB) | (uint32_t)g;
#pragma unroll
        for (int ph = 0; ph < (1 << PHB); ++ph) {
            if (X > 0 || ph > 0)
                __syncthreads();   // the previous reads of this region are done
#pragma unroll
            for (int j = ph * EP; j < (ph + 1) * EP; ++j)
                L[(from + ((R ? lx_reg_row_rl<W, EB, LR, GB>(j) : lx_reg_row<W, EB, LR, X>(j))
                           << GB)) & MASK] = x[j];
            __syncthreads();
#pragma unroll
            for (int j = ph * EP; j < (ph + 1) * EP; ++j)
                x[j] = L[(to + (lx_reg_row<W, EB, LR, X + 1>(j) << GB)) & MASK];
        }
        register_stages<X + 1 == NX ? C - 1 : C, E>(x);
        LxRounds<V, KR, GB, W, EB, PHB, X + 1, NX, RL>::run(x, L, lane_row, g, wave);
    }
};
template <typename V, int KR, int GB, int W, int EB, int PHB, int NX, bool RL>
struct LxRounds<V, KR, GB, W, EB, PHB, NX, NX, RL> {
    __device__ __forceinline__ static void run(V*, V*, int, int, int) {}
};

// Compile-time shape of a lane-exchange tile and the steps of one tile:
// address, load, transform, store.
template <typename T, int KR_, int EB_, int W_, int PHB_, int GB_, bool ROW_>
struct LxShape {
    using V = typename Vec<T>::type;
    static constexpr int KR = KR_, EB = EB_, W = W_, PHB = PHB_, GB = GB_;
    static constexpr bool ROW = ROW_;
    static constexpr int WB = Vec<T>::WB;
    static constexpr int E = 1 << EB;
    static constexpr int LR = 6 - GB;              // row bits held by lanes
    static constexpr int NX = (W + EB - 1) / EB;   // exchanges
    // register bit of the last stage, the top one the last exchange moves
    static constexpr int LAST = (W - (NX - 1) * EB < EB ? W - (NX - 1) * EB : EB) - 1;
    static constexpr bool SPLIT = W < EB;          // top row bit stays a register bit
    // Row tiles of 8 or more registers per lane use the mirrored lane order
    // (mirrored_lane), so that lane bit 2 is a DPP stage too: a DPP
    // multiply-add in fp32, two DPP moves and a multiply-add in fp64.
    // (With 2 or 4 fp32 registers the fixed wait states of each DPP stage
    // cost more than the swizzles they replace: n = 13 +1.7 %, n = 20
    // +0.13 %, against n = 14 -4.8 %, n = 15 -2.7 % with 8; fp64 n = 13
    // -4.5 %, n = 24 -0.4 %.)
    static constexpr bool MI = GB == 0 && EB >= 3;
    static_assert(KR == EB + LR + W && EB >= 1 && W >= 1 && W <= 4, "lane-exchange tile");
    static_assert(!ROW || GB == 0, "row passes have one column group");
};

// Workgroup-uniform base of tile t; lanes then address group g of row r at
// (g << 4) + (r << rsh) bytes from it.
template <typename S, typename T>
__device__ __forceinline__ unsigned char* lx_tile_base(T* buf, const TileArgs& a, int64_t t,
                                                       uint32_t* rsh)
{
    int64_t base;
    if (S::ROW) {
        base = t << (S::KR + S::WB);
        *rsh = 4;
    } else {
        const int64_t blk_mask = ((int64_t)1 << a.nblk_bits) - 1;
        base = ((t >> a.nblk_bits) << (a.lo + S::KR)) + ((t & blk_mask) << (S::GB + S::WB));
        *rsh = (uint32_t)a.lo + (sizeof(T) == 8 ? 3u : 2u);
    }
    return reinterpret_cast<unsigned char*>(buf + base);
}

// When the exchange moves fewer wave bits than there are register bits
// (W < EB), the top row bit is the top register bit in the load and the
// store layout.  The registers with it set then address from a second base
// half a tile further on, so 32-bit lane offsets need only span half the
// tile: a column tile may span up to 8 GiB (fp64 n = 30, bits 20..29).
// Which base a register uses is a compile-time choice.
template <typename S, int X>
__device__ __forceinline__ const unsigned char* lx_reg_base(int j, const unsigned char* p,
                                                            const unsigned char* p_hi)
{
    return (S::SPLIT && ((j >> (S::EB - 1)) & 1)) ? p_hi : p;
}
template <typename S, int X>
__device__ __forceinline__ constexpr uint32_t lx_reg_off_row(int j)
{
    const uint32_t r = lx_reg_row<S::W, S::EB, S::LR, X>(j);
    return S::SPLIT ? (r & ~(1u << (S::KR - 1))) : r;
}

template <typename S>
__device__ __forceinline__ void lx_load(typename S::V* x, const unsigned char* p,
                                        const unsigned char* p_hi, uint32_t gbase, uint32_t rsh,
                                        uint32_t r0, int nt)
{
    using V = typename S::V;
    if (nt) {
#pragma unroll
        for (int j = 0; j < S::E; ++j)
            x[j] = load16_nt<V>(lx_reg_base<S, 0>(j, p, p_hi),
                                gbase + ((r0 + lx_reg_off_row<S, 0>(j)) << rsh));
    } else {
#pragma unroll
        for (int j = 0; j < S::E; ++j)
            x[j] = load16<V>(lx_reg_base<S, 0>(j, p, p_hi),
                             gbase + ((r0 + lx_reg_off_row<S, 0>(j)) << rsh));
    }
}

// Every stage of the tile, then the scale; leaves x in the layout of the
// last exchange.  The first exchange writes LDS without a barrier before
// it, so a caller that reuses L for another tile must place one first.
template <typename S, typename T>
__device__ __forceinline__ void lx_process(typename S::V* x, typename S::V* L, int lane,
                                           int lane_row, int g, int wave, int do_scale,
                                           double scale)
{
    using V = typename S::V;
    if (S::ROW) {
#pragma unroll
        for (int j = 0; j < S::E; ++j)
            in_vector(x[j]);
    }
    register_stages<S::EB, S::E>(x);
    // Lane bits 4 and 5 leave their swaps in place when register bits 0 and
    // 1 lie below the phase bits: the first exchange's writes relabel.
    constexpr bool RL = S::EB >= 2 + S::PHB;
    if constexpr (RL)
        LaneStagesNR<0, S::LR, S::GB, S::E, V, T, S::MI>::run(x, lane);
    else
        LaneStages<0, S::LR, S::GB, S::E, V, T, S::MI>::run(x, lane);
    LxRounds<V, S::KR, S::GB, S::W, S::EB, S::PHB, 0, S::NX, RL>::run(x, L, lane_row, g, wave);
    // The last stage.  Where the fp32 DPP lane stages (bits 0, 1, 3) leave a
    // sign (lanes keep their lane bits through the exchanges), it is fused
    // with the scale times that sign: for a scale that is a power of two
    // (even n) or +-1 the fused form gives the same bits as the butterfly
    // and then the multiply; for odd n it rounds c b first, within one unit
    // of the other order.  Elsewhere the multiply follows the butterfly (a
    // fused form behind a run-time branch costs these kernels 30 VGPRs).
    constexpr unsigned SM = sizeof(T) == 4 ? dpp_sign_lanes(S::GB, S::LR, S::MI) : 0u;
    constexpr int LB = 1 << S::LAST;
    if constexpr (SM != 0) {
        T c = do_scale ? (T)scale : T(1);
        if (__popc((unsigned)lane & SM) & 1)
            c = -c;
#pragma unroll
        for (int j = 0; j < S::E; ++j)
            if (!(j & LB))
                butterfly_scaled(x[j], x[j | LB], c);
    } else {
#pragma unroll
        for (int j = 0; j < S::E; ++j)
            if (!(j & LB))
                butterfly(x[j], x[j | LB]);
        if (do_scale) {
            const T c = (T)scale;
#pragma unroll
            for (int j = 0; j < S::E; ++j)
                x[j] *= c;
        }
    }
}

template <typename S>
__device__ __forceinline__ void lx_store(const typename S::V* x, unsigned char* p,
                                         unsigned char* p_hi, uint32_t gbase, uint32_t rsh,
                                         uint32_t rf, int pol)
{
    using V = typename S::V;
    with_store_policy(pol, [&](auto P) {
#pragma unroll
        for (int j = 0; j < S::E; ++j)
            store16<decltype(P)::value, V>(
                const_cast<unsigned char*>(lx_reg_base<S, S::NX>(j, p, p_hi)),
                gbase + ((rf + lx_reg_off_row<S, S::NX>(j)) << rsh), x[j]);
    });
}

template <typename T, int KR, int EB, int W, int PHB, int GB, bool ROW>
__global__ void __launch_bounds__(64 << W)
    lx_kernel(T* __restrict__ re, T* __restrict__ im, TileArgs a)
{
    using S = LxShape<T, KR, EB, W, PHB, GB, ROW>;
    using V = typename S::V;
    extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
    V* const L = reinterpret_cast<V*>(lds_raw);
    const int64_t t = a.tile0 + xcd_group(blockIdx.x, a.xcd_bits, a.wg_count);
    if (t >= a.tiles)
        return;   // uniform across the workgroup
    const LateArgs la = late_args(a);
    // The logical lane: which rows this lane holds (mirrored_lane for fp32
    // row tiles); addresses, LDS slots and stage signs all follow it.
    const int lane = S::MI ? mirrored_lane(threadIdx.x & 63) : (threadIdx.x & 63);
    const int wave = threadIdx.x >> 6;
    const int g = lane & ((1 << GB) - 1);
    const int lane_row = lane >> GB;
    uint32_t rsh;
    unsigned char* const p = lx_tile_base<S>(blockIdx.y ? im : re, a, t, &rsh);
    unsigned char* const p_hi = p + ((uint64_t)1 << (KR - 1) << rsh);
    const uint32_t gbase = (uint32_t)g << 4;
    V x[S::E];
    lx_load<S>(x, p, p_hi, gbase, rsh, lx_thread_row<W, EB, S::LR, 0>(lane_row, wave), a.ld_nt);
    lx_process<S, T>(x, L, lane, lane_row, g, wave, la.do_scale, la.scale);
    lx_store<S>(x, p, p_hi, gbase, rsh, lx_thread_row<W, EB, S::LR, S::NX>(lane_row, wave),
                la.st_policy);
}

__global__ void __launch_bounds__(256)
    pair_f32_kernel(float* __restrict__ re, float* __restrict__ im, int64_t pairs, int do_scale,
                    float scale)
{
    typedef float f2 __attribute__((ext_vector_type(2)));
    f2* const buf = reinterpret_cast<f2*>(blockIdx.y ? im : re);
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < pairs; i += stride) {
        const f2 v = buf[i];
        f2 r;
        r.x = v.x + v.y;
        r.y = v.x - v.y;
        if (do_scale)
            r *= scale;
        buf[i] = r;
    }
}

// Streaming copy: each workgroup moves 256 threads x 8 vectors of 16 bytes,
// all loads issued before the stores, like a pass's tile.
__global__ void __launch_bounds__(256)
    stream_copy_kernel(int4* __restrict__ dst, const int4* __restrict__ src, int64_t nvec)
{
    constexpr int U = 8;
    const int64_t chunk = (int64_t)blockDim.x * U;
    for (int64_t b = (int64_t)blockIdx.x * chunk; b < nvec; b += (int64_t)gridDim.x * chunk) {
        const int64_t i0 = b + threadIdx.x;
        if (b + chunk <= nvec) {
            int4 v0 = src[i0], v1 = src[i0 + 256], v2 = src[i0 + 512], v3 = src[i0 + 768];
            int4 v4 = src[i0 + 1024], v5 = src[i0 + 1280], v6 = src[i0 + 1536];
            int4 v7 = src[i0 + 1792];
            dst[i0] = v0;
            dst[i0 + 256] = v1;
            dst[i0 + 512] = v2;
            dst[i0 + 768] = v3;
            dst[i0 + 1024] = v4;
            dst[i0 + 1280] = v5;
            dst[i0 + 1536] = v6;
            dst[i0 + 1792] = v7;
        } else {
            for (int64_t i = i0; i < nvec; i += blockDim.x)
                dst[i] = src[i];
        }
    }
}

struct Entry {
    KernelKey key;
    const void* fn;
};

template <typename T, bool ROW, int KR, int EB, int GB, int PHB>
void add_variant(std::vector<Entry>& v)
{
    v.push_back({{sizeof(T) == 8 ? 1 : 0, KR, EB, GB, PHB, ROW ? 1 : 0, 0, 0},
                 reinterpret_cast<const void*>(&tile_kernel<T, KR, EB, GB, PHB, ROW>)});
    // The pipelined form, for tiles of at least 32 KiB whose workgroup fits
    // 512 threads (it holds two register sets).
    if constexpr (KR + GB >= 11 && KR - EB + GB <= 9 && EB <= 4)
        v.push_back({{sizeof(T) == 8 ? 1 : 0, KR, EB, GB, PHB, ROW ? 1 : 0, 1, 0},
                     reinterpret_cast<const void*>(&tile_kernel_pipe<T, KR, EB, GB, PHB, ROW>)});
}

// Column groups 2^GB for GB in [0, 4] (row passes: GB = 0) whose tile fits
// 160 KiB of LDS and 1024 (EB <= 4) or 512 (EB = 5) threads; column passes
// of at least 9 row bits and 8 groups also get the phased exchange
// (PHB = 1, 2).
template <typename T, bool ROW, int KR, int EB, int GB>
void add_groups(std::vector<Entry>& v)
{
    constexpr int max_tt_bits = EB >= 5 ? 9 : 10;
    if constexpr ((KR - EB + GB) <= max_tt_bits) {
        constexpr long slots = 1L << (KR + GB);
        constexpr long lds = 16 * (slots + (slots >> (EB + GB)));
        if constexpr (KR <= EB || lds <= 160 * 1024)
            add_variant<T, ROW, KR, EB, GB, 0>(v);
        if constexpr (!ROW && KR >= 9 && GB >= 3 && KR > EB) {
            add_variant<T, ROW, KR, EB, GB, 1>(v);
            add_variant<T, ROW, KR, EB, GB, 2>(v);
        }
    }
    if constexpr (!ROW && GB < 4)
        add_groups<T, ROW, KR, EB, GB + 1>(v);
}

// Variants for every KR in [KRMIN, KR]: EB = min(KR, 4), plus EB = 3 and
// (row passes) EB = 5 where they fit.
template <typename T, bool ROW, int KR, int KRMIN>
struct Register {
    static void add(std::vector<Entry>& v)
    {
        add_groups<T, ROW, KR, (KR < 4 ? KR : 4), 0>(v);
        if constexpr (ROW && KR >= 5)
            add_groups<T, ROW, KR, 5, 0>(v);
        if constexpr (KR >= 4)
            add_groups<T, ROW, KR, 3, 0>(v);
        if constexpr (KR > KRMIN)
            Register<T, ROW, KR - 1, KRMIN>::add(v);
    }
};

// Wave-tile kernels: EB = the fewest register bits that leave at most
// 6 - GB row bits for the lanes (at least 1 when lane bits 4/5 are used,
// whose swaps pair registers), and one more where it fits.
template <typename T, bool ROW, int KR, int GB, int EB>
void add_wave(std::vector<Entry>& v)
{
    constexpr int LB = KR - EB;
    if constexpr (EB >= 0 && EB <= 5 && EB <= KR && LB >= 0 && LB + GB <= 6 &&
                  !(EB == 0 && LB + GB >= 5))
        v.push_back({{sizeof(T) == 8 ? 1 : 0, KR, EB, GB, 0, ROW ? 1 : 0, 0, 1},
                     reinterpret_cast<const void*>(&wave_kernel<T, KR, EB, GB, ROW>)});
}

template <typename T, bool ROW, int KR, int GB>
struct WaveVariants {
    static constexpr int lane_room = 6 - GB;
    static constexpr int eb0 = KR - lane_room > 0 ? KR - lane_room : 0;
    static void add(std::vector<Entry>& v)
    {
        add_wave<T, ROW, KR, GB, eb0>(v);
        add_wave<T, ROW, KR, GB, eb0 + 1>(v);
        if constexpr (!ROW && GB < 4)
            WaveVariants<T, ROW, KR, GB + 1>::add(v);
    }
};

template <typename T, bool ROW, int KR, int KRMIN>
struct RegisterWave {
    static void add(std::vector<Entry>& v)
    {
        WaveVariants<T, ROW, KR, 0>::add(v);
        if constexpr (KR > KRMIN)
            RegisterWave<T, ROW, KR - 1, KRMIN>::add(v);
    }
};

// Lane-exchange tiles: W in [1, 4] with EB = KR - (6 - GB) - W in [2, 5],
// or EB = W = 1; tiles of 2^11+ slots with W < EB also in two phases.  Row
// passes (GB = 0) for KR in [8, 13]; column passes with 8 or 16 groups
// (128- or 256-byte row segments) for KR in [6, 11].
template <typename T, int KR, int W, int GB, bool ROW>
void add_lx(std::vector<Entry>& v)
{
    constexpr int EB = KR - (6 - GB) - W;
    if constexpr (W >= 1 && W <= 4 && ((EB >= 2 && EB <= 5) || (EB == 1 && W == 1))) {
        // LDS: 2^(KR + GB) 16-byte slots, halved by the phases; at most 128 KiB
        if constexpr (KR + GB <= 13)
            v.push_back({{sizeof(T) == 8 ? 1 : 0, KR, EB, GB, 0, ROW ? 1 : 0, 0, 2},
                         reinterpret_cast<const void*>(&lx_kernel<T, KR, EB, W, 0, GB, ROW>)});
        if constexpr (KR + GB >= 11 && KR + GB <= 14 && W < EB)
            v.push_back({{sizeof(T) == 8 ? 1 : 0, KR, EB, GB, 1, ROW ? 1 : 0, 0, 2},
                         reinterpret_cast<const void*>(&lx_kernel<T, KR, EB, W, 1, GB, ROW>)});
    }
}

template <typename T, int KR, int KRMIN, int GB, bool ROW>
struct LaneExchange {
    static void add(std::vector<Entry>& v)
    {
        add_lx<T, KR, 1, GB, ROW>(v);
        add_lx<T, KR, 2, GB, ROW>(v);
        add_lx<T, KR, 3, GB, ROW>(v);
        add_lx<T, KR, 4, GB, ROW>(v);
        if constexpr (KR > KRMIN)
            LaneExchange<T, KR - 1, KRMIN, GB, ROW>::add(v);
    }
};

const std::vector<Entry>& table()
{
    static const std::vector<Entry> t = [] {
        std::vector<Entry> v;
        RegisterWave<float, true, 11, 0>::add(v);
        RegisterWave<double, true, 11, 0>::add(v);
        RegisterWave<float, false, 11, 1>::add(v);
        RegisterWave<double, false, 11, 1>::add(v);
        LaneExchange<float, 13, 8, 0, true>::add(v);
        LaneExchange<double, 13, 8, 0, true>::add(v);
        LaneExchange<float, 11, 6, 3, false>::add(v);
        LaneExchange<float, 11, 6, 4, false>::add(v);
        LaneExchange<double, 11, 6, 3, false>::add(v);
        LaneExchange<double, 11, 6, 4, false>::add(v);
        Register<float, true, 13, 0>::add(v);
        Register<double, true, 13, 0>::add(v);
        Register<float, false, 12, 1>::add(v);
        Register<double, false, 12, 1>::add(v);
        return v;
    }();
    return t;
}

const void* find(const KernelKey& k)
{
    for (const Entry& e : table())
        if (e.key.f64 == k.f64 && e.key.kr == k.kr && e.key.eb == k.eb && e.key.gb == k.gb &&
            e.key.phb == k.phb && e.key.row == k.row && e.key.pipe == k.pipe &&
            e.key.wave == k.wave)
            return e.fn;
    return nullptr;
}

}  // namespace

bool kernel_available(const KernelKey& key) { return find(key) != nullptr; }

hipError_t kernels_init_device()
{
    for (const Entry& e : table()) {
        hipError_t err = hipFuncSetAttribute(e.fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                             160 * 1024);
        if (err != hipSuccess)
            return err;
    }
    return hipSuccess;
}

hipError_t launch_tile_pass(const KernelKey& key, void* re, void* im, int ncomp,
                            const TileArgs& args, unsigned block, size_t lds_bytes,
                            hipStream_t stream, hipEvent_t start, hipEvent_t stop)
{
    const void* fn = find(key);
    if (!fn)
        return hipErrorInvalidDeviceFunction;
    // One workgroup per group of 2^tpw_bits tiles; grids beyond 2^30
    // workgroups are split into several launches.  Timing events, when
    // given, are recorded at the first launch's start and the last launch's
    // end by the dispatch itself.
    constexpr int64_t kMaxGrid = (int64_t)1 << 30;
    TileArgs a = args;
    if (key.pipe) {
        // Persistent: `args.grid` workgroups (per component) walk all tile
        // groups.
        a.tile0 = 0;
        void* kargs[] = {&re, &im, &a};
        const int64_t nw = args.grid < args.wg_count ? args.grid : args.wg_count;
        const dim3 grid((unsigned)(nw > 0 ? nw : 1), (unsigned)ncomp, 1);
        if (start || stop)
            return hipExtLaunchKernel(fn, grid, dim3(block, 1, 1), kargs, lds_bytes, stream,
                                      start, stop, 0);
        return hipLaunchKernel(fn, grid, dim3(block, 1, 1), kargs, lds_bytes, stream);
    }
    for (int64_t w0 = 0; w0 < args.wg_count; w0 += kMaxGrid) {
        const int64_t nw = args.wg_count - w0 < kMaxGrid ? args.wg_count - w0 : kMaxGrid;
        const bool first = (w0 == 0), last = (w0 + nw >= args.wg_count);
        a.tile0 = w0 << args.tpw_bits;
        void* kargs[] = {&re, &im, &a};
        const dim3 grid((unsigned)nw, (unsigned)ncomp, 1);
        hipError_t e;
        if (start || stop)
            e = hipExtLaunchKernel(fn, grid, dim3(block, 1, 1), kargs, lds_bytes, stream,
                                   first ? start : nullptr, last ? stop : nullptr, 0);
        else
            e = hipLaunchKernel(fn, grid, dim3(block, 1, 1), kargs, lds_bytes, stream);
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

hipError_t launch_pair_f32(float* re, float* im, int64_t pairs, int do_scale, float scale,
                           hipStream_t stream, hipEvent_t start, hipEvent_t stop)
{
    const int64_t blocks64 = (pairs + 255) / 256;
    const unsigned blocks = (unsigned)(blocks64 < 65536 ? (blocks64 > 0 ? blocks64 : 1) : 65536);
    void* kargs[] = {&re, &im, &pairs, &do_scale, &scale};
    const void* fn = reinterpret_cast<const void*>(&pair_f32_kernel);
    const dim3 grid(blocks, im ? 2 : 1, 1);
    if (start || stop)
        return hipExtLaunchKernel(fn, grid, dim3(256, 1, 1), kargs, 0, stream, start, stop, 0);
    return hipLaunchKernel(fn, grid, dim3(256, 1, 1), kargs, 0, stream);
}

hipError_t launch_stream_copy(void* dst, const void* src, int64_t bytes, hipStream_t stream)
{
    const int64_t nvec = bytes / 16;
    const int64_t chunk = 256 * 8;
    int64_t blocks64 = (nvec + chunk - 1) / chunk;
    if (blocks64 < 1)
        blocks64 = 1;
    if (blocks64 > (1 << 30))
        blocks64 = 1 << 30;
    hipLaunchKernelGGL(stream_copy_kernel, dim3((unsigned)blocks64, 1, 1), dim3(256, 1, 1), 0,
                       stream, reinterpret_cast<int4*>(dst), reinterpret_cast<const int4*>(src),
                       nvec);
    return hipGetLastError();
}


}  // namespace qse
