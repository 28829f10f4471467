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

namespace qse {
namespace {

template <typename T>
struct Vec;
template <>
struct Vec<float> {
    typedef float type __attribute__((ext_vector_type(4)));
    static constexpr int WB = 2;  // log2 elements per 16-byte vector
};
template <>
struct Vec<double> {
    typedef double type __attribute__((ext_vector_type(2)));
    static constexpr int WB = 1;
};

__device__ __forceinline__ float fma_sign(float x, float s, float p)
{
    return __builtin_fmaf(x, s, p);
}
__device__ __forceinline__ double fma_sign(double x, double s, double p)
{
    return __builtin_fma(x, s, p);
}

template <typename V>
__device__ __forceinline__ void butterfly(V& a, V& b)
{
    const V s = a + b;
    const V d = a - b;
    a = s;
    b = d;
}

// The butterfly times c: (c (a + b), c (a - b)) as t = c b, fma(a, c, +-t):
// three operations for two outputs instead of four.  When c is a power of
// two (or +-1), c b is exact and the results equal, bit for bit, the
// butterfly followed by the multiply.
template <typename V, typename T>
__device__ __forceinline__ void butterfly_scaled(V& a, V& b, T c)
{
    constexpr int W = sizeof(V) / sizeof(T);
#pragma unroll
    for (int k = 0; k < W; ++k) {
        const T t = b[k] * c;
        const T u = a[k];
        a[k] = fma_sign(u, c, t);
        b[k] = fma_sign(u, c, -t);
    }
}

// Stages on the vb index bits inside one vector (row passes only).
__device__ __forceinline__ void in_vector(Vec<float>::type& v)
{
    const float s0 = v.x + v.y, d0 = v.x - v.y;   // bit 0: (0,1), (2,3)
    const float s1 = v.z + v.w, d1 = v.z - v.w;
    v.x = s0 + s1;                                // bit 1: (0,2), (1,3)
    v.z = s0 - s1;
    v.y = d0 + d1;
    v.w = d0 - d1;
}
__device__ __forceinline__ void in_vector(Vec<double>::type& v)
{
    const double s = v.x + v.y, d = v.x - v.y;
    v.x = s;
    v.y = d;
}

// Butterflies on register bits [0, NB) of x[0..E).
template <int NB, int E, typename V>
__device__ __forceinline__ void register_stages(V* x)
{
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
        for (int j = 0; j < E; ++j) {
            if (!(j & (1 << b)))
                butterfly(x[j], x[j | (1 << b)]);
        }
    }
}

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

template <int LBIT, bool MI = false>
__device__ __forceinline__ unsigned lane_partner_u32(unsigned v)
{
    if constexpr (LBIT == 0)
        return (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);  // quad [1,0,3,2]
    else if constexpr (LBIT == 1)
        return (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true);  // quad [2,3,0,1]
    else if constexpr (LBIT == 2 && MI)
        return (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, true); // row_half_mirror
    else if constexpr (LBIT == 2)
        return (unsigned)__builtin_amdgcn_ds_swizzle((int)v, (4 << 10) | 0x1F);   // xor 4
    else
        return (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, true); // row_ror:8
}

template <int LBIT, bool MI = false>
__device__ __forceinline__ float lane_partner(float v)
{
    return __uint_as_float(lane_partner_u32<LBIT, MI>(__float_as_uint(v)));
}
template <int LBIT, bool MI = false>
__device__ __forceinline__ double lane_partner(double v)
{
    const unsigned long long u = (unsigned long long)__double_as_longlong(v);
    const unsigned lo = lane_partner_u32<LBIT, MI>((unsigned)u);
    const unsigned hi = lane_partner_u32<LBIT, MI>((unsigned)(u >> 32));
    return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

// Swap lane bit 4 (LBIT = 4) or 5 with the register pair (a, b).
template <int LBIT>
__device__ __forceinline__ void permlane_swap_u32(unsigned& a, unsigned& b)
{
    if constexpr (LBIT == 4) {
        const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
        a = r[0];
        b = r[1];
    } else {
        const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
        a = r[0];
        b = r[1];
    }
}
template <int LBIT>
__device__ __forceinline__ void permlane_swap(float& a, float& b)
{
    unsigned ua = __float_as_uint(a), ub = __float_as_uint(b);
    permlane_swap_u32<LBIT>(ua, ub);
    a = __uint_as_float(ua);
    b = __uint_as_float(ub);
}
template <int LBIT>
__device__ __forceinline__ void permlane_swap(double& a, double& b)
{
    const unsigned long long ua = (unsigned long long)__double_as_longlong(a);
    const unsigned long long ub = (unsigned long long)__double_as_longlong(b);
    unsigned alo = (unsigned)ua, ahi = (unsigned)(ua >> 32);
    unsigned blo = (unsigned)ub, bhi = (unsigned)(ub >> 32);
    permlane_swap_u32<LBIT>(alo, blo);
    permlane_swap_u32<LBIT>(ahi, bhi);
    a = __longlong_as_double((long long)(((unsigned long long)ahi << 32) | alo));
    b = __longlong_as_double((long long)(((unsigned long long)bhi << 32) | blo));
}

// fp32 stages on lane bits 0, 1 and 3: one vector-ALU instruction per
// value, v_fmac_f32 with a DPP lane permutation on its first source (quad
// permutations for bits 0 and 1; for bit 3 a rotation of each 16-lane row
// by 8, which is lane xor 8), so each lane keeps x + s * partner (s = -1 on
// the upper lane of each pair).  The upper lane then holds the difference
// negated.  The negation is exact and carries through every later stage
// unchanged (a stage's two operands come from lanes with equal bits 0, 1
// and 3, so they carry the same sign), and the kernel removes it with its
// final scaling (dpp_sign_lanes).  Each
// asm block begins with five wait states: a DPP read of a VGPR needs two
// after a vector-ALU write of it, and a DPP instruction five after a write
// of EXEC; the compiler cannot see the DPP inside the block.
#define QSE_FMAC_DPP(Q, R, S) "v_fmac_f32_dpp %" #R ", %" #R ", %" #S " " Q \
                              " row_mask:0xf bank_mask:0xf\n\t"
#define QSE_FMAC_DPP_0(Q, S)                                                           \
    QSE_FMAC_DPP(Q, 0, S) QSE_FMAC_DPP(Q, 1, S) QSE_FMAC_DPP(Q, 2, S) QSE_FMAC_DPP(Q, 3, S) \
        QSE_FMAC_DPP(Q, 4, S) QSE_FMAC_DPP(Q, 5, S) QSE_FMAC_DPP(Q, 6, S) QSE_FMAC_DPP(Q, 7, S)
#define QSE_FMAC_DPP_8(Q, S)                                                             \
    QSE_FMAC_DPP(Q, 8, S) QSE_FMAC_DPP(Q, 9, S) QSE_FMAC_DPP(Q, 10, S) QSE_FMAC_DPP(Q, 11, S) \
        QSE_FMAC_DPP(Q, 12, S) QSE_FMAC_DPP(Q, 13, S) QSE_FMAC_DPP(Q, 14, S)                \
            QSE_FMAC_DPP(Q, 15, S)
#define QSE_FMAC_DPP_16(Q, S)                                                               \
    QSE_FMAC_DPP(Q, 16, S) QSE_FMAC_DPP(Q, 17, S) QSE_FMAC_DPP(Q, 18, S) QSE_FMAC_DPP(Q, 19, S) \
        QSE_FMAC_DPP(Q, 20, S) QSE_FMAC_DPP(Q, 21, S) QSE_FMAC_DPP(Q, 22, S)                  \
            QSE_FMAC_DPP(Q, 23, S)
#define QSE_FMAC_DPP_24(Q, S)                                                               \
    QSE_FMAC_DPP(Q, 24, S) QSE_FMAC_DPP(Q, 25, S) QSE_FMAC_DPP(Q, 26, S) QSE_FMAC_DPP(Q, 27, S) \
        QSE_FMAC_DPP(Q, 28, S) QSE_FMAC_DPP(Q, 29, S) QSE_FMAC_DPP(Q, 30, S)                  \
            QSE_FMAC_DPP(Q, 31, S)
// Eight in-out operands v[b .. b + 7].
#define QSE_OPS8(b)                                                                       \
    "+v"(v[b]), "+v"(v[b + 1]), "+v"(v[b + 2]), "+v"(v[b + 3]), "+v"(v[b + 4]), "+v"(v[b + 5]), \
        "+v"(v[b + 6]), "+v"(v[b + 7])
// The stage on 8, 16 or 32 values with DPP control Q; s is the last
// operand.
#define QSE_DPP_STAGE(Q)                                                                     \
    if constexpr (NR == 2)                                                                   \
        asm("s_nop 4\n\t" QSE_FMAC_DPP_0(Q, 8) : QSE_OPS8(0) : "v"(s));                       \
    else if constexpr (NR == 4)                                                              \
        asm("s_nop 4\n\t" QSE_FMAC_DPP_0(Q, 16) QSE_FMAC_DPP_8(Q, 16)                          \
            : QSE_OPS8(0), QSE_OPS8(8)                                                        \
            : "v"(s));                                                                        \
    else                                                                                     \
        asm("s_nop 4\n\t" QSE_FMAC_DPP_0(Q, 32) QSE_FMAC_DPP_8(Q, 32) QSE_FMAC_DPP_16(Q, 32)   \
                QSE_FMAC_DPP_24(Q, 32)                                                        \
            : QSE_OPS8(0), QSE_OPS8(8), QSE_OPS8(16), QSE_OPS8(24)                            \
            : "v"(s));

// One stage on lane bit LBIT over the NR = 2, 4 or 8 fp32 registers at x.
template <int LBIT, int NR>
__device__ __forceinline__ void fmac_dpp_regs(Vec<float>::type* x, float s)
{
    static_assert(LBIT >= 0 && LBIT <= 3, "DPP pairs lanes within a row of 16");
    static_assert(NR == 2 || NR == 4 || NR == 8, "blocks of 2, 4 or 8 registers");
    float v[4 * NR];
#pragma unroll
    for (int j = 0; j < NR; ++j)
#pragma unroll
        for (int c = 0; c < 4; ++c)
            v[4 * j + c] = x[j][c];
    if constexpr (LBIT == 0) {
        QSE_DPP_STAGE("quad_perm:[1,0,3,2]")
    } else if constexpr (LBIT == 1) {
        QSE_DPP_STAGE("quad_perm:[2,3,0,1]")
    } else if constexpr (LBIT == 2) {
        QSE_DPP_STAGE("row_half_mirror")
    } else {
        QSE_DPP_STAGE("row_ror:8")
    }
#pragma unroll
    for (int j = 0; j < NR; ++j)
        x[j] = Vec<float>::type{v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]};
}
#undef QSE_DPP_STAGE
#undef QSE_OPS8
#undef QSE_FMAC_DPP_24
#undef QSE_FMAC_DPP_16
#undef QSE_FMAC_DPP_8
#undef QSE_FMAC_DPP_0
#undef QSE_FMAC_DPP

// Lane bits among 0, 1, 3 (and 2 with the mirrored lane order below) whose
// fp32 stages leave a sign (those in [gb, gb + lb), the lane row bits of a
// tile); a lane's outputs carry (-1)^popcount(logical lane & mask).
__host__ __device__ constexpr unsigned dpp_sign_lanes(int gb, int lb, bool mirror = false)
{
    return (gb <= 0 && lb > 0 ? 1u : 0u) | (gb <= 1 && gb + lb > 1 ? 2u : 0u) |
           (mirror && gb <= 2 && gb + lb > 2 ? 4u : 0u) | (gb <= 3 && gb + lb > 3 ? 8u : 0u);
}

// Mirrored lane order: in each group of 8 lanes the upper 4 hold their rows
// in reverse (logical lane = lane ^ 3 when lane bit 2 is set).  Lane xor 4
// on logical lanes is then DPP row_half_mirror on physical ones (lane ->
// 7 - lane in each group of 8), while xor 1, 2 and 8 stay the quad
// permutations and the row rotation: they leave bit 2 alone.
__device__ __forceinline__ int mirrored_lane(int lane)
{
    return lane ^ (((lane >> 2) & 1) * 3);
}

// Stage on lane bit LBIT for all E registers; `lane` is the logical lane
// (mirrored_lane when MI).
template <int LBIT, int E, typename V, typename T, bool MI = false>
__device__ __forceinline__ void lane_stage(V* x, int lane)
{
    constexpr int W = sizeof(V) / sizeof(T);
    if constexpr ((LBIT < 2 || LBIT == 3 || (MI && LBIT == 2)) && sizeof(T) == 4 && E >= 2) {
        const float s = ((lane >> LBIT) & 1) ? -1.f : 1.f;
        constexpr int NR = E < 8 ? E : 8;
#pragma unroll
        for (int j = 0; j < E; j += NR)
            fmac_dpp_regs<LBIT, NR>(x + j, s);
    } else if constexpr (LBIT < 4) {
        const T s = ((lane >> LBIT) & 1) ? T(-1) : T(1);
#pragma unroll
        for (int j = 0; j < E; ++j) {
#pragma unroll
            for (int c = 0; c < W; ++c) {
                const T v = x[j][c];
                x[j][c] = fma_sign(v, s, lane_partner<LBIT, MI>(v));
            }
        }
    } else {
        static_assert(E >= 2, "lane bits 4 and 5 pair registers");
#pragma unroll
        for (int j = 0; j < E; j += 2) {
#pragma unroll
            for (int c = 0; c < W; ++c) {
                T a = x[j][c], b = x[j + 1][c];
                permlane_swap<LBIT>(a, b);
                const T sum = a + b, dif = a - b;
                a = sum;
                b = dif;
                permlane_swap<LBIT>(a, b);
                x[j][c] = a;
                x[j + 1][c] = b;
            }
        }
    }
}

// The same stage, except that lane bits 4 and 5 are left exchanged with
// register bits 0 and 1: the second swap of each pair is dropped.  After
// it, lane bit 4 (5) holds the row bit register bit 0 (1) held, and
// register bit 0 (1) holds the row bit of lane bit 4 (5); a caller must
// address the data with that relabelling (lx_thread_row_rl, lx_reg_row_rl).
template <int LBIT, int E, typename V, typename T, bool MI = false>
__device__ __forceinline__ void lane_stage_nr(V* x, int lane)
{
    constexpr int W = sizeof(V) / sizeof(T);
    if constexpr (LBIT < 4) {
        lane_stage<LBIT, E, V, T, MI>(x, lane);
    } else {
        constexpr int RB = LBIT - 4;   // register bit paired with the lane bit
        static_assert(E >= 4, "lane bits 4 and 5 pair register bits 0 and 1");
#pragma unroll
        for (int j = 0; j < E; ++j) {
            if (j & (1 << RB))
                continue;
#pragma unroll
            for (int c = 0; c < W; ++c) {
                T a = x[j][c], b = x[j | (1 << RB)][c];
                permlane_swap<LBIT>(a, b);
                x[j][c] = a + b;
                x[j | (1 << RB)][c] = a - b;
            }
        }
    }
}

template <int B, int LB, int GB, int E, typename V, typename T, bool MI = false>
struct LaneStagesNR {
    __device__ __forceinline__ static void run(V* x, int lane)
    {
        lane_stage_nr<GB + B, E, V, T, MI>(x, lane);
        LaneStagesNR<B + 1, LB, GB, E, V, T, MI>::run(x, lane);
    }
};
template <int LB, int GB, int E, typename V, typename T, bool MI>
struct LaneStagesNR<LB, LB, GB, E, V, T, MI> {
    __device__ __forceinline__ static void run(V*, int) {}
};

template <int B, int LB, int GB, int E, typename V, typename T, bool MI = false>
struct LaneStages {
    __device__ __forceinline__ static void run(V* x, int lane)
    {
        lane_stage<GB + B, E, V, T, MI>(x, lane);
        LaneStages<B + 1, LB, GB, E, V, T, MI>::run(x, lane);
    }
};
template <int LB, int GB, int E, typename V, typename T, bool MI>
struct LaneStages<LB, LB, GB, E, V, T, MI> {
    __device__ __forceinline__ static void run(V*, int) {}
};

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

// ---- one HBM pass for fp32 n = 20: groups of workgroups on one XCD -----
//
// The Kronecker split H_20 = H_5 (x) H_15 (Apache Mahout pull request
// "[QDP] [feature] Pr4 kronecker fwt", sections "Why" and "How"; iThome
// "Day 18" article, "Kronecker block GEMM idea") without a second pass
// over HBM.  A vector component is a 32 x 2^15 matrix: row m is the
// 2^15-element block whose element bits 15..19 equal m.  Workgroup m of a
// group (32 workgroups, one per CU of one XCD) loads row m into its
// registers and applies H_15 to it (the row factor); the group then moves
// the matrix through a ring buffer that stays in the XCD's L2, so that
// workgroup m ends up holding the 1024-column slice m of all 32 rows, and
// applies H_5 down the columns (the column factor) before storing.  HBM
// sees one read and one write of the state; the intermediate only crosses
// the L2.
//
// Layouts (element bits of a row block; lanes l = 0..63, waves w = 0..7,
// 16 float4 registers j per thread; bits 0-1 lie inside a float4):
//  load L0:  lanes 0-4 = bits 2-6, lane 5 = bit 10, waves = bits 7-9,
//            registers j = bit 14 << 3 | bits 11-13;
//  row L1:   after one LDS exchange, waves = bits 11-13 and registers
//            j = bit 14 << 3 | bits 7-9.  Element bits 10-14 are then the
//            destination column slice (lane 5, waves, register bit 3), and
//            register bits 0-2 (element bits 7-9) the ring slice s.
//  column R0 (as read from the ring): lanes 0-4 = bits 2-6 as before,
//            lane 5 = row bit 0, waves = row bits 1-3, registers
//            j = row bit 4 << 3 | s;
//  store R1: after one LDS exchange, waves = s and registers j = row bit 4
//            << 3 | row bits 1-3.
// Lanes 0-4 keep element bits 2-6 throughout, so the sign that the fp32
// DPP lane stages leave on lanes with odd popcount(lane & 0xB) is still
// attached to the same lanes at the end and is removed with the scale.
//
// The ring exchange, per slice s (8 per component, 512 KiB each, ring of 2
// slots per group): each workgroup stores its registers of slice s (the
// values for all 32 destinations), then loads slice s - 1 as written by
// every member, waits for both with one s_waitcnt, and publishes "slices
// written" and "slices read" in its two progress words (plain stores: they
// land in the XCD's L2).  Before storing into a slot it needs every member
// to have read the slice that last used it; before loading a slice, every
// member to have written it.  Wave 0 reads the group's 64 progress words
// with device-scope loads (sc1: they miss the CU's L1 and hit the L2; a
// device-scope atomic would leave the L2 and take about 1.2 us here) in
// the same round trip as the slice's data, so a wait costs a round trip
// only when a member is behind.  The slice loads are device-scope too: a
// plain load can return a line the CU's L1 kept from the slot's previous
// use.  Every member of a group runs on the same XCD: a workgroup reads its
// XCD and CU from the XCC_ID and HW_ID registers and joins a group with two
// atomic adds (the dispatcher deals the 512 workgroups to the 8 XCDs in
// turn, 64 each, two per CU, but the first XCD it serves varies), so one L2
// serves the group, and the two workgroups of a CU belong to different
// groups (two members of one group on one CU would halve that pair's
// share of the CU, and the whole group waits for them).  All 2 x 256 workgroups are resident together
// (at most 128 VGPRs and 64 KiB of LDS each), so every wait ends; the spin
// bounds are only a guard, recorded in the workspace's error word.
//
// Components are spread over the XCDs by index (c = xcd + 8 i) and over
// an XCD's two groups by a queue: the group's first workgroup takes the
// index of the group's next component with one atomic add while its loads
// are in flight, and publishes it for the group (double-buffered by the
// parity of the group's component count, so a fast leader cannot
// overwrite a value a slow member has not read).  The second workgroup on
// a CU issues later than the first, so a static split ended 20 % later.

constexpr int kOpSpin = 1 << 20;
constexpr int kOpRegs = 16;        // float4 per thread: a 2^15-element row block
constexpr int kOpRowF4 = 8192;     // float4 per row block

struct OnepassArgs {
    float* re;
    float* im;        // null: components are consecutive vectors of re
    unsigned char* ws;
    int ncomp;
    float scale;
};

__device__ __forceinline__ int xcc_id()
{
    int x;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(x));
    return x & 15;
}

typedef unsigned int op_u4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t op_rsrc(const void* p)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, -1, 0x00020000);
}
// 16-byte buffer accesses with a cache-policy operand: 2 = nontemporal,
// 16 = device scope (sc1), 0 = plain.
template <int AUX>
__device__ __forceinline__ Vec<float>::type op_load(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                    uint32_t soff)
{
    return __builtin_bit_cast(Vec<float>::type,
                              __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, AUX));
}
template <int AUX>
__device__ __forceinline__ void op_store(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                         const Vec<float>::type& v)
{
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(op_u4, v), r, (int)voff, (int)soff,
                                           AUX);
}
constexpr int kOpNt = 2, kOpDevice = 16;

// Keeps the compiler from sinking the stages into their consumers (which
// keeps their inputs alive and spills).
__device__ __forceinline__ void op_pin(Vec<float>::type (&x)[kOpRegs])
{
#pragma unroll
    for (int j = 0; j < kOpRegs; ++j)
        asm volatile("" : "+v"(x[j]));
}

__global__ void __launch_bounds__(kOpThreads)
    onepass_reset_kernel(unsigned char* ws)
{
    for (int i = threadIdx.x; i < (int)(kOpHeaderBytes / 16); i += blockDim.x)
        reinterpret_cast<int4*>(ws)[i] = int4{0, 0, 0, 0};
}

__global__ void __launch_bounds__(kOpThreads) __attribute__((amdgpu_waves_per_eu(4)))
    onepass_kernel(OnepassArgs a)
{
    using V = Vec<float>::type;
    constexpr int S = kOpSlices, R = kOpRingSlots, UL = 256 / S;
    static_assert(S == 8 && kOpRegs == 2 * S, "slice s is registers s and 8 + s");
    extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
    V* const L = reinterpret_cast<V*>(lds_raw);
    __shared__ int sh_min[2][2];   // cached minima of the progress words, by parity
    __shared__ int sh_next, sh_broken, sh_xcd, sh_rank;
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    int* const err = reinterpret_cast<int*>(a.ws + kOpErrOff);
    // The workgroup's XCD and CU, from the hardware (the dispatcher deals
    // workgroups to the XCDs in turn, but not always starting from the
    // first one, e.g. in graph replays).  The two workgroups of a CU join
    // different groups (the first to arrive group 0), and take member
    // ranks in their group by arrival, so every group spans 32 CUs.
    if (t == 0) {
        const int x = xcc_id();
        int hw;
        asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));
        const int cu = (hw >> 8) & 0xff;   // CU, shader array and engine of the XCD
        int grp = -1, r = -1;
        if (x < kOpXcds)
            grp = __hip_atomic_fetch_add(reinterpret_cast<int*>(a.ws + kOpCuOff) + 256 * x + cu, 1,
                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (grp >= 0 && grp < kOpGroupsPerXcd)
            r = __hip_atomic_fetch_add(reinterpret_cast<int*>(a.ws + kOpMemberOff) +
                                           kOpGroupsPerXcd * x + grp,
                                       1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (r < 0 || r >= kOpMembers) {
            atomicOr(err, kOpErrPlacement);
            r = -1;
        }
        sh_xcd = x;
        sh_rank = r < 0 ? -1 : grp * kOpMembers + r;
    }
    __syncthreads();
    if (sh_rank < 0)
        return;   // uniform across the workgroup
    const int xcd = sh_xcd, rank = sh_rank;
    const int gi = rank / kOpMembers, m = rank % kOpMembers;
    const int g = gi * kOpXcds + xcd;
    int* const queue = reinterpret_cast<int*>(a.ws + kOpQueueOff);
    unsigned long long* const nxt = reinterpret_cast<unsigned long long*>(a.ws + kOpNextOff) + 2 * g;
    int* const prog = reinterpret_cast<int*>(a.ws + kOpFlagOff) + 64 * g;
    const __amdgpu_buffer_rsrc_t ring =
        op_rsrc(a.ws + kOpHeaderBytes + (size_t)g * R * kOpSlotBytes);
    if (t == 0) {
        sh_min[0][0] = sh_min[0][1] = sh_min[1][0] = sh_min[1][1] = 0;
        sh_broken = 0;
    }
    __syncthreads();
    const int ul = lane & 31, lh = lane >> 5;
    // Thread parts of the byte offsets (the register parts are constants).
    const uint32_t ld_v = ((uint32_t)m * kOpRowF4 + ul + (wv << 5) + (lh << 8)) * 16;
    const uint32_t xw_v = ((uint32_t)((lh | (wv << 1)) * 32 + m) * UL + ul) * 16;
    const uint32_t xr_v = ((uint32_t)(m * 32 + (lh | (wv << 1))) * UL + ul) * 16;
    const uint32_t st_v = ((uint32_t)lh * kOpRowF4 + m * 256 + (wv << 5) + ul) * 16;
    float cs = a.scale;
    if (__popc((unsigned)lane & dpp_sign_lanes(0, 6)) & 1)
        cs = -cs;

    // Wave 0 waits until every member has written >= need_w slices and read
    // >= need_r; the decision to call this is the same in every wave.
    auto wait_flags = [&](int need_w, int need_r) {
        __syncthreads();
        if (t < 64 && !sh_broken) {
            bool ok = false;
            for (int i = 0; i < kOpSpin; ++i) {
                const int v = __hip_atomic_load(prog + lane, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
                if (__ballot(v < (lane < 32 ? need_w : need_r)) == 0) {
                    ok = true;
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
            if (t == 0 && !ok) {
                sh_broken = 1;
                atomicOr(err, kOpErrTimeout);
            }
        }
        __syncthreads();
    };

    const int cx = (a.ncomp - xcd + kOpXcds - 1) / kOpXcds;   // components c = xcd + 8 i
    int q = 0;                                                // slices so far
    int seq = 0;                                              // components so far
    V x[kOpRegs];
    for (int i = gi; i < cx;) {
        const int c = xcd + kOpXcds * i;
        float* const base = a.im ? ((c & 1) ? a.im : a.re) + ((size_t)(c >> 1) << kOpN)
                                 : a.re + ((size_t)c << kOpN);
        const __amdgpu_buffer_rsrc_t comp = op_rsrc(base);
#pragma unroll
        for (int j = 0; j < kOpRegs; ++j)
            x[j] = op_load<kOpNt>(comp, ld_v, (((j & 7) << 9) | ((j >> 3) << 12)) * 16);
        if (m == 0 && t == 0) {
            const int nx = __hip_atomic_fetch_add(queue + xcd, 1, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT) + kOpGroupsPerXcd;
            __hip_atomic_store(nxt + ((seq + 1) & 1),
                               ((unsigned long long)(seq + 1) << 32) | (unsigned)nx,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        op_pin(x);
        // Row factor H_15: in-vector bits 0-1, register bits 11-14, lane bits
        // 2-6 and 10, then the exchange to L1 and register bits 7-9.
#pragma unroll
        for (int j = 0; j < kOpRegs; ++j)
            in_vector(x[j]);
        register_stages<4, kOpRegs>(x);
        LaneStages<0, 6, 0, kOpRegs, V, float, false>::run(x, lane);
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            __syncthreads();
#pragma unroll
            for (int r = 0; r < 8; ++r)
                L[ul | (wv << 5) | (lh << 8) | (r << 9)] = x[(p << 3) | r];
            __syncthreads();
#pragma unroll
            for (int s = 0; s < 8; ++s)
                x[(p << 3) | s] = L[ul | (s << 5) | (lh << 8) | (wv << 9)];
        }
        register_stages<3, kOpRegs>(x);
        op_pin(x);
        // The ring exchange: iteration s stores slice s and loads slice s - 1.
#pragma unroll
        for (int s = 0; s <= S; ++s) {
            const int qw = q + s, qr = q + s - 1;
            const int need_w = s >= 1 ? qr + 1 : 0;
            const int need_r = s < S ? qw - R + 1 : 0;
            const int cb = qw & 1;
            if (!(sh_min[cb][0] >= need_w && sh_min[cb][1] >= need_r))
                wait_flags(need_w, need_r);
            if (s < S) {
                const uint32_t so = (uint32_t)(qw % R) * (uint32_t)kOpSlotBytes;
                op_store<0>(ring, xw_v, so, x[s]);
                op_store<0>(ring, xw_v, so + 16u * 16 * 32 * UL, x[8 + s]);
            }
            if (s >= 1) {
                const uint32_t so = (uint32_t)(qr % R) * (uint32_t)kOpSlotBytes;
                x[s - 1] = op_load<kOpDevice>(ring, xr_v, so);
                x[8 + s - 1] = op_load<kOpDevice>(ring, xr_v, so + 16u * 16 * UL);
            }
            int pv = 0;
            if (t < 64)
                pv = __hip_atomic_load(prog + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            if (t < 64) {
                for (int o = 16; o >= 1; o >>= 1)
                    pv = min(pv, __shfl_xor(pv, o));
                const int mw = __shfl(pv, 0), mr = __shfl(pv, 32);
                if (t == 0) {
                    sh_min[cb ^ 1][0] = mw;
                    sh_min[cb ^ 1][1] = mr;
                }
            }
            __syncthreads();
            if (t == 0) {
                if (s < S)
                    __hip_atomic_store(prog + m, qw + 1, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_WORKGROUP);
                if (s >= 1)
                    __hip_atomic_store(prog + 32 + m, qr + 1, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_WORKGROUP);
            }
        }
        q += S;
        op_pin(x);
        // Column factor H_5: row bit 4 in registers, row bit 0 on lane 5,
        // then the exchange to R1 and row bits 1-3 in registers.
#pragma unroll
        for (int j = 0; j < 8; ++j)
            butterfly(x[j], x[j | 8]);
        lane_stage<5, kOpRegs, V, float>(x, lane);
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            __syncthreads();
#pragma unroll
            for (int s = 0; s < 8; ++s)
                L[ul | (s << 5) | (lh << 8) | (wv << 9)] = x[(p << 3) | s];
            __syncthreads();
#pragma unroll
            for (int k = 0; k < 8; ++k)
                x[(p << 3) | k] = L[ul | (wv << 5) | (lh << 8) | (k << 9)];
        }
        register_stages<3, kOpRegs>(x);
#pragma unroll
        for (int j = 0; j < kOpRegs; ++j)
            x[j] *= cs;
#pragma unroll
        for (int j = 0; j < kOpRegs; ++j)
            op_store<kOpNt>(comp, st_v, ((((j & 7) << 1) | ((j >> 3) << 4)) * kOpRowF4) * 16, x[j]);
        // The group's next component.
        if (t == 0) {
            unsigned long long v = 0;
            for (int k = 0; k < kOpSpin; ++k) {
                v = __hip_atomic_load(nxt + ((seq + 1) & 1), __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
                if ((int)(v >> 32) == seq + 1)
                    break;
                __builtin_amdgcn_s_sleep(1);
            }
            if ((int)(v >> 32) != seq + 1) {
                atomicOr(err, kOpErrQueue);
                v = 0x7fffffffu;
            }
            sh_next = (int)(unsigned)v;
        }
        __syncthreads();
        i = sh_next;
        ++seq;
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

hipError_t onepass_occupancy(int* blocks_per_cu)
{
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&onepass_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)kOpLdsBytes);
    if (e != hipSuccess)
        return e;
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(
        blocks_per_cu, reinterpret_cast<const void*>(&onepass_kernel), kOpThreads, kOpLdsBytes);
}

hipError_t launch_onepass(float* re, float* im, int ncomp, void* ws, float scale,
                          hipStream_t stream, hipEvent_t start, hipEvent_t stop)
{
    unsigned char* const w = reinterpret_cast<unsigned char*>(ws);
    hipLaunchKernelGGL(onepass_reset_kernel, dim3(1), dim3(kOpThreads), 0, stream, w);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    OnepassArgs a{re, im, w, ncomp, scale};
    void* kargs[] = {&a};
    const dim3 grid(kOpGroups * kOpMembers, 1, 1);
    if (start || stop)
        return hipExtLaunchKernel(reinterpret_cast<const void*>(&onepass_kernel), grid,
                                  dim3(kOpThreads, 1, 1), kargs, kOpLdsBytes, stream, start, stop,
                                  0);
    return hipLaunchKernel(reinterpret_cast<const void*>(&onepass_kernel), grid,
                           dim3(kOpThreads, 1, 1), kargs, kOpLdsBytes, stream);
}

}  // namespace qse
