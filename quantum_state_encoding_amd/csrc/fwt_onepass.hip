// One HBM pass for the fp32 n = 20 transform: groups of workgroups on one
// XCD exchange the Kronecker factors' intermediate through the XCD's L2.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "fwt_device.h"
#include "fwt_internal.h"

namespace qse {
namespace {

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
//  column:   slice s as read from the ring: registers s and 8 + s hold
//            source rows (l >> 2) and 16 + (l >> 2), columns (l & 3) |
//            w << 2 of the slice (element bits 2-6).  The five source bits
//            are lane bits 2-5 and one register bit, so the column factor
//            runs on the slice's two registers alone, inside the ring loop,
//            and the slice goes to HBM while the next slice is exchanged.
// The fp32 DPP lane stages leave a sign on some lanes: the row stages on
// lane bits 0-3 by element bits 2-5 (in the column layout lane bits 0-1
// and wave bits 0-1), the column stages on lane bits 2-3 by those lanes;
// the scale removes both.
//
// The ring exchange, per slice s (8 per component, 512 KiB each, ring of 2
// slots per group): each workgroup stores its registers of slice s (the
// values for all 32 destinations), loads slice s - 1 as written by every
// member, applies the column factor to slice s - 2 and stores it to HBM,
// waits for everything but those HBM stores with one s_waitcnt, and
// publishes "slices written" and "slices read" in its two progress words
// (plain stores: they land in the XCD's L2).  A slot holds float4 (destination d, source r, column u)
// at ((d * 8 + u / 4) * 32 + r) * 4 + u % 4, so a reader's wave loads
// 1 KiB in one piece.  The ring's size is set by the L2: two groups'
// rings of 2 x 512 KiB share an XCD's 4 MB with the HBM streams; a third
// slot (loads two slices behind the stores, so their progress words are
// usually published before they are polled) made every ring round trip
// about three times slower and the call 21 % slower.  Before storing into
// a slot a workgroup needs every member to have read the slice that last
// used it; before loading a slice, every member to have written it.  Wave
// 0 reads the group's 64 progress words with device-scope loads (sc1:
// they miss the CU's L1 and hit the L2; a device-scope atomic would leave
// the L2 and take about 1.2 us here) in the same round trip as the
// slice's data, so a wait costs a round trip only when a member is behind.
// The slice loads are device-scope too: a plain load can return a line the
// CU's L1 kept from the slot's previous use.  Every member of a group runs
// on the same XCD: a workgroup reads its XCD and CU from the XCC_ID and
// HW_ID registers and joins a group with two atomic adds (the dispatcher
// deals the 512 workgroups to the 8 XCDs in turn, 64 each, two per CU, but
// the first XCD it serves varies), so one L2 serves the group, and the two
// workgroups of a CU belong to different groups (two members of one group
// on one CU would halve that pair's share of the CU, and the whole group
// waits for them).  All 2 x 256 workgroups are resident together (at most
// 128 VGPRs and 64 KiB of LDS each), so every wait ends; the spin bounds
// are only a guard, recorded in the workspace's error word.
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
    constexpr int S = kOpSlices, R = kOpRingSlots, LAG = kOpLag, UL = 256 / S;
    static_assert(LAG >= 1 && R > LAG, "a slot is rewritten only after its slice was read");
    static_assert(S == 8 && kOpRegs == 2 * S, "slice s is registers s and 8 + s");
    extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
    V* const L = reinterpret_cast<V*>(lds_raw);
    __shared__ int sh_ok[2];   // the last poll met the next iteration's needs, by parity
    __shared__ int sh_next, sh_spec, sh_broken, sh_xcd, sh_rank;
    // The logical lane: mirrored_lane order makes lane bit 2 a DPP stage.
    const int t = threadIdx.x, lane = mirrored_lane(t & 63), wv = t >> 6;
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
        sh_ok[0] = 1;   // the first iteration needs nothing
        sh_ok[1] = 0;
        sh_broken = 0;
    }
    __syncthreads();
    const int ul = lane & 31, lh = lane >> 5;
    // Thread parts of the byte offsets (the register parts are constants).
    const uint32_t ld_v = ((uint32_t)m * kOpRowF4 + ul + (wv << 5) + (lh << 8)) * 16;
    // Ring slot layout: float4 (destination d, source r, column u of the
    // slice) at ((d * 8 + u / 4) * 32 + r) * 4 + u % 4, so that a reader's
    // wave loads 1 KiB in one piece (lanes 0-1 = u % 4, lanes 2-5 = r % 16).
    const uint32_t xw_v =
        ((uint32_t)(((lh | (wv << 1)) * 8 + (ul >> 2)) * 32 + m) * 4 + (ul & 3)) * 16;
    const uint32_t xr_v = ((uint32_t)((m * 8 + wv) * 32 + (lane >> 2)) * 4 + (lane & 3)) * 16;
    // Column output: source row lane >> 2 (+ 16), column u = (lane & 3) |
    // wv << 2 of the slice, in member m's 1024-column slice.
    const uint32_t st_v =
        ((uint32_t)(lane >> 2) * kOpRowF4 + m * 256 + (wv << 2) + (lane & 3)) * 16;
    // The scale times the signs of the fp32 DPP lane stages: the row stages
    // on lane bits 0-3 left them by element bits 2-5, now lane bits 0-1 and
    // wave bits 0-1; the column stages on lane bits 2-3 leave them by
    // those lanes.
    float cs = a.scale;
    if ((__popc((unsigned)lane & 15u) + __popc((unsigned)wv & 3u)) & 1)
        cs = -cs;

    // Wave 0 waits until every member has written >= need_w slices and read
    // >= need_r; the decision to call this is the same in every wave.  The
    // iteration's closing barrier already ordered every wave before it, and
    // only wave 0 touches the words it reads, so it starts at once.  Each
    // poll waits for its own load's round trip through the L2 (about a
    // microsecond), which paces the loop without a sleep and bounds the
    // whole wait to about a second.
    auto wait_flags = [&](int need_w, int need_r) {
        if (t < 64 && !sh_broken) {
            bool ok = false;
            for (int i = 0; i < kOpSpin; ++i) {
                const int v = __hip_atomic_load(prog + lane, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
                if (__ballot(v < (lane < 32 ? need_w : need_r)) == 0) {
                    ok = true;
                    break;
                }
            }
            if (t == 0 && !ok) {
                sh_broken = 1;
                atomicOr(err, kOpErrTimeout);
            }
        }
        __syncthreads();
    };

    unsigned long long spec_next = 0;                          // thread 0 only
    const int cx = (a.ncomp - xcd + kOpXcds - 1) / kOpXcds;   // components c = xcd + 8 i
    int q = 0;                                                // slices so far
    int seq = 0;                                              // components so far
    V x[kOpRegs];
    auto comp_rsrc = [&](int i) {
        const int c = xcd + kOpXcds * i;
        return op_rsrc(a.im ? ((c & 1) ? a.im : a.re) + ((size_t)(c >> 1) << kOpN)
                            : a.re + ((size_t)c << kOpN));
    };
    auto load_offset = [](int j) -> uint32_t {
        return (uint32_t)((((j & 7) << 9) | ((j >> 3) << 12)) * 16);
    };
    __amdgpu_buffer_rsrc_t comp = comp_rsrc(gi);
    bool loaded = false;   // the component's loads were issued with the last stores
    // Column factor H_5 on slice k as loaded from the ring: registers k and
    // 8 + k hold source rows (lane >> 2) and 16 + (lane >> 2), columns
    // (lane & 3) | wv << 2 of the slice: the source bits are register bit 3
    // and lane bits 2-5, so the whole factor runs in registers and lanes.
    auto column_factor = [&](int k, V (&y)[2]) {
        y[0] = x[k];
        y[1] = x[8 + k];
        butterfly(y[0], y[1]);
        lane_stage<2, 2, V, float, true>(y, lane);
        lane_stage<3, 2, V, float, true>(y, lane);
        lane_stage<4, 2, V, float, true>(y, lane);
        lane_stage<5, 2, V, float, true>(y, lane);
        y[0] *= cs;
        y[1] *= cs;
    };
    auto column_store = [&](__amdgpu_buffer_rsrc_t dst, int k, const V (&y)[2]) {
        op_store<kOpNt>(dst, st_v, (uint32_t)(k * UL) * 16, y[0]);
        op_store<kOpNt>(dst, st_v, (uint32_t)(16 * kOpRowF4 + k * UL) * 16, y[1]);
    };
    auto column_slice = [&](int k) {
        V y[2];
        column_factor(k, y);
        column_store(comp, k, y);
    };
    for (int i = gi; i < cx;) {
        if (!loaded) {     // uniform across the workgroup
            comp = comp_rsrc(i);
#pragma unroll
            for (int j = 0; j < kOpRegs; ++j)
                x[j] = op_load<kOpNt>(comp, ld_v, load_offset(j));
        }
        loaded = false;
        if (m == 0 && t == 0) {
            const int nx = __hip_atomic_fetch_add(queue + xcd, 1, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT) + kOpGroupsPerXcd;
            __hip_atomic_store(nxt + ((seq + 1) & 1),
                               ((unsigned long long)(seq + 1) << 32) | (unsigned)nx,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        op_pin(x);
        // Wave priority: the row factor runs at the lowest level, the ring
        // exchange and everything up to the next row factor at a higher
        // one.  The two workgroups of a CU belong to different groups, and
        // a group's ring moves at the pace of its slowest member, so a CU
        // serves the exchange first and fits the row factor around it.
        __builtin_amdgcn_s_setprio(0);
        // Row factor H_15: in-vector bits 0-1, register bits 11-14, lane bits
        // 2-6 and 10, then the exchange to L1 and register bits 7-9.
#pragma unroll
        for (int j = 0; j < kOpRegs; ++j)
            in_vector(x[j]);
        register_stages<4, kOpRegs>(x);
        LaneStages<0, 6, 0, kOpRegs, V, float, true>::run(x, lane);
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
        // The ring exchange: iteration s stores slice s, loads slice s - LAG,
        // and applies the column factor to slice s - LAG - 1 (loaded in the
        // previous iteration) and stores it to HBM, while the slice loads
        // and stores of this iteration are in flight.
        static_assert(LAG == 1, "column work trails the loads by one iteration");
        static_assert((S + LAG) % 2 == 1, "the flag's buffer parity counts components");
        __builtin_amdgcn_s_setprio(2);   // until the next component's row factor
#pragma unroll
        for (int s = 0; s < S + LAG; ++s) {
            const int qw = q + s, qr = q + s - LAG;
            const int need_w = s >= LAG ? qr + 1 : 0;
            const int need_r = s < S ? qw - R + 1 : 0;
            // What the next iteration will need (the next component's first
            // iteration after the last one).
            const int next_w = s + 1 >= S + LAG ? 0 : s + 1 >= LAG ? qr + 2 : 0;
            const int next_r = s + 1 >= S + LAG ? q + S - R + 1 : s + 1 < S ? qw - R + 2 : 0;
            // Iterations alternate the flag's buffer; a component has an odd
            // number of them, so the parity includes the component count.
            const int cb = (s + seq) & 1;
            if (!sh_ok[cb])
                wait_flags(need_w, need_r);
            if (s < S) {
                const uint32_t so = (uint32_t)(qw % R) * (uint32_t)kOpSlotBytes;
                op_store<0>(ring, xw_v, so, x[s]);
                op_store<0>(ring, xw_v, so + 16u * 16 * 8 * 32 * 4, x[8 + s]);
            }
            if (s >= LAG) {
                const uint32_t so = (uint32_t)(qr % R) * (uint32_t)kOpSlotBytes;
                x[s - LAG] = op_load<kOpDevice>(ring, xr_v, so);
                x[8 + s - LAG] = op_load<kOpDevice>(ring, xr_v, so + 16u * 16 * 4);
            }
            int pv = 0;
            if (t < 64)
                pv = __hip_atomic_load(prog + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (s == S + LAG - 1 && t == 0)   // the group's next component, published long ago
                spec_next = __hip_atomic_load(nxt + ((seq + 1) & 1), __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
            // The column slice's two HBM stores are issued last and left out
            // of the wait (operations complete in issue order): the next
            // iteration's wait covers them.  The last iteration leaves its
            // slice to the component's tail.
            if (s >= LAG + 1 && s < S + LAG - 1) {
                column_slice(s - LAG - 1);
                asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
            } else {
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            }
            if (t < 64) {
                const bool ok = __ballot(pv < (lane < 32 ? next_w : next_r)) == 0;
                if (t == 0) {
                    sh_ok[cb ^ 1] = ok;
                    if (s == S + LAG - 1)   // read by every thread after the barrier
                        sh_spec = (int)(spec_next >> 32) == seq + 1 ? (int)(unsigned)spec_next
                                                                    : -1;
                }
            }
            __syncthreads();
            if (t == 0) {
                if (s < S)
                    __hip_atomic_store(prog + m, qw + 1, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_WORKGROUP);
                if (s >= LAG)
                    __hip_atomic_store(prog + 32 + m, qr + 1, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_WORKGROUP);
            }
        }
        q += S;
        // The last two slices' column factors (the last iteration leaves
        // slice S - 2 here too).  When the next component is known, its
        // loads are issued before these slices' stores: memory operations
        // complete in issue order, so the row factor's wait for the loads
        // does not also wait for the stores' acknowledgement.
        V yprev[2], ylast[2];
        column_factor(S - 2, yprev);
        column_factor(S - 1, ylast);
        const __amdgpu_buffer_rsrc_t done_comp = comp;
        const int spec = sh_spec;
        if (spec >= 0) {
            if (spec < cx) {
                comp = comp_rsrc(spec);
#pragma unroll
                for (int j = 0; j < kOpRegs; ++j)
                    x[j] = op_load<kOpNt>(comp, ld_v, load_offset(j));
                loaded = true;
            }
            column_store(done_comp, S - 2, yprev);
            column_store(done_comp, S - 1, ylast);
            i = spec;
            ++seq;
            continue;
        }
        column_store(done_comp, S - 2, yprev);
        column_store(done_comp, S - 1, ylast);
        // The group's next component.
        if (t == 0) {
            unsigned long long v = spec_next;
            for (int k = 0; k < kOpSpin && (int)(v >> 32) != seq + 1; ++k) {
                __builtin_amdgcn_s_sleep(1);
                v = __hip_atomic_load(nxt + ((seq + 1) & 1), __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
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

}  // namespace

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
