// Internal interface between the planner (fwt_api.cpp) and the gfx950
// kernels (fwt_kernels.hip).  Not installed; not part of the C ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace qse {

// Runtime description of one tile pass.  A pass transforms the index bits
// [lo, lo + k) of every real vector.  It views the vector as
// [outer][2^k rows][2^lo columns] and processes tiles of all 2^k rows by
// G = 2^gbits 16-byte column groups.  A row pass (lo = 0) instead views its
// 2^k contiguous elements as 2^(k - vb) rows of one 16-byte vector
// (vb = log2 of elements per vector) and also transforms the vb bits
// inside each vector.
struct TileArgs {
    int64_t tiles;       // tiles per component (real or imaginary buffer)
    int64_t wg_count;    // workgroups needed: ceil(tiles / tiles per workgroup)
    int64_t tile0;       // first tile of this launch (set by the launcher)
    int64_t grid;        // persistent kernels: workgroups per component
    int lo;              // log2 of the element stride between rows (col passes)
    int nblk_bits;       // log2 of column blocks per outer index (col passes)
    int tpw_bits;        // log2 of tiles per workgroup
    int tt_bits;         // log2 of threads per tile
    int xcd_bits;        // >= 0: the 2^xcd_bits workgroups of each vector
                         // component share an XCD (xcd_group); -1: launch order
    int do_scale;        // multiply by `scale` before the final store
    int ld_nt;           // nontemporal loads (input not reused by this call)
    int st_policy;       // cache policy of the stores (StorePolicy)
    double scale;        // 2^(-n/2) rounded to the element type
};

// Cache policy of a pass's stores.
enum StorePolicy : int {
    kStorePlain = 0,          // write-back L2: the next launch may hit it
    kStoreNontemporal = 1,    // streaming: this call does not read it again
    kStoreWriteThrough = 2,   // device-scope stores (sc1): intermediate
                              // results of states of 256 MiB and more
};

// Kernel variant: element type, row bits KR, register-round bits EB,
// column-group bits GB, exchange-phase bits PHB, and whether it is a row
// (contiguous) pass.
struct KernelKey {
    int f64;   // 0: float, 1: double
    int kr;    // log2 rows per tile
    int eb;    // log2 16-byte vectors per thread per round
    int gb;    // log2 16-byte column groups per tile (0 for row passes)
    int phb;   // log2 of the phases an LDS exchange is split into
    int row;   // 1: contiguous row pass
    int pipe;  // 1: persistent software-pipelined kernel
    int wave;  // 1: wave-tile kernel (whole tile in one wave, lane stages);
               // 2: lane-exchange row kernel (lane stages, one LDS exchange)
};

// Number of register rounds of a (kr, eb) kernel: ceil(kr / eb), at least 1.
__host__ __device__ constexpr int rounds_of(int kr, int eb)
{
    return kr <= eb ? 1 : 1 + (kr - eb + eb - 1) / eb;
}

// Whether a (kr, eb, gb) tile kernel stores from its load layout after one
// more LDS exchange: when the last round's layout gives runs of consecutive
// lanes shorter than 128 bytes and the load layout gives longer ones.  The
// run of the layout whose register bits start at row bit a is 16 * 2^(gb+a)
// bytes.
__host__ __device__ constexpr bool store_back(int kr, int eb, int gb)
{
    return rounds_of(kr, eb) > 1 &&
           (16 << (gb + (kr - eb * rounds_of(kr, eb) > 0 ? kr - eb * rounds_of(kr, eb) : 0))) <
               128 &&
           (16 << (gb + kr - eb)) >
               (16 << (gb + (kr - eb * rounds_of(kr, eb) > 0 ? kr - eb * rounds_of(kr, eb) : 0)));
}

// The tile group of workgroup w of a launch of wg workgroups.  The
// dispatcher hands consecutive workgroups to the eight XCDs in turn
// (workgroup w on XCD w mod 8).  With xb >= 0 the 2^xb workgroups of
// vector component v are the ones with w mod 8 = v mod 8, so every pass of
// a call, and every call, runs v on the same XCD and finds in its L2 what
// the previous launch wrote there.  That covers the largest multiple of
// 2^(xb + 3) workgroups; the rest keep the launch order.  A bijection of
// [0, wg); xb < 0 keeps the launch order throughout.
__host__ __device__ constexpr int64_t xcd_group(int64_t w, int xb, int64_t wg)
{
    return (xb < 0 || w >= (wg & ~(((int64_t)8 << xb) - 1)))
               ? w
               : ((((w & 7) + (((w >> 3) >> xb) << 3)) << xb) |
                  ((w >> 3) & (((int64_t)1 << xb) - 1)));
}

// True if the variant is compiled into this library.
bool kernel_available(const KernelKey& key);

// Sets the dynamic-LDS limit of every compiled variant on the current
// device.  Returns hipSuccess or the first error.
hipError_t kernels_init_device();

// Enqueue one tile pass.  `re` and `im` (im may be null) are device
// pointers; ncomp = 1 or 2.  start/stop (may be null) are recorded by the
// dispatch itself at the kernel's start and end.
hipError_t launch_tile_pass(const KernelKey& key, void* re, void* im, int ncomp,
                            const TileArgs& args, unsigned block, size_t lds_bytes,
                            hipStream_t stream, hipEvent_t start, hipEvent_t stop);

// Enqueue the two-element transform used for fp32 vectors of 2 elements
// (n = 1): pairs (a, b) -> (a + b, a - b) * scale.
hipError_t launch_pair_f32(float* re, float* im, int64_t pairs, int do_scale,
                           float scale, hipStream_t stream, hipEvent_t start, hipEvent_t stop);

// Enqueue a 16-byte streaming copy of `bytes` (a multiple of 16).
hipError_t launch_stream_copy(void* dst, const void* src, int64_t bytes,
                              hipStream_t stream);

// Ablations (fwt_ablation.hip): the pages' own designs for the transform.
hipError_t ablation_stagewise(int f64, void* re, void* im, int64_t batch, int n, int normalize,
                              double c, hipStream_t stream);
hipError_t ablation_popc_gemm(int f64, void* re, void* im, void* ws_re, void* ws_im,
                              int64_t batch, int n, int normalize, double c, hipStream_t stream);
// ---- INT8 / CRT (Ozaki) ablation, fp64 (fwt_ozaki.hip) ----
constexpr int kOzMaxModuli = 16;
constexpr int kOzScaleBits = 48;     // |X| <= 2^48 after scaling
constexpr int kOzRowTileBits = 12;   // residue words per row-pass tile
constexpr int kOzPack = 4;           // moduli per 32-bit residue word
constexpr int kOzMinN = 5;
constexpr int kOzMaxN = 28;
// The 16 largest primes below 256: balanced residues fit int8.
constexpr int kOzPrimes[kOzMaxModuli] = {251, 241, 239, 233, 229, 227, 223, 211,
                                         199, 197, 193, 191, 181, 179, 173, 167};
struct OzConst {
    int m;                          // moduli in use
    int p[kOzMaxModuli];
    double inv_pd[kOzMaxModuli];
    int magic[kOzMaxModuli];        // round(2^20 / p_j), for reduce_mod
    int crt_c[kOzMaxModuli];        // (M / p_j)^-1 mod p_j
    uint64_t crt_lo[kOzMaxModuli];  // M / p_j, low and high 64 bits
    uint64_t crt_hi[kOzMaxModuli];
    uint64_t m_lo, m_hi;            // M = prod of the m moduli
};
// A Kronecker pass over the residue words: row (bits [0, kt), xb line
// bits per tile) or column (bits [lo, lo + kt), 2^xb-word row segments).
struct OzPass {
    int row, lo, kt, xb;
};
int oz_num_moduli(int n);
void oz_pass_plan(int n, OzPass* passes, int* npasses);
// Workspace bytes for `comps` components; offsets of the partial maxima
// and the exponents inside it (the residue words start at 0).
size_t oz_workspace_layout(int64_t batch, int n, int comps, size_t* off_partial,
                           size_t* off_exps);
hipError_t ablation_ozaki(double* re, double* im, int64_t batch, int n, double c, void* ws,
                          hipStream_t stream);

// Matrix-core block products on both Kronecker factors with a transposed
// staging buffer in between (n1 = n / 2, n2 = n - n1, each 8..15 for fp32,
// 8..14 for fp64); ws_re / ws_im hold batch * 2^n elements each.
hipError_t ablation_mfma_transpose(int f64, void* re, void* im, void* ws_re, void* ws_im,
                                   int64_t batch, int n, int normalize, double c,
                                   hipStream_t stream);

// Matrix-core row pass over the km contiguous low bits (8 <= km <= 15
// for fp32, 14 for fp64).
hipError_t ablation_mfma_row(int f64, void* re, void* im, int64_t batch, int n, int km,
                             int do_scale, double c, hipStream_t stream);

// Ablation dispatch shared by fwt_ablation_execute (caller workspace) and
// fwt_ablation_execute_static (the library's static scratch; ws_owned =
// true skips the allocation-range check of the workspace).  dtype is an
// fwt_dtype value; returns an FWT_* status.
int ablation_run(int kind, int64_t batch, int n, int dtype, void* re, void* im, int normalize,
                 void* ws, size_t ws_bytes, bool ws_owned, hipStream_t stream);
// The argument checks of ablation_run for a call on the library's own
// scratch (everything but the workspace); returns an FWT_* status.
int ablation_validate(int kind, int64_t batch, int n, int dtype, const void* re, const void* im);
// Records `e` as the calling thread's last HIP error (fwt_last_hip_error)
// and returns FWT_EHIP.
int hip_status(hipError_t e);
// Workspace bytes ablation `kind` needs (0 if none).
size_t ablation_workspace_size(int kind, int64_t batch, int n, int dtype, int with_im);

// ---- One-pass transform of fp32 n = 20 states (fwt_kernels.hip) ----
// Each vector component (2^20 floats, 4 MiB) is transformed by one group
// of 32 workgroups on one XCD, one workgroup per CU, with the state read
// from and written to HBM once.  Each workgroup holds a 2^15-element row
// block in registers and applies the factor on the 15 low bits; the group
// then exchanges the blocks through a ring in its XCD's L2 (kOpSlices
// slices, kOpRingSlots slots) and each workgroup applies the factor on the
// 5 high bits to its 2^10-column slice.  Two groups share each XCD and take
// components from a per-XCD queue.  The caller's workspace holds the ring
// and the synchronisation words; the first 32-bit word collects error bits
// (kOpErr*) of the call.
constexpr int kOpN = 20;
constexpr int kOpXcds = 8;
constexpr int kOpMembers = 32;          // workgroups per group (CUs per XCD)
constexpr int kOpGroupsPerXcd = 2;
constexpr int kOpGroups = kOpXcds * kOpGroupsPerXcd;
constexpr int kOpThreads = 512;
constexpr int kOpSlices = 8;
constexpr int kOpRingSlots = 2;
constexpr int kOpLag = 1;                // slices between a slice's store and its load
constexpr size_t kOpSlotBytes = ((size_t)4 << 20) / kOpSlices;   // one slice of a component
constexpr size_t kOpErrOff = 0;          // int: error bits
constexpr size_t kOpQueueOff = 256;      // int[kOpXcds]: components taken per XCD
constexpr size_t kOpMemberOff = 384;     // int[kOpXcds][kOpGroupsPerXcd]: members that joined
constexpr size_t kOpNextOff = 512;       // uint64[kOpGroups][2]: (sequence << 32) | next index
constexpr size_t kOpFlagOff = 1024;      // int[kOpGroups][64]: slices written, slices read
constexpr size_t kOpCuOff = 8192;        // int[kOpXcds][256]: workgroups seen per CU
constexpr size_t kOpHeaderBytes = 16384; // the words above, cleared by each call
constexpr size_t kOpWorkspaceBytes =
    kOpHeaderBytes + (size_t)kOpGroups * kOpRingSlots * kOpSlotBytes;
constexpr size_t kOpLdsBytes = 64 * 1024;
enum : int {
    kOpErrTimeout = 1,     // a wait for the group's progress words ran out
    kOpErrPlacement = 2,   // a CU or an XCD received more workgroups than planned
    kOpErrQueue = 4,       // a wait for the next component's index ran out
};
// Workgroups of the one-pass kernel that fit one CU at once (0 if it cannot
// run on the current device).
hipError_t onepass_occupancy(int* blocks_per_cu);
// Enqueue a call: clear the workspace header, then the transform of
// `ncomp` components (re: components 0, 2, 4, ... when im is given, else
// 0, 1, 2, ...).  start/stop (may be null) are recorded at the transform
// kernel's start and end by the dispatch itself.
hipError_t launch_onepass(float* re, float* im, int ncomp, void* ws, float scale,
                          hipStream_t stream, hipEvent_t start, hipEvent_t stop);

}  // namespace qse
