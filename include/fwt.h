/*
 * fwt.h - batched in-place Walsh-Hadamard transform on MI355X (gfx950).
 *
 * Operation.  For every vector b < batch and each of the two planar
 * components (real part re, imaginary part im) independently:
 *
 *     y_k = c * sum_{i=0}^{2^n - 1} (-1)^{popcount(k AND i)} * x_i
 *
 * in natural (Sylvester) order, with c = 1, or c = 2^(-n/2) when
 * `normalize` is non-zero.  The matrix entry is the on-the-fly Walsh
 * coefficient of the Apache Mahout pull request "[QDP] [feature] Pr4
 * kronecker fwt" (section "How"); the transform is the butterfly network
 * of n add/subtract stages at strides 1, 2, 4, ... described in the iThome
 * "Day 18" native-FWT article (section "Tensor Core wants matrix
 * multiplication").  Because the matrix is real, a complex state stored as
 * separate real and imaginary buffers (the planar layout of the pull
 * request's section "How") is two independent real transforms.
 *
 * Execution.  A plan splits the n index bits into passes (the Kronecker
 * factorisation H_n = H_{n1} (x) H_{n2} of the pull request's sections
 * "Why" and "Why submit PR4"; the iThome article's "Kronecker block GEMM
 * idea").  Each pass streams the state through memory once, in place, with
 * no transpose and no temporary buffer.  n <= 15 (fp32) / 14 (fp64) runs
 * as a single pass whose tiles hold a whole vector on chip; up to n = 26
 * (fp32) / 25 (fp64), two passes; above, three.  Large multi-pass calls run
 * in chunks sized to the Infinity Cache: chunks of vectors, or of
 * sub-vector blocks when one vector exceeds it (fwt_plan_call_schedule).
 *
 * Conventions common to every entry point:
 *  - Status codes are the FWT_* values below; no C++ exception crosses
 *    this interface.
 *  - Nothing here allocates device memory; fwt_execute never synchronises.
 *    (The library's code object holds one static array of
 *    FWT_STATIC_SCRATCH_BYTES per device, placed by the runtime when the
 *    library is loaded on that device; only fwt_ablation_execute_static
 *    uses it.)
 *  - Plans hold host metadata only, are immutable after creation, and may
 *    be used concurrently from several host threads and streams.
 */
#ifndef QSE_FWT_H
#define QSE_FWT_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct fwt_plan_s* fwt_plan_t;

/* Element type of both planar buffers. */
typedef enum { FWT_F32 = 0, FWT_F64 = 1 } fwt_dtype;

/* Execution path chosen at plan creation.
 *  AUTO          single pass while a vector fits one tile (n <= 15 for
 *                fp32, n <= 14 for fp64), otherwise multi-pass.
 *  SINGLE_BLOCK  one pass, one vector per tile; FWT_EUNSUPPORTED above the
 *                single-pass limit.
 *  MULTIPASS     Kronecker split into >= 2 passes whenever n allows it
 *                (n >= 4 for fp32, n >= 3 for fp64, where the first factor
 *                still holds a 16-byte vector; below that one pass).
 *  MFMA_ABLATION the pages' matrix-core form, for measurement: AUTO's
 *                split, with the row pass (the low 8..15 bits) done as dense
 *                H_16 block products on the 16x16x4 fp32 / fp64 matrix
 *                instructions (see FWT_ABLATION_MFMA); FWT_EUNSUPPORTED for
 *                n < 8 and where AUTO is. */
typedef enum {
    FWT_PATH_AUTO = 0,
    FWT_PATH_SINGLE_BLOCK = 1,
    FWT_PATH_MULTIPASS = 2,
    FWT_PATH_MFMA_ABLATION = 3
} fwt_path;

enum {
    FWT_OK = 0,
    FWT_EINVAL = -1,       /* bad argument: null, range, n mismatch, overlap */
    FWT_EALIGN = -2,       /* a buffer is not 16-byte aligned */
    FWT_EUNSUPPORTED = -3, /* valid request the library does not implement */
    FWT_EHIP = -4,         /* the HIP runtime reported an error */
    FWT_ENOMEM = -5,       /* host allocation of the plan failed */
    FWT_ESCRATCH = -6      /* fwt_ablation_execute_static: the call needs more
                              workspace than FWT_STATIC_SCRATCH_BYTES */
};

/* Largest supported n (2^30 amplitudes per vector). */
#define FWT_MAX_N 30

/* Create a plan for vectors of 2^n amplitudes of `dtype`.
 *  out    receives the plan (set to NULL on failure); must not be NULL.
 *  n      0 <= n <= FWT_MAX_N; n = 0 is the identity.
 * Returns FWT_OK, FWT_EINVAL (null out, n out of range, unknown dtype or
 * path), FWT_EUNSUPPORTED (SINGLE_BLOCK above its limit, MFMA_ABLATION),
 * FWT_ENOMEM, or FWT_EHIP (the kernels' launch attributes could not be
 * set on the current device). */
int fwt_plan_create(fwt_plan_t* out, int n, fwt_dtype dtype, fwt_path path);

/* Create a plan with an explicit Kronecker split: npasses factors whose
 * bit counts bits[0..npasses-1] sum to n.  bits[0] is the factor on the
 * lowest (contiguous) index bits, bits[1] the next, and so on; so the
 * two-factor split n = n1 + n2 of the pull request's section "How" is
 * {n2, n1}.  Each factor must be within the per-pass limit (15 bits fp32 /
 * 14 bits fp64 for bits[0], 12 bits for the others) and every factor after
 * the first needs at least 2 (fp32) / 1 (fp64) bits below it.
 * Returns FWT_OK, FWT_EINVAL (null pointers, npasses < 1, sum != n, a
 * factor < 1 or out of its limit), FWT_ENOMEM or FWT_EHIP. */
int fwt_plan_create_split(fwt_plan_t* out, int n, fwt_dtype dtype, int npasses,
                          const int* bits);

/* Per-pass tiling overrides for fwt_plan_create_tuned; -1 in a field
 * selects the default. */
typedef struct {
    int eb;      /* log2 of the 16-byte vectors a thread holds per register
                    round (0..5, at most the pass's row bits; LDS tiles with
                    row bits need at least 1) */
    int gbits;   /* log2 of the 16-byte column groups per tile of a column
                    pass (0..4; 0 or -1 for the first pass) */
    int phases;  /* log2 of the phases a column pass splits each LDS exchange
                    into (0..2, at most gbits; column passes of >= 9 bits and
                    >= 8 groups only); for the lane-exchange kernel
                    (wave = 2), 0 or 1, where 1 needs w < eb and halves the
                    tile's LDS */
    int pipe;    /* 1: persistent software-pipelined kernel (tiles of >= 2^11
                    16-byte vectors in workgroups of <= 512 threads); 0: one
                    workgroup per tile group; default: pipelined when one
                    workgroup fills a CU's LDS */
    int wave;    /* 1: wave-tile kernel (a whole tile in one wave, lane bits
                    crossed with DPP / ds_swizzle / permlane swaps, no LDS;
                    row bits - eb <= 6 - gbits); 2: lane-exchange kernel
                    (lanes hold the 6 - gbits lowest row bits and, in a
                    column pass, the gbits column-group bits; a workgroup
                    of 2^(6 + w) threads holds the tile with
                    w = row bits - (6 - gbits) - eb wave bits, 1 <= w <= 4
                    and 2 <= eb <= 5 or eb = w = 1, and ceil(w / eb) LDS
                    exchanges move the wave bits into registers.  Row
                    passes: 8..13 row bits; default eb gives
                    w = min(4, row bits - 8), or 1 below 10 row bits,
                    except eb = 4 with 2 exchange phases for the
                    13-row-bit row pass of a multi-pass plan, and eb = 3
                    for a one-pass plan of 12 row bits on a state of at
                    most 256 MiB (fwt_plan_call_pass_config).  Column
                    passes: 6..11 bits, gbits 3 or 4 (2^(bits + gbits)
                    16-byte slots at most 2^14, and at most 2^13 without
                    phases); default gbits 4 up to 9 bits when a row
                    holds 16 groups, else 3; eb = min(4, row bits -
                    (6 - gbits) - 1), or 5 at 11 bits; 2 phases from
                    2^11 slots when w < eb); 0: LDS tiles.  Default, when
                    every field of the entry is -1: the wave-tile kernel
                    for a one-pass plan with 3 <= n <= 10; else the
                    lane-exchange kernel for a row pass of 8..13 row bits,
                    except the row pass of a multi-pass plan with 11, for
                    a column pass of 8..11 bits whose rows hold at least 8
                    groups, and for a 7-bit column pass whose rows hold at
                    least 16 groups (16 groups, eb = 2); else LDS tiles.  "Row bits" of a row
                    pass counts 16-byte vectors: the pass's bits less 2
                    (fp32) or 1 (fp64); of a column pass, the pass's
                    bits. */
} fwt_pass_tuning;

/* As fwt_plan_create_split, with the on-chip tiling of each pass forced
 * (tuning and testing of kernel variants; the result is the same up to
 * rounding order).  `tuning` holds npasses entries, or is NULL (all
 * defaults).  Returns as fwt_plan_create_split, plus FWT_EINVAL for a value
 * out of range or a tile that exceeds the LDS, lane or workgroup limits,
 * and FWT_EUNSUPPORTED for a variant that is not compiled in. */
int fwt_plan_create_tuned(fwt_plan_t* out, int n, fwt_dtype dtype, int npasses,
                          const int* bits, const fwt_pass_tuning* tuning);

/* Transform in place, asynchronously on `stream` (0 = the null stream;
 * otherwise a stream of the calling thread's current device, else
 * FWT_EINVAL).
 *  re, im   device buffers of batch * 2^n elements of the plan's dtype,
 *           vector b at offset b * 2^n; 16-byte aligned; must not overlap.
 *           im may be NULL (real-only transform).  The caller owns them.
 *  batch    >= 0; 0 is a no-op.
 *  n        must equal the plan's n.
 *  normalize  non-zero multiplies the result by 2^(-n/2) (applied once,
 *           in the last pass; an exact power of two for even n).
 * Validation happens on the host before anything is enqueued: FWT_EINVAL
 * for a NULL plan or re, batch < 0, n mismatch, re == im, overlapping
 * buffers, or a buffer that is not device memory or too small for
 * batch * 2^n elements; FWT_EALIGN for misalignment.  A launch failure
 * returns FWT_EHIP (earlier passes may already be enqueued; the buffers
 * are then undefined).  Faults during execution surface at the caller's
 * next synchronisation of the stream.  The call only enqueues kernel
 * launches (no memsets, no allocation, no synchronisation), so it may be
 * captured into a HIP graph.
 * Cache hints (they change speed, never results): in a multi-pass plan the
 * first pass loads nontemporally; the last pass stores nontemporally when
 * the call's state exceeds 256 MiB (the chunked schedules); earlier passes
 * store with device scope when the state exceeds 32 MiB and their tiles
 * hold at most 2^10 16-byte slots; all other stores are plain. */
int fwt_execute(fwt_plan_t plan, int64_t batch, int n, void* re, void* im,
                int normalize, hipStream_t stream);

/* ---- One HBM pass on a caller's workspace --------------------------------
 * The Kronecker split H_20 = H_5 (x) H_15 (the pull request's sections "Why"
 * and "How"; the iThome article's "Kronecker block GEMM idea") done in a
 * single read and write of the state: each vector component (4 MiB) is
 * transformed by a group of 32 workgroups on one XCD, one per CU, which
 * apply the 15-bit factor to the rows they hold in registers, exchange the
 * rows through a ring buffer that stays in the XCD's 4 MB L2, and apply the
 * 5-bit factor to the columns.  It serves default (FWT_PATH_AUTO) fp32
 * n = 20 plans on a device of 8 XCDs x 32 CUs (MI355X) where two of its
 * workgroups fit one CU; every other call runs fwt_execute's passes.
 *
 * fwt_workspace_size: *bytes = the workspace a call of `plan` on `batch`
 * vectors (with_im != 0: both components) needs for the one-pass kernel
 * (about 16 MiB), or 0 when such a call runs fwt_execute's passes (another
 * plan, batch 0, an unsupported device).  Returns FWT_OK, FWT_EINVAL (null
 * argument, batch < 0) or FWT_EHIP (the device could not be queried).
 *
 * fwt_execute_ws: the transform of fwt_execute, same arguments and
 * validation, with `ws` a device buffer of `ws_bytes` (caller-owned,
 * 256-byte aligned, inside one device allocation, overlapping neither re
 * nor im).  When fwt_workspace_size is 0, `ws` is ignored (it may be NULL)
 * and this is exactly fwt_execute.  Otherwise it enqueues two kernels: one
 * workgroup that clears the workspace's 16 KiB header (a kernel, not a
 * memset, so the call may be captured into a HIP graph), and the
 * transform.  Statuses as fwt_execute, plus FWT_EINVAL for a missing or too
 * small workspace or one that overlaps the state, FWT_EALIGN for a
 * misaligned one.  Results equal fwt_execute's within rounding (bit for
 * bit on small-integer inputs; the sums are associated differently).  Two
 * calls that share a workspace must not run at the same time (each call
 * uses all of it); calls on different workspaces may.  The kernel needs
 * all of its 512 workgroups resident together: a concurrent kernel that
 * holds CUs delays it, and its waits are bounded (about a second), after
 * which it records an error and the result is undefined.
 *
 * fwt_execute_ws_timed: fwt_execute_ws with `start` and `stop` recorded by
 * the dispatch of the transform kernel itself (its duration without launch
 * gaps).  FWT_EINVAL for null events or a call that would not run the
 * one-pass kernel.
 *
 * fwt_workspace_status: *bits = the error bits the last one-pass call on
 * `ws` recorded (0: none; 1: a wait for the group's progress ran out,
 * 2: an XCD received more workgroups than its two groups hold, 4: a wait
 * for the next component's index ran out; any of them means the result is
 * undefined).  Reads device memory synchronously: call it after the
 * stream that ran the call has been synchronised.  Returns FWT_OK,
 * FWT_EINVAL (null argument) or FWT_EHIP. */
int fwt_workspace_size(fwt_plan_t plan, int64_t batch, int with_im, size_t* bytes);
int fwt_execute_ws(fwt_plan_t plan, int64_t batch, int n, void* re, void* im, int normalize,
                   void* ws, size_t ws_bytes, hipStream_t stream);
int fwt_execute_ws_timed(fwt_plan_t plan, int64_t batch, int n, void* re, void* im,
                         int normalize, void* ws, size_t ws_bytes, hipStream_t stream,
                         hipEvent_t start, hipEvent_t stop);
int fwt_workspace_status(const void* ws, int* bits);

/* Vectors per chunk that fwt_execute uses for a call on `batch` vectors
 * (with_im != 0: both components): a multi-pass call whose state exceeds
 * the 256 MiB Infinity Cache runs every pass on one chunk of vectors before
 * the next chunk, so later passes re-read what earlier passes left in the
 * cache.  fwt_execute is then exactly, for each chunk in order,
 * fwt_execute_pass for passes 0..P-1 on that chunk.  *out = 0 means no
 * chunking by whole vectors: none at all, or the chunks of blocks smaller
 * than a vector that fwt_plan_call_schedule describes.  Returns FWT_OK or
 * FWT_EINVAL (null argument, batch < 0). */
int fwt_plan_chunk_vectors(fwt_plan_t plan, int64_t batch, int with_im, int64_t* out);

/* The whole chunk schedule of an fwt_execute call on `batch` vectors
 * (with_im != 0: both components).  Passes 0 .. *chunked_passes - 1 run
 * chunk by chunk, in order, each chunk being *blocks_per_chunk consecutive
 * blocks of 2^*block_bits elements of each component (the last chunk may
 * hold fewer); the remaining passes then run over the whole state.
 * *chunked_passes = 0: no chunking.  Blocks are whole vectors
 * (*block_bits = n) unless one vector exceeds the 256 MiB Infinity Cache:
 * then the leading passes whose bits all lie below *block_bits are the
 * chunked ones (a transform of each block on its own), e.g. fp32 n = 27,
 * batch 2, passes [10, 9, 8]: passes 0 and 1 on chunks of 64 blocks of
 * 2^19 elements, then pass 2.  Chunking never changes the arithmetic of a
 * pass: the result is bit for bit that of running the passes in order
 * over the whole state.  Returns FWT_OK or FWT_EINVAL (null argument,
 * batch < 0). */
int fwt_plan_call_schedule(fwt_plan_t plan, int64_t batch, int with_im, int* chunked_passes,
                           int* block_bits, int64_t* blocks_per_chunk);

/* Enqueue only pass `pass` (0 <= pass < fwt_plan_num_passes; 0 for an
 * n = 0 plan, which has none and does nothing) of the plan, with the
 * arguments and validation of fwt_execute.  Running passes 0, 1, ..., P-1
 * in order on the same buffers and stream is exactly fwt_execute; the
 * factors commute, so any order gives the same transform up to rounding.
 * `normalize` takes effect only in the last pass.  Meant for per-kernel
 * timing and for interleaving passes with other work.  The cache hints
 * are fwt_execute's, with a state of 256 MiB or more taken as one chunk of
 * a chunked call: running fwt_execute's chunk schedule pass by pass
 * launches the same kernels with the same hints.  Returns as
 * fwt_execute, plus FWT_EINVAL for a pass index out of range. */
int fwt_execute_pass(fwt_plan_t plan, int pass, int64_t batch, int n, void* re,
                     void* im, int normalize, hipStream_t stream);

/* fwt_execute_pass with the pass's kernel timed by the dispatch itself:
 * `start` and `stop` (timing-enabled events the caller owns) are recorded
 * when the kernel starts and ends, so their elapsed time is the kernel's
 * duration without launch gaps.  Returns as fwt_execute_pass, plus
 * FWT_EINVAL for a null event or a call with nothing to launch (batch 0,
 * n = 0). */
int fwt_execute_pass_timed(fwt_plan_t plan, int pass, int64_t batch, int n, void* re,
                           void* im, int normalize, hipStream_t stream,
                           hipEvent_t start, hipEvent_t stop);

/* Run exactly the host-side validation of fwt_execute (same arguments,
 * same status codes, including the device-memory and size checks) without
 * enqueuing anything.  Returns FWT_OK when fwt_execute would launch. */
int fwt_execute_check(fwt_plan_t plan, int64_t batch, int n, const void* re,
                      const void* im);

/* Number of HBM passes one fwt_execute of this plan makes (each reads and
 * writes the state once).  Returns FWT_OK or FWT_EINVAL (null argument). */
int fwt_plan_num_passes(fwt_plan_t plan, int* out_passes);

/* Bit count of pass i (the pass on the lowest bits is i = 0).  Returns
 * FWT_OK or FWT_EINVAL (null argument, i out of range). */
int fwt_plan_pass_bits(fwt_plan_t plan, int i, int* out_bits);

/* Tiling of pass i, for logging and profiling: out[0..9] = first index
 * bit, bit count, kind (0 row pass, 1 column pass, 2 two-element kernel),
 * row bits KR of the tile, register-round bits EB, column-group bits,
 * exchange-phase bits, workgroup size, dynamic LDS bytes, log2 tiles per
 * workgroup, pipelined (1) or not (0), wave-tile kernel (1) or not (0).
 * `out` must hold 12 ints.  Returns FWT_OK or FWT_EINVAL. */
int fwt_plan_pass_config(fwt_plan_t plan, int i, int* out);

/* The tiling (as fwt_plan_pass_config) that pass i of an fwt_execute call
 * on `batch` vectors (with_im != 0: both components) launches.  A one-pass
 * plan may carry a second tiling for states that fit the 256 MiB Infinity
 * Cache (fp32 n = 14 and fp64 n = 13 by default: one LDS exchange in
 * 512-thread workgroups instead of two in 1024-thread ones); other plans
 * launch fwt_plan_pass_config's tiling at every size.  The transform is
 * the same either way.  Returns FWT_OK or FWT_EINVAL (null argument, i out
 * of range, batch < 0). */
int fwt_plan_call_pass_config(fwt_plan_t plan, int i, int64_t batch, int with_im, int* out);

/* Release a plan; NULL is a no-op.  Returns FWT_OK. */
int fwt_plan_destroy(fwt_plan_t plan);

/* Static description of a status code (never NULL). */
const char* fwt_strerror(int status);

/* HIP error code recorded by the most recent FWT_EHIP on the calling
 * thread (hipSuccess if none). */
int fwt_last_hip_error(void);

/* ---- Ablations: the pages' own designs for the same transform ----------
 * Each computes exactly what fwt_execute computes (the same sums in a
 * different association), so they share its parity bars; they exist to be
 * measured against the tile passes. */
typedef enum {
    /* One launch per butterfly stage, each streaming the whole state: the
     * global-memory FWT of the Apache Mahout pull request "[QDP] [feature]
     * Pr4 kronecker fwt" ("Benchmark Results", "Why submit PR4").
     * n >= 2 (fp32) / 1 (fp64). */
    FWT_ABLATION_STAGEWISE = 1,
    /* The pull request's Kronecker scaffold (section "How"): on the
     * 2^(n/2) x 2^(n - n/2) view, every row times H_{n-n/2} by a direct
     * sum with each sign generated from popcount(k AND i), a batch
     * transpose into the workspace, the same GEMM for H_{n/2}, a transpose
     * back.  2 <= n <= 26; needs a workspace of the state's size. */
    FWT_ABLATION_POPC_GEMM = 2,
    /* Matrix-core block Hadamard (the iThome "Day 18" native-FWT article,
     * "Kronecker block GEMM idea", "TF32 path"): a FWT_PATH_MFMA_ABLATION
     * plan, i.e. fwt_execute's split and column passes with the row pass
     * (the low 8..15 bits) done as dense H_16 block products on the fp32
     * / fp64 16x16x4 matrix instructions (leftover bits butterflied in
     * LDS).  8 <= n <= 30 (fp32) / 29 (fp64); no workspace. */
    FWT_ABLATION_MFMA = 3,
    /* INT8 / CRT emulation of the fp64 transform (the iThome article,
     * "INT8 / Ozaki path", "Data flow of the implementation", radix form
     * of "case_3 experimental judgements"): each vector component scaled
     * by its own power of two to integers of at most 48 bits, split into
     * residues mod m <= 10 primes below 256 (balanced int8), transformed
     * in residue space by Kronecker passes of 32-position blocks on
     * v_mfma_i32_16x16x32_i8 with reduction mod p, rebuilt by CRT with a
     * rounded fp64 quotient (the sum exact in 128-bit integers) and scaled
     * back.  Exact
     * for integer-valued inputs; otherwise within 2^-46 of max |x| times
     * sqrt(2^n) per output.  fp64 only (fp32: FWT_EUNSUPPORTED); finite
     * inputs; 5 <= n <= 28; needs a workspace (the residues, 4 ceil(m / 4)
     * bytes per element, plus per-vector scales). */
    FWT_ABLATION_OZAKI = 4,
    /* Matrix-core block Hadamard on both Kronecker factors with a
     * transposed staging buffer (the iThome article's TF32 data flow on
     * the fp32 / fp64 16x16x4 matrix instructions): block products on the
     * contiguous n - n/2 bits, a transpose of every vector into the
     * workspace, block products on the n/2 bits, a transpose back.
     * 16 <= n <= 30 (fp32) / 28 (fp64); needs a workspace of the state's
     * size. */
    FWT_ABLATION_MFMA_TRANSPOSE = 5
} fwt_ablation;

/* Workspace bytes fwt_ablation_execute needs for `batch` vectors (0 if
 * none).  Returns FWT_OK or FWT_EINVAL. */
int fwt_ablation_workspace(int kind, int64_t batch, int n, fwt_dtype dtype, int with_im,
                           size_t* out);

/* Run ablation `kind` on planar device buffers in place, asynchronously on
 * `stream`, with the argument rules of fwt_execute; `workspace` (device
 * memory of at least fwt_ablation_workspace bytes, 16-byte aligned, not
 * overlapping re/im; NULL when none is needed) is scratch owned by the
 * caller.  Returns FWT_OK, FWT_EINVAL, FWT_EALIGN, FWT_EUNSUPPORTED (kind
 * or n outside its range) or FWT_EHIP. */
int fwt_ablation_execute(int kind, int64_t batch, int n, fwt_dtype dtype, void* re, void* im,
                         int normalize, void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/* Size of the static device scratch array of fwt_ablation_execute_static
 * (32 MiB per device, held until the process ends). */
#define FWT_STATIC_SCRATCH_BYTES (32u << 20)

/* fwt_ablation_execute for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same kinds, arguments, layout and results as
 * fwt_ablation_execute, but the workspace is the library's static scratch
 * array on the current device (FWT_STATIC_SCRATCH_BYTES), so no workspace
 * is passed.  The call allocates no device memory and calls no device
 * allocation routine.  (As with fwt_ablation_execute, the matrix-core kind
 * builds its small host-side plan on its first call for each dtype and n,
 * and keeps it for the process.)  The caller still provides re and im.
 *  - Returns FWT_ESCRATCH when fwt_ablation_workspace for the call exceeds
 *    FWT_STATIC_SCRATCH_BYTES (e.g. the popcount GEMM or the transposed
 *    matrix-core form beyond 32 MiB of state, the INT8 / CRT form beyond
 *    about 2^21 fp64 elements per component), otherwise the statuses of
 *    fwt_ablation_execute.
 *  - Every call on one device shares that device's array, and the array
 *    keeps the last call's contents (no kernel reads it before writing it).
 *    Calls that overlap in time on one device (concurrent streams, or host
 *    threads whose streams are not ordered) race on it and give undefined
 *    results: order them on one stream. */
int fwt_ablation_execute_static(int kind, int64_t batch, int n, fwt_dtype dtype, void* re,
                                void* im, int normalize, hipStream_t stream);

/* Measurement aid, not part of the transform: copies `bytes` (a multiple
 * of 16) from src to dst with the same 16-byte streaming access the passes
 * use, so a benchmark can price one read plus one write of the state.
 * Both device buffers 16-byte aligned and non-overlapping.  Returns
 * FWT_OK, FWT_EINVAL, FWT_EALIGN or FWT_EHIP. */
int fwt_stream_copy(void* dst, const void* src, int64_t bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* QSE_FWT_H */
