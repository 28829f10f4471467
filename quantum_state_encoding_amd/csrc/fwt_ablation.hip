// The pages' own designs for the same transform, rebuilt on gfx950 as
// measured ablations of the tile-pass path (fwt_kernels.hip):
//
//  * stage-wise global FWT: one launch per butterfly stage, each reading and
//    writing the whole state (the global-memory FWT the Apache Mahout pull
//    request "[QDP] [feature] Pr4 kronecker fwt" benchmarks against,
//    sections "Benchmark Results" and "Why submit PR4": one DRAM
//    traversal per stage);
//  * matrix-core block Hadamard: the contiguous row pass rewritten as
//    dense H_16 block products on v_mfma_*_16x16x4 (the iThome "Day 18"
//    native-FWT article, sections "Kronecker block GEMM idea" and "TF32
//    path": reshape, block Hadamard GEMM, with the layout change fused into
//    the kernel; gfx950 has no TF32, so fp32 and fp64 matrix cores);
//  * Kronecker GEMM scaffold: Z = X . H_{n2} on every row of the
//    2^n1 x 2^n2 view with each Walsh entry generated from the population
//    count of k AND i, a batched transpose, the same GEMM for H_{n1}, and a
//    transpose back (the pull request's section "How": the naive implicit
//    Hadamard GEMM placeholder, the batch transpose between the two GEMM
//    stages, the temporary buffers; its "4-step blocked algorithm");
//  * matrix-core blocks on both Kronecker factors: the block-Hadamard row
//    kernel on the low n2 bits, a batched transpose into a staging buffer,
//    the same kernel on the other n1 bits, and a transpose back (the
//    iThome article, sections "TF32 path" and "Data flow of the
//    implementation": block GEMM, transpose into a staging buffer, block
//    GEMM, transpose back).
//
// All of them compute exactly the transform of the tile passes (a
// different association of the same sums), so they share its parity
// tests.
#include <hip/hip_runtime.h>

#include "fwt_internal.h"

namespace qse {
namespace {

template <typename T>
struct Vec16;
template <>
struct Vec16<float> {
    typedef float type __attribute__((ext_vector_type(4)));
    static constexpr int WB = 2;
};
template <>
struct Vec16<double> {
    typedef double type __attribute__((ext_vector_type(2)));
    static constexpr int WB = 1;
};

// ---- stage-wise global FWT ------------------------------------------------
//
// Stage s >= vb: thread t owns the 16-byte vector pair (v, v + 2^(s-vb)) with
// bit (s - vb) of v clear; stage s < vb works inside each vector.  One launch
// per stage; the last multiplies by `scale` when do_scale.

template <typename T>
__global__ void __launch_bounds__(256)
    stage_pair_kernel(T* __restrict__ re, T* __restrict__ im, int64_t pairs, int sv,
                      int do_scale, T scale)
{
    using V = typename Vec16<T>::type;
    V* const buf = reinterpret_cast<V*>(blockIdx.y ? im : re);
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t low_mask = ((int64_t)1 << sv) - 1;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < pairs; t += stride) {
        const int64_t v = ((t >> sv) << (sv + 1)) | (t & low_mask);
        V a = buf[v], b = buf[v + ((int64_t)1 << sv)];
        V s = a + b, d = a - b;
        if (do_scale) {
            s *= scale;
            d *= scale;
        }
        buf[v] = s;
        buf[v + ((int64_t)1 << sv)] = d;
    }
}

__device__ __forceinline__ void stage_in_vector(Vec16<float>::type& v, int s)
{
    if (s == 0) {
        const float a0 = v.x + v.y, a1 = v.x - v.y, a2 = v.z + v.w, a3 = v.z - v.w;
        v.x = a0;
        v.y = a1;
        v.z = a2;
        v.w = a3;
    } else {
        const float a0 = v.x + v.z, a2 = v.x - v.z, a1 = v.y + v.w, a3 = v.y - v.w;
        v.x = a0;
        v.y = a1;
        v.z = a2;
        v.w = a3;
    }
}
__device__ __forceinline__ void stage_in_vector(Vec16<double>::type& v, int)
{
    const double a = v.x + v.y, b = v.x - v.y;
    v.x = a;
    v.y = b;
}

template <typename T>
__global__ void __launch_bounds__(256)
    stage_in_vector_kernel(T* __restrict__ re, T* __restrict__ im, int64_t nvec, int s,
                           int do_scale, T scale)
{
    using V = typename Vec16<T>::type;
    V* const buf = reinterpret_cast<V*>(blockIdx.y ? im : re);
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < nvec; t += stride) {
        V v = buf[t];
        stage_in_vector(v, s);
        if (do_scale)
            v *= scale;
        buf[t] = v;
    }
}

// ---- Kronecker GEMM scaffold ----------------------------------------------
//
// popc_gemm_kernel: every row of length 2^m (rows contiguous) is replaced by
// z_k = sum_i (-1)^popcount(k AND i) x_i, computed directly (2^m products
// per output), the row staged in LDS first so the update is in place.
// One workgroup per row (or several rows when a row is short).

template <typename T>
__global__ void __launch_bounds__(256)
    popc_gemm_kernel(T* __restrict__ re, T* __restrict__ im, int64_t rows, int m, int do_scale,
                     T scale)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
    T* const lds = reinterpret_cast<T*>(lds_raw);
    T* const buf = blockIdx.y ? im : re;
    const int L = 1 << m;
    const int rows_per_wg = L >= 256 ? 1 : 256 / L;
    for (int64_t r0 = (int64_t)blockIdx.x * rows_per_wg; r0 < rows;
         r0 += (int64_t)gridDim.x * rows_per_wg) {
        // stage rows_per_wg rows (or what is left) in LDS
        const int nrows = (int)(rows - r0 < rows_per_wg ? rows - r0 : rows_per_wg);
        for (int i = threadIdx.x; i < nrows * L; i += blockDim.x)
            lds[i] = buf[r0 * L + i];
        __syncthreads();
        for (int o = threadIdx.x; o < nrows * L; o += blockDim.x) {
            const int rr = o >> m, k = o & (L - 1);
            const T* x = lds + rr * L;
            T acc = 0;
            for (int i = 0; i < L; ++i)
                acc += (__builtin_popcount((unsigned)(k & i)) & 1) ? -x[i] : x[i];
            buf[r0 * L + o] = do_scale ? acc * scale : acc;
        }
        __syncthreads();
    }
}

// Batched transpose of R x C row-major matrices (R, C powers of two), out
// of place: dst[b][c][r] = src[b][r][c], through 32 x 32 LDS tiles (padded
// by one element against bank conflicts).
template <typename T>
__global__ void __launch_bounds__(256)
    transpose_kernel(const T* __restrict__ src_re, const T* __restrict__ src_im,
                     T* __restrict__ dst_re, T* __restrict__ dst_im, int rbits, int cbits,
                     int64_t mats)
{
    __shared__ T tile[32][33];
    const T* const src = blockIdx.z ? src_im : src_re;
    T* const dst = blockIdx.z ? dst_im : dst_re;
    const int R = 1 << rbits, C = 1 << cbits;
    const int tr = R < 32 ? R : 32, tc = C < 32 ? C : 32;
    const int64_t tiles_c = C / tc, tiles_r = R / tr;
    const int64_t tiles_per_mat = tiles_c * tiles_r;
    for (int64_t t = blockIdx.x; t < mats * tiles_per_mat; t += gridDim.x) {
        const int64_t mat = t / tiles_per_mat;
        const int64_t rem = t % tiles_per_mat;
        const int64_t r0 = (rem / tiles_c) * tr, c0 = (rem % tiles_c) * tc;
        const T* s = src + (mat << (rbits + cbits));
        T* d = dst + (mat << (rbits + cbits));
        for (int i = threadIdx.x; i < tr * tc; i += blockDim.x) {
            const int rr = i / tc, cc = i % tc;
            tile[rr][cc] = s[(r0 + rr) * C + c0 + cc];
        }
        __syncthreads();
        for (int i = threadIdx.x; i < tr * tc; i += blockDim.x) {
            const int cc = i / tr, rr = i % tr;
            d[(c0 + cc) * R + r0 + rr] = tile[rr][cc];
        }
        __syncthreads();
    }
}

// ---- matrix-core block Hadamard row pass -----------------------------------
//
// A workgroup stages TPW contiguous tiles of 2^KM elements in LDS (one pad
// element per 16).  For each group of 4 index bits [4q, 4q + 4), q < KM / 4,
// the tile's 2^(KM-4) "lines" (16 elements differing only in those bits)
// are multiplied by H_16 on the matrix cores: 16 lines at a time form the
// A operand (lane l holds line l mod 16, column 4 kb + l / 16), the B
// operand is the H_16 slab with entries (-1)^popcount(k AND j), and four
// K = 4 products accumulate the 16 x 16 result, written back over the same
// lines.  The KM mod 4 remaining top bits are butterflied in LDS.

template <typename T>
struct MfmaOps;
template <>
struct MfmaOps<float> {
    typedef float acc_t __attribute__((ext_vector_type(4)));
    __device__ __forceinline__ static acc_t mma(float a, float b, acc_t c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    // Result row (line within the block) of lane l, register r.
    __device__ __forceinline__ static int row(int l, int r) { return 4 * (l >> 4) + r; }
};
template <>
struct MfmaOps<double> {
    typedef double acc_t __attribute__((ext_vector_type(4)));
    __device__ __forceinline__ static acc_t mma(double a, double b, acc_t c)
    {
        return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
    }
    __device__ __forceinline__ static int row(int l, int r) { return (l >> 4) + 4 * r; }
};

__device__ __forceinline__ int pad16(int e) { return e + (e >> 4); }

// Element index of line lam, column k (4 bits) for the bit group at 4q.
__device__ __forceinline__ int line_elem(int lam, int k, int q)
{
    const int lo = lam & ((1 << (4 * q)) - 1);
    const int hi = lam >> (4 * q);
    return (hi << (4 * q + 4)) | (k << (4 * q)) | lo;
}

// Workgroups of 256 threads, 1024 for tiles of 2^13 elements and more.
template <int KM>
constexpr int mfma_threads() { return KM >= 13 ? 1024 : 256; }

template <typename T, int KM>
__global__ void __launch_bounds__(mfma_threads<KM>())
    mfma_row_kernel(T* __restrict__ re, T* __restrict__ im, int64_t tiles, int do_scale, T scale)
{
    constexpr int NT = mfma_threads<KM>(), NW = NT / 64;
    using Ops = MfmaOps<T>;
    using acc_t = typename Ops::acc_t;
    constexpr int TPW = KM >= 12 ? 1 : 1 << (12 - KM);   // tiles per workgroup
    constexpr int L = 1 << KM;
    constexpr int TL = L + (L >> 4);                      // padded tile length
    constexpr int G = KM / 4;                             // MFMA bit groups
    constexpr int LINES = L >> 4;                         // lines per tile and group
    extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
    T* const lds = reinterpret_cast<T*>(lds_raw);
    T* const buf = blockIdx.y ? im : re;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t t0 = (int64_t)blockIdx.x * TPW;
    const int ntile = (int)(tiles - t0 < TPW ? tiles - t0 : TPW);

    // 16-byte global accesses; the W elements of one vector stay inside one
    // padded run of 16, so they land on consecutive LDS words.
    using V = typename Vec16<T>::type;
    constexpr int W = 16 / sizeof(T);
    V* const gv = reinterpret_cast<V*>(buf + t0 * L);
    for (int i = tid; i < ntile * (L / W); i += NT) {
        const V v = gv[i];
        const int e = i * W;
        T* const d = lds + (e / L) * TL + pad16(e % L);
#pragma unroll
        for (int w = 0; w < W; ++w)
            d[w] = v[w];
    }
    __syncthreads();

    // B operand slabs: B[kb][l] = H_16[4 kb + l / 16][l mod 16].
    T h[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
        h[kb] = (__builtin_popcount((unsigned)((4 * kb + (lane >> 4)) & (lane & 15))) & 1) ? T(-1)
                                                                                            : T(1);
#pragma unroll
    for (int q = 0; q < G; ++q) {
        // blocks of 16 lines, over all tiles of the workgroup, split by wave
        const int blocks = ntile * (LINES >> 4);
        for (int blk = wave; blk < blocks; blk += NW) {
            const int tile = blk / (LINES >> 4);
            const int lam0 = (blk % (LINES >> 4)) << 4;
            T* const tl = lds + tile * TL;
            acc_t acc = {0, 0, 0, 0};
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const T a = tl[pad16(line_elem(lam0 + (lane & 15), 4 * kb + (lane >> 4), q))];
                acc = Ops::mma(a, h[kb], acc);
            }
            // every lane has read its operands (the MFMA consumed them)
            // before any lane of this wave writes the block back
#pragma unroll
            for (int r = 0; r < 4; ++r)
                tl[pad16(line_elem(lam0 + Ops::row(lane, r), lane & 15, q))] = acc[r];
        }
        __syncthreads();
    }
    // remaining top bits [4G, KM): butterflies in LDS
#pragma unroll
    for (int b = 4 * G; b < KM; ++b) {
        for (int i = tid; i < ntile * (L >> 1); i += NT) {
            const int tile = i / (L >> 1), p = i % (L >> 1);
            const int e = ((p >> b) << (b + 1)) | (p & ((1 << b) - 1));
            T* const tl = lds + tile * TL;
            const T x = tl[pad16(e)], y = tl[pad16(e + (1 << b))];
            tl[pad16(e)] = x + y;
            tl[pad16(e + (1 << b))] = x - y;
        }
        __syncthreads();
    }
    for (int i = tid; i < ntile * (L / W); i += NT) {
        const int e = i * W;
        const T* const d = lds + (e / L) * TL + pad16(e % L);
        V v;
#pragma unroll
        for (int w = 0; w < W; ++w)
            v[w] = do_scale ? d[w] * scale : d[w];
        gv[i] = v;
    }
}

template <typename T, int KM>
hipError_t mfma_row_launch(T* re, T* im, int64_t tiles, int do_scale, double c,
                           hipStream_t stream)
{
    constexpr int TPW = KM >= 12 ? 1 : 1 << (12 - KM);
    constexpr size_t lds = (size_t)TPW * ((1 << KM) + ((1 << KM) >> 4)) * sizeof(T);
    const void* fn = reinterpret_cast<const void*>(&mfma_row_kernel<T, KM>);
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess)
        return e;
    // at most 2^20 workgroups (2^28 work-items) per launch
    const int64_t per_launch = (int64_t)TPW << 20;
    for (int64_t t0 = 0; t0 < tiles; t0 += per_launch) {
        const int64_t nt = tiles - t0 < per_launch ? tiles - t0 : per_launch;
        const int64_t off = t0 << KM;
        hipLaunchKernelGGL((mfma_row_kernel<T, KM>),
                           dim3((unsigned)((nt + TPW - 1) / TPW), im ? 2 : 1),
                           dim3(mfma_threads<KM>()), lds, stream, re + off, im ? im + off : nullptr,
                           nt, do_scale, (T)c);
        e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

template <typename T>
hipError_t mfma_row_dispatch(T* re, T* im, int64_t tiles, int km, int do_scale, double c,
                             hipStream_t stream)
{
    switch (km) {
    case 8: return mfma_row_launch<T, 8>(re, im, tiles, do_scale, c, stream);
    case 9: return mfma_row_launch<T, 9>(re, im, tiles, do_scale, c, stream);
    case 10: return mfma_row_launch<T, 10>(re, im, tiles, do_scale, c, stream);
    case 11: return mfma_row_launch<T, 11>(re, im, tiles, do_scale, c, stream);
    case 12: return mfma_row_launch<T, 12>(re, im, tiles, do_scale, c, stream);
    case 13: return mfma_row_launch<T, 13>(re, im, tiles, do_scale, c, stream);
    case 14: return mfma_row_launch<T, 14>(re, im, tiles, do_scale, c, stream);
    case 15:
        // 2^15 padded fp64 elements exceed the LDS
        if (sizeof(T) == 4)
            return mfma_row_launch<T, 15>(re, im, tiles, do_scale, c, stream);
        return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
    }
}

unsigned grid_for(int64_t work, int64_t per_block)
{
    int64_t g = (work + per_block - 1) / per_block;
    if (g < 1)
        g = 1;
    if (g > (1 << 20))
        g = 1 << 20;
    return (unsigned)g;
}

template <typename T>
hipError_t stagewise_impl(T* re, T* im, int64_t batch, int n, int normalize, double c,
                          hipStream_t stream)
{
    constexpr int WB = Vec16<T>::WB;
    const int ncomp = im ? 2 : 1;
    const int64_t nvec = (batch << n) >> WB;
    for (int s = 0; s < n; ++s) {
        const int last = (s == n - 1);
        const int do_scale = normalize && last;
        if (s < WB) {
            hipLaunchKernelGGL(stage_in_vector_kernel<T>, dim3(grid_for(nvec, 256), ncomp),
                               dim3(256), 0, stream, re, im, nvec, s, do_scale, (T)c);
        } else {
            const int64_t pairs = nvec / 2;
            hipLaunchKernelGGL(stage_pair_kernel<T>, dim3(grid_for(pairs, 256), ncomp),
                               dim3(256), 0, stream, re, im, pairs, s - WB, do_scale, (T)c);
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

template <typename T>
hipError_t popc_gemm_impl(T* re, T* im, T* ws_re, T* ws_im, int64_t batch, int n, int normalize,
                          double c, hipStream_t stream)
{
    const int ncomp = im ? 2 : 1;
    const int n1 = n / 2, n2 = n - n1;   // H_n = H_{n1} (x) H_{n2}; n2 on the contiguous bits
    auto gemm = [&](T* a, T* b, int m, int64_t rows, int do_scale) {
        const int L = 1 << m;
        const int rows_per_wg = L >= 256 ? 1 : 256 / L;
        const size_t lds = (size_t)rows_per_wg * L * sizeof(T);
        hipLaunchKernelGGL(popc_gemm_kernel<T>, dim3(grid_for(rows, rows_per_wg), ncomp),
                           dim3(256), lds, stream, a, b, rows, m, do_scale, (T)c);
        return hipGetLastError();
    };
    auto transpose = [&](const T* sa, const T* sb, T* da, T* db, int rbits, int cbits) {
        const int tr = rbits < 5 ? 1 << rbits : 32, tc = cbits < 5 ? 1 << cbits : 32;
        const int64_t tiles = batch * ((int64_t)1 << (rbits + cbits)) / ((int64_t)tr * tc);
        hipLaunchKernelGGL(transpose_kernel<T>, dim3(grid_for(tiles, 1), 1, ncomp), dim3(256), 0,
                           stream, sa, sb, da, db, rbits, cbits, batch);
        return hipGetLastError();
    };
    hipError_t e;
    // 1. Z = X . H_{n2} on the 2^n1 rows of length 2^n2 of every vector
    if ((e = gemm(re, im, n2, batch << n1, 0)) != hipSuccess)
        return e;
    // 2. transpose each 2^n1 x 2^n2 matrix into the workspace
    if ((e = transpose(re, im, ws_re, ws_im, n1, n2)) != hipSuccess)
        return e;
    // 3. the 2^n2 rows of length 2^n1 times H_{n1}
    if ((e = gemm(ws_re, ws_im, n1, batch << n2, normalize)) != hipSuccess)
        return e;
    // 4. transpose back
    return transpose(ws_re, ws_im, re, im, n2, n1);
}

// The matrix-core design with a transposed staging buffer, in the order of
// the iThome "Day 18" native-FWT article's TF32 data flow: block-Hadamard
// products on the contiguous n2 = n - n/2 bits, a transpose of every
// 2^n1 x 2^n2 matrix into the workspace, block products on the n1 bits
// (now contiguous), and a transpose back.
template <typename T>
hipError_t mfma_transpose_impl(T* re, T* im, T* ws_re, T* ws_im, int64_t batch, int n,
                               int normalize, double c, hipStream_t stream)
{
    const int ncomp = im ? 2 : 1;
    const int n1 = n / 2, n2 = n - n1;
    auto transpose = [&](const T* sa, const T* sb, T* da, T* db, int rbits, int cbits) {
        const int tr = rbits < 5 ? 1 << rbits : 32, tc = cbits < 5 ? 1 << cbits : 32;
        const int64_t tiles = batch * ((int64_t)1 << (rbits + cbits)) / ((int64_t)tr * tc);
        hipLaunchKernelGGL(transpose_kernel<T>, dim3(grid_for(tiles, 1), 1, ncomp), dim3(256), 0,
                           stream, sa, sb, da, db, rbits, cbits, batch);
        return hipGetLastError();
    };
    hipError_t e;
    if ((e = mfma_row_dispatch<T>(re, im, batch << n1, n2, 0, c, stream)) != hipSuccess)
        return e;
    if ((e = transpose(re, im, ws_re, ws_im, n1, n2)) != hipSuccess)
        return e;
    if ((e = mfma_row_dispatch<T>(ws_re, ws_im, batch << n2, n1, normalize, c, stream)) !=
        hipSuccess)
        return e;
    return transpose(ws_re, ws_im, re, im, n2, n1);
}

}  // namespace

hipError_t ablation_mfma_transpose(int f64, void* re, void* im, void* ws_re, void* ws_im,
                                   int64_t batch, int n, int normalize, double c,
                                   hipStream_t stream)
{
    if (f64)
        return mfma_transpose_impl<double>((double*)re, (double*)im, (double*)ws_re,
                                           (double*)ws_im, batch, n, normalize, c, stream);
    return mfma_transpose_impl<float>((float*)re, (float*)im, (float*)ws_re, (float*)ws_im,
                                      batch, n, normalize, c, stream);
}

hipError_t ablation_mfma_row(int f64, void* re, void* im, int64_t batch, int n, int km,
                             int do_scale, double c, hipStream_t stream)
{
    const int64_t tiles = batch << (n - km);
    if (f64)
        return mfma_row_dispatch<double>((double*)re, (double*)im, tiles, km, do_scale, c, stream);
    return mfma_row_dispatch<float>((float*)re, (float*)im, tiles, km, do_scale, c, stream);
}

hipError_t ablation_stagewise(int f64, void* re, void* im, int64_t batch, int n, int normalize,
                              double c, hipStream_t stream)
{
    if (f64)
        return stagewise_impl<double>((double*)re, (double*)im, batch, n, normalize, c, stream);
    return stagewise_impl<float>((float*)re, (float*)im, batch, n, normalize, c, stream);
}

hipError_t ablation_popc_gemm(int f64, void* re, void* im, void* ws_re, void* ws_im,
                              int64_t batch, int n, int normalize, double c, hipStream_t stream)
{
    if (f64)
        return popc_gemm_impl<double>((double*)re, (double*)im, (double*)ws_re, (double*)ws_im,
                                      batch, n, normalize, c, stream);
    return popc_gemm_impl<float>((float*)re, (float*)im, (float*)ws_re, (float*)ws_im, batch, n,
                                 normalize, c, stream);
}

}  // namespace qse
