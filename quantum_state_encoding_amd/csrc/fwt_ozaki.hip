// INT8 / CRT ("Ozaki") form of the fp64 transform, built as a measured
// ablation of the tile passes: the data flow of the iThome "Day 18"
// native-FWT article, sections "INT8 / Ozaki path" and "Data flow of the
// implementation" (floating input, scaled integer, residues mod p as
// balanced int8, INT8 matrix products against the +-1 Hadamard block with
// int32 accumulation, reduction mod p, CRT reconstruction and scaling),
// in its Kronecker ("radix") form from "case_3 experimental judgements".
//
// For each vector component b with max |x| < 2^e_b (e_b from frexp):
//   X_i = rint(x_i * 2^(48 - e_b)), an integer with |X_i| <= 2^48;
//   Y = H_n X is an integer with |Y_k| <= 2^(48 + n);
//   m primes p_j <= 251 with prod p_j > 2^(49 + n) carry Y through CRT:
//   residue planes r_j = X mod p_j (|r| <= 127, int8), transformed in
//   residue space, then Y rebuilt from the residues (Garner's mixed-radix
//   digits, balanced, summed exactly in 128-bit integers), and
//   y_k = Y_k * 2^(e_b - 48) * c.
// Integer-valued inputs are transformed exactly.  Otherwise the error is
// that of rounding X: at most 2^(2 - 48) of max |x| per output times
// sqrt(2^n) (normalised), far inside fp64 tolerances.
//
// Kernels: per-slice maxima -> per-vector exponents -> split into residue
// planes -> Kronecker passes over the planes (32-position blocks on
// v_mfma_i32_16x16x32_i8) -> merge (Garner + scaling).  The planes live in
// a caller-provided workspace.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "fwt_internal.h"

namespace qse {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef double f64x2 __attribute__((ext_vector_type(2)));

constexpr int kSliceBits = 16;   // elements per partial maximum

// ---- maxima and exponents -----------------------------------------------

__global__ void __launch_bounds__(256)
    oz_max_kernel(const double* __restrict__ re, const double* __restrict__ im, int n,
                  int64_t batch, int slice_bits, double* __restrict__ partial)
{
    const double* const x = blockIdx.y ? im : re;
    const int64_t slices = (int64_t)1 << (n - slice_bits);
    __shared__ double wmax[4];
    for (int64_t idx = blockIdx.x; idx < batch * slices; idx += gridDim.x) {
        const int64_t b = idx / slices, s = idx % slices;
        const f64x2* const v =
            reinterpret_cast<const f64x2*>(x + (b << n) + (s << slice_bits));
        double mx = 0.0;
        for (int i = threadIdx.x; i < (1 << (slice_bits - 1)); i += 256) {
            const f64x2 a = v[i];
            mx = fmax(mx, fmax(fabs(a.x), fabs(a.y)));
        }
        for (int off = 32; off > 0; off >>= 1)
            mx = fmax(mx, __shfl_xor(mx, off));
        if ((threadIdx.x & 63) == 0)
            wmax[threadIdx.x >> 6] = mx;
        __syncthreads();
        if (threadIdx.x == 0)
            partial[(int64_t)blockIdx.y * batch * slices + idx] =
                fmax(fmax(wmax[0], wmax[1]), fmax(wmax[2], wmax[3]));
        __syncthreads();
    }
}

__global__ void __launch_bounds__(256)
    oz_exponent_kernel(const double* __restrict__ partial, int64_t vectors, int64_t slices,
                       int* __restrict__ exps)
{
    const int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (v >= vectors)
        return;
    double mx = 0.0;
    for (int64_t s = 0; s < slices; ++s)
        mx = fmax(mx, partial[v * slices + s]);
    int e = 0;
    if (mx > 0.0)
        frexp(mx, &e);   // mx = f * 2^e, 0.5 <= f < 1, so every |x| < 2^e
    exps[v] = e;
}

// ---- split into residue planes ------------------------------------------
//
// Thread g takes 8 consecutive elements of one component; plane j of
// component c starts at planes + (c * m + j) * plane_len.

__global__ void __launch_bounds__(256)
    oz_split_kernel(const double* __restrict__ re, const double* __restrict__ im, int n,
                    int64_t groups, const int* __restrict__ exps, int64_t batch,
                    int8_t* __restrict__ planes, int64_t plane_len, OzConst k)
{
    const double* const x = blockIdx.y ? im : re;
    const int* const ex = exps + blockIdx.y * batch;
    int8_t* const base = planes + (int64_t)blockIdx.y * k.m * plane_len;
    for (int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x; g < groups;
         g += (int64_t)gridDim.x * 256) {
        const int64_t e0 = g * 8;
        const int sh = kOzScaleBits - ex[e0 >> n];
        const f64x2* const v = reinterpret_cast<const f64x2*>(x + e0);
        double X[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f64x2 a = v[i];
            X[2 * i] = rint(ldexp(a.x, sh));
            X[2 * i + 1] = rint(ldexp(a.y, sh));
        }
        for (int j = 0; j < k.m; ++j) {
            const double p = (double)k.p[j];
            uint64_t packed = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                // X - p * nearest(X / p) is exact (|X| <= 2^48); |r| <= (p + 1) / 2
                const double r = fma(-p, rint(X[i] * k.inv_pd[j]), X[i]);
                packed |= (uint64_t)(uint8_t)(int8_t)(int)r << (8 * i);
            }
            *reinterpret_cast<uint64_t*>(base + (int64_t)j * plane_len + e0) = packed;
        }
    }
}

// ---- Kronecker passes over the residue planes -----------------------------
//
// A workgroup owns one tile of 2^TB residues of one plane in LDS.  Tile
// index t:
//   ROW (bits [0, kt)):  t = line << kt | position, 2^TB contiguous bytes;
//   COL (bits [lo, lo + kt)): t = position << cb | column, 2^kt rows of
//     2^cb contiguous bytes at stride 2^lo.
// Each stage transforms up to 5 tile-index bits inside a 5-bit window at w
// (`mask` marks which window bits to transform; the others are identity).
// Sixteen "lines" (the tile-index bits outside the window) at a time form
// the B operand of v_mfma_i32_16x16x32_i8 (lane l: line l mod 16,
// positions 8 (l / 16) .. + 7, one byte each), and two 16 x 32 slabs of
// the window matrix M[o][k] = [(o ^ k) & ~mask = 0] (-1)^popcount(o & k &
// mask) form A (lane l: output l mod 16, positions 8 (l / 16) .. + 7).
// Result register r of lane l is output 4 (l / 16) + r of line l mod 16;
// it is reduced mod p and written over the line.

__device__ __forceinline__ int window_addr(int lam, int k, int w)
{
    return ((lam >> w) << (w + 5)) | (k << w) | (lam & ((1 << w) - 1));
}

__device__ __forceinline__ int reduce_mod(int d, int p, float inv_p)
{
    return d - p * (int)rintf((float)d * inv_p);
}

template <bool ROW>
__global__ void __launch_bounds__(256)
    oz_pass_kernel(int8_t* __restrict__ planes, int64_t plane_len, int m, int64_t tile0, int lo,
                   int kt, int xb, int nstage, int w0, int mask0, int w1, int mask1, OzConst k)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
    int8_t* const lds = reinterpret_cast<int8_t*>(lds_raw);
    const int TB = kt + xb;
    const int plane = blockIdx.y;
    const int p = k.p[plane % m];
    const float inv_p = k.inv_pf[plane % m];
    int8_t* const pl = planes + (int64_t)plane * plane_len;
    const int64_t tile = tile0 + blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    // load (16-byte chunks)
    int64_t base;
    int valid;   // ROW: bytes of this tile inside the plane
    if (ROW) {
        base = tile << TB;
        const int64_t left = plane_len - base;
        valid = (int)(left < ((int64_t)1 << TB) ? left : ((int64_t)1 << TB));
        for (int i = tid; i < (1 << (TB - 4)); i += 256) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (i * 16 < valid)
                v = *reinterpret_cast<const uint4*>(pl + base + i * 16);
            *reinterpret_cast<uint4*>(lds + i * 16) = v;
        }
    } else {
        const int cb = xb;
        const int64_t cblk = tile & (((int64_t)1 << (lo - cb)) - 1);
        const int64_t outer = tile >> (lo - cb);
        base = (outer << (kt + lo)) | (cblk << cb);
        valid = 1 << TB;
        const int per_row = 1 << (cb - 4);
        for (int i = tid; i < (1 << (TB - 4)); i += 256) {
            const int row = i / per_row, ch = i % per_row;
            *reinterpret_cast<uint4*>(lds + i * 16) =
                *reinterpret_cast<const uint4*>(pl + base + ((int64_t)row << lo) + ch * 16);
        }
    }
    __syncthreads();

    for (int st = 0; st < nstage; ++st) {
        const int w = st ? w1 : w0, mask = st ? mask1 : mask0;
        // window-matrix slabs: A[o][kk] for o = 16 s + (lane mod 16)
        long a[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            uint64_t packed = 0;
            const int o = 16 * s + (lane & 15);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int kk = 8 * (lane >> 4) + j;
                int v = 0;
                if (((o ^ kk) & ~mask & 31) == 0)
                    v = (__builtin_popcount((unsigned)(o & kk & mask)) & 1) ? -1 : 1;
                packed |= (uint64_t)(uint8_t)(int8_t)v << (8 * j);
            }
            a[s] = (long)packed;
        }
        const int nblk = 1 << (TB - 9);   // blocks of 16 lines x 32 positions
        for (int blk = wave; blk < nblk; blk += 4) {
            const int lam = (blk << 4) + (lane & 15);
            uint64_t packed = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                packed |= (uint64_t)(uint8_t)lds[window_addr(lam, 8 * (lane >> 4) + j, w)]
                          << (8 * j);
            const i32x4 zero = {0, 0, 0, 0};
            const i32x4 d0 = __builtin_amdgcn_mfma_i32_16x16x32_i8(a[0], (long)packed, zero, 0, 0, 0);
            const i32x4 d1 = __builtin_amdgcn_mfma_i32_16x16x32_i8(a[1], (long)packed, zero, 0, 0, 0);
            // every lane's operand bytes are in registers before any write
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int o = 4 * (lane >> 4) + r;
                lds[window_addr(lam, o, w)] = (int8_t)reduce_mod(d0[r], p, inv_p);
                lds[window_addr(lam, o + 16, w)] = (int8_t)reduce_mod(d1[r], p, inv_p);
            }
        }
        __syncthreads();
    }

    if (ROW) {
        for (int i = tid; i < (1 << (TB - 4)); i += 256)
            if (i * 16 < valid)
                *reinterpret_cast<uint4*>(pl + base + i * 16) =
                    *reinterpret_cast<const uint4*>(lds + i * 16);
    } else {
        const int per_row = 1 << (xb - 4);
        for (int i = tid; i < (1 << (TB - 4)); i += 256) {
            const int row = i / per_row, ch = i % per_row;
            *reinterpret_cast<uint4*>(pl + base + ((int64_t)row << lo) + ch * 16) =
                *reinterpret_cast<const uint4*>(lds + i * 16);
        }
    }
}

// ---- merge: Garner CRT, exact 128-bit sum, scaling ------------------------

template <int M>
__global__ void __launch_bounds__(256)
    oz_merge_kernel(double* __restrict__ re, double* __restrict__ im, int n, int64_t groups,
                    const int* __restrict__ exps, int64_t batch,
                    const int8_t* __restrict__ planes, int64_t plane_len, double c, OzConst k)
{
    double* const x = blockIdx.y ? im : re;
    const int* const ex = exps + blockIdx.y * batch;
    const int8_t* const base = planes + (int64_t)blockIdx.y * M * plane_len;
    for (int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x; g < groups;
         g += (int64_t)gridDim.x * 256) {
        const int64_t e0 = g * 8;
        uint64_t res[M];
#pragma unroll
        for (int j = 0; j < M; ++j)
            res[j] = *reinterpret_cast<const uint64_t*>(base + (int64_t)j * plane_len + e0);
        const int sh = ex[e0 >> n] - kOzScaleBits;
        double y[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            // balanced mixed-radix digits: Y = v0 + p0 (v1 + p1 (v2 + ...))
            int v[M];
#pragma unroll
            for (int j = 0; j < M; ++j) {
                int t = (int)(int8_t)(uint8_t)(res[j] >> (8 * i));
#pragma unroll
                for (int a = 0; a < j; ++a)
                    t = reduce_mod((t - v[a]) * (int)k.ginv[a][j], k.p[j], k.inv_pf[j]);
                v[j] = t;
            }
            __int128 Y = v[M - 1];
#pragma unroll
            for (int j = M - 2; j >= 0; --j)
                Y = Y * k.p[j] + v[j];
            const bool neg = Y < 0;
            const unsigned __int128 u = neg ? (unsigned __int128)(-Y) : (unsigned __int128)Y;
            const double d = (double)(uint64_t)(u >> 64) * 18446744073709551616.0 +
                             (double)(uint64_t)u;
            y[i] = ldexp(neg ? -d : d, sh) * c;
        }
        f64x2* const out = reinterpret_cast<f64x2*>(x + e0);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            out[i] = f64x2{y[2 * i], y[2 * i + 1]};
    }
}

unsigned stride_grid(int64_t groups)
{
    const int64_t blocks = (groups + 255) / 256;
    return (unsigned)(blocks < (1 << 20) ? blocks : (1 << 20));
}

int mod_inverse(int a, int p)
{
    int t = 0, nt = 1, r = p, nr = a % p;
    while (nr) {
        const int q = r / nr;
        int tmp = t - q * nt;
        t = nt;
        nt = tmp;
        tmp = r - q * nr;
        r = nr;
        nr = tmp;
    }
    return t < 0 ? t + p : t;
}

}  // namespace

int oz_num_moduli(int n)
{
    // smallest m with prod p_j > 2^(49 + n), tracked in log2 with a margin
    double bits = 0.0;
    for (int j = 0; j < kOzMaxModuli; ++j) {
        bits += std::log2((double)kOzPrimes[j]);
        if (bits > kOzScaleBits + n + 1 + 0.01)
            return j + 1;
    }
    return -1;
}

OzConst oz_constants(int n)
{
    OzConst k{};
    k.m = oz_num_moduli(n);
    for (int j = 0; j < kOzMaxModuli; ++j) {
        k.p[j] = kOzPrimes[j];
        k.inv_pf[j] = 1.0f / (float)kOzPrimes[j];
        k.inv_pd[j] = 1.0 / (double)kOzPrimes[j];
        for (int i = 0; i < j; ++i)
            k.ginv[i][j] = (unsigned char)mod_inverse(kOzPrimes[i], kOzPrimes[j]);
    }
    return k;
}

void oz_pass_plan(int n, OzPass* passes, int* npasses)
{
    const int kt = n < 10 ? n : 10;
    int np = 0;
    passes[np++] = OzPass{1, 0, kt, kOzRowTileBits - kt};
    const int rest = n - kt;
    const int ncol = (rest + 9) / 10;
    int lo = kt;
    for (int i = 0; i < ncol; ++i) {
        const int k = rest / ncol + (i < rest % ncol ? 1 : 0);
        passes[np++] = OzPass{0, lo, k, 9 - k > 6 ? 9 - k : 6};
        lo += k;
    }
    *npasses = np;
}

size_t oz_workspace_layout(int64_t batch, int n, int comps, size_t* off_partial,
                           size_t* off_exps)
{
    const int m = oz_num_moduli(n);
    const size_t plane_len = (size_t)batch << n;
    const int sb = n < kSliceBits ? n : kSliceBits;
    const size_t slices = (size_t)1 << (n - sb);
    size_t off = (size_t)comps * m * plane_len;
    off = (off + 255) & ~(size_t)255;
    *off_partial = off;
    off += (size_t)comps * batch * slices * sizeof(double);
    off = (off + 255) & ~(size_t)255;
    *off_exps = off;
    off += (size_t)comps * batch * sizeof(int);
    return (off + 255) & ~(size_t)255;
}

hipError_t ablation_ozaki(double* re, double* im, int64_t batch, int n, double c, void* ws,
                          hipStream_t stream)
{
    const int comps = im ? 2 : 1;
    const OzConst k = oz_constants(n);
    size_t off_partial, off_exps;
    oz_workspace_layout(batch, n, comps, &off_partial, &off_exps);
    int8_t* const planes = (int8_t*)ws;
    double* const partial = (double*)((char*)ws + off_partial);
    int* const exps = (int*)((char*)ws + off_exps);
    const int64_t plane_len = batch << n;
    const int sb = n < kSliceBits ? n : kSliceBits;
    const int64_t slices = (int64_t)1 << (n - sb);
    hipError_t e;

    const int64_t nslice = batch * slices;
    hipLaunchKernelGGL(oz_max_kernel,
                       dim3((unsigned)(nslice < (1 << 20) ? nslice : (1 << 20)), comps),
                       dim3(256), 0, stream, re, im, n, batch, sb, partial);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    const int64_t vectors = comps * batch;
    hipLaunchKernelGGL(oz_exponent_kernel, dim3((unsigned)((vectors + 255) / 256)), dim3(256), 0,
                       stream, partial, vectors, slices, exps);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    const int64_t groups = plane_len / 8;
    hipLaunchKernelGGL(oz_split_kernel, dim3(stride_grid(groups), comps), dim3(256), 0, stream,
                       re, im, n, groups, exps, batch, planes, plane_len, k);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;

    OzPass ps[4];
    int np = 0;
    oz_pass_plan(n, ps, &np);
    for (int i = 0; i < np; ++i) {
        const OzPass& q = ps[i];
        const int TB = q.kt + q.xb;
        const int pb = q.row ? 0 : q.xb;
        int w[2] = {0, 0}, mask[2] = {0, 0};
        const int nstage = (q.kt + 4) / 5;
        for (int s = 0; s < nstage; ++s) {
            const int a = pb + 5 * s, b = (pb + 5 * s + 5 < pb + q.kt) ? pb + 5 * s + 5 : pb + q.kt;
            w[s] = a < TB - 5 ? a : TB - 5;
            for (int bit = 0; bit < 5; ++bit)
                if (w[s] + bit >= a && w[s] + bit < b)
                    mask[s] |= 1 << bit;
        }
        const int64_t tiles =
            q.row ? (plane_len + ((int64_t)1 << TB) - 1) >> TB : plane_len >> TB;
        const void* fn = q.row ? reinterpret_cast<const void*>(&oz_pass_kernel<true>)
                               : reinterpret_cast<const void*>(&oz_pass_kernel<false>);
        if ((e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     64 * 1024)) != hipSuccess)
            return e;
        for (int64_t t0 = 0; t0 < tiles; t0 += (1 << 20)) {
            const int64_t nt = tiles - t0 < (1 << 20) ? tiles - t0 : (1 << 20);
            if (q.row)
                hipLaunchKernelGGL(oz_pass_kernel<true>, dim3((unsigned)nt, comps * k.m),
                                   dim3(256), (size_t)1 << TB, stream, planes, plane_len, k.m, t0,
                                   q.lo, q.kt, q.xb, nstage, w[0], mask[0], w[1], mask[1], k);
            else
                hipLaunchKernelGGL(oz_pass_kernel<false>, dim3((unsigned)nt, comps * k.m),
                                   dim3(256), (size_t)1 << TB, stream, planes, plane_len, k.m, t0,
                                   q.lo, q.kt, q.xb, nstage, w[0], mask[0], w[1], mask[1], k);
            if ((e = hipGetLastError()) != hipSuccess)
                return e;
        }
    }

    const dim3 grid(stride_grid(groups), comps);
    switch (k.m) {
    case 7: hipLaunchKernelGGL(oz_merge_kernel<7>, grid, dim3(256), 0, stream, re, im, n, groups, exps, batch, planes, plane_len, c, k); break;
    case 8: hipLaunchKernelGGL(oz_merge_kernel<8>, grid, dim3(256), 0, stream, re, im, n, groups, exps, batch, planes, plane_len, c, k); break;
    case 9: hipLaunchKernelGGL(oz_merge_kernel<9>, grid, dim3(256), 0, stream, re, im, n, groups, exps, batch, planes, plane_len, c, k); break;
    case 10: hipLaunchKernelGGL(oz_merge_kernel<10>, grid, dim3(256), 0, stream, re, im, n, groups, exps, batch, planes, plane_len, c, k); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace qse
