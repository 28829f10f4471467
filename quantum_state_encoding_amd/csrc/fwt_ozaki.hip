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
//   residues r_j = X mod p_j (|r| <= 127, int8, four moduli packed in a
//   32-bit word per element), transformed in residue space, then Y
//   rebuilt from the residues by the CRT with a rounded quotient:
//   t_j = r_j (M / p_j)^-1 mod p_j (within p_j / 2 + 1),
//   q = nearest integer to sum_j t_j / p_j (fp64), Y = sum_j t_j M / p_j -
//   q M in 128-bit integers (exact: |Y| / M stays below 1/2 by a margin of
//   at least 0.003, the fp64 quotient errs by under 1e-12), and
//   y_k = Y_k * 2^(e_b - 48) * c.
// Integer-valued inputs are transformed exactly.  Otherwise the error is
// that of rounding X: at most 2^(2 - 48) of max |x| per output times
// sqrt(2^n) (normalised), far inside fp64 tolerances.
//
// Kernels: per-slice maxima -> per-vector exponents -> split into residue
// words -> Kronecker passes over the words (32-position blocks on
// v_mfma_i32_16x16x32_i8) -> merge (CRT + scaling).  The residues live in a
// caller-provided workspace.
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

// ---- split into residue words ----------------------------------------------
//
// Residues are stored four moduli to a 32-bit word (byte q of word group g
// holds the residue mod p_(4g+q); slots past m stay zero): word group g of
// component c starts at words + (c * G + g) * plane_len.  Thread i takes 8
// consecutive elements of one component.

__global__ void __launch_bounds__(256)
    oz_split_kernel(const double* __restrict__ re, const double* __restrict__ im, int n,
                    int64_t groups, const int* __restrict__ exps, int64_t batch,
                    uint32_t* __restrict__ words, int64_t plane_len, OzConst k)
{
    const double* const x = blockIdx.y ? im : re;
    const int* const ex = exps + blockIdx.y * batch;
    const int G = (k.m + kOzPack - 1) / kOzPack;
    uint32_t* const base = words + (int64_t)blockIdx.y * G * plane_len;
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
        for (int grp = 0; grp < G; ++grp) {
            uint32_t w[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
            for (int q = 0; q < kOzPack; ++q) {
                const int j = kOzPack * grp + q;
                if (j >= k.m)
                    break;
                const double p = (double)k.p[j];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    // X - p * nearest(X / p) is exact (|X| <= 2^48); |r| <= (p + 1) / 2
                    const double r = fma(-p, rint(X[i] * k.inv_pd[j]), X[i]);
                    w[i] |= (uint32_t)(uint8_t)(int8_t)(int)r << (8 * q);
                }
            }
            uint4* const out = reinterpret_cast<uint4*>(base + (int64_t)grp * plane_len + e0);
            out[0] = make_uint4(w[0], w[1], w[2], w[3]);
            out[1] = make_uint4(w[4], w[5], w[6], w[7]);
        }
    }
}

// ---- Kronecker passes over the residue words --------------------------------
//
// A workgroup owns one tile of 2^TB residue words (4 moduli each) of one
// word group in LDS.  Tile index t:
//   ROW (bits [0, kt)):  t = line << kt | position, 2^TB contiguous words;
//   COL (bits [lo, lo + kt)): t = position << cb | column, 2^kt rows of
//     2^cb contiguous words at stride 2^lo.
// Each stage transforms up to 5 tile-index bits inside a 5-bit window at w
// (`mask` marks which window bits to transform; the others are identity).
// Sixteen "lines" (the tile-index bits outside the window) at a time form
// the B operands of v_mfma_i32_16x16x32_i8, one per modulus (lane l: line
// l mod 16, positions 8 (l / 16) .. + 7, one byte each, cut out of the
// lane's 8 words by a 4 x 4 byte transpose), and two 16 x 32 slabs of the
// window matrix M[o][k] = [(o ^ k) & ~mask = 0] (-1)^popcount(o & k & mask)
// form A (lane l: output l mod 16, positions 8 (l / 16) .. + 7).  Result
// register r of lane l is output 4 (l / 16) + r of line l mod 16; reduced
// mod p and packed again four moduli to a word, it is written over the
// line.

__device__ __forceinline__ int window_addr(int lam, int k, int w)
{
    return ((lam >> w) << (w + 5)) | (k << w) | (lam & ((1 << w) - 1));
}

// d - p * q with q the integer nearest to d / p up to 0.015: for |d| <=
// 31500 the result is congruent to d and within p / 2 + 1 of zero (so an
// int8 for p <= 251), in three full-rate 24-bit integer operations.
__device__ __forceinline__ int reduce_mod(int d, int p, int magic)
{
    const int q = (__mul24(d, magic) + (1 << 19)) >> 20;
    return d - __mul24(q, p);
}

// o[q] = byte q of d[0], d[1], d[2], d[3] (in that byte order)
__device__ __forceinline__ void transpose4(const uint32_t* d, uint32_t* o)
{
#pragma unroll
    for (int q = 0; q < 4; ++q)
        o[q] = ((d[0] >> (8 * q)) & 0xFFu) | (((d[1] >> (8 * q)) & 0xFFu) << 8) |
               (((d[2] >> (8 * q)) & 0xFFu) << 16) | (((d[3] >> (8 * q)) & 0xFFu) << 24);
}

// At most 64 VGPRs (8 waves per SIMD): the stages cannot overlap a
// workgroup's own loads, so other workgroups have to.
template <bool ROW>
__global__ void __launch_bounds__(256, 8)
    oz_pass_kernel(uint32_t* __restrict__ words, int64_t plane_len, int G, int64_t tile0, int lo,
                   int kt, int xb, int nstage, int w0, int mask0, int w1, int mask1, OzConst k)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
    uint32_t* const lds = reinterpret_cast<uint32_t*>(lds_raw);
    const int TB = kt + xb;
    const int grp = blockIdx.y % G;
    int p[kOzPack], magic[kOzPack];
#pragma unroll
    for (int q = 0; q < kOzPack; ++q) {
        p[q] = k.p[kOzPack * grp + q];
        magic[q] = k.magic[kOzPack * grp + q];
    }
    uint32_t* const pl = words + (int64_t)blockIdx.y * plane_len;
    const int64_t tile = tile0 + blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    // load (16-byte chunks of 4 words)
    int64_t base;
    int64_t valid = (int64_t)1 << TB;   // ROW: words of this tile inside the plane
    if (ROW) {
        base = tile << TB;
        const int64_t left = plane_len - base;
        if (left < valid)
            valid = left;
        for (int i = tid; i < (1 << (TB - 2)); i += 256) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (i * 4 < valid)
                v = *reinterpret_cast<const uint4*>(pl + base + i * 4);
            *reinterpret_cast<uint4*>(lds + i * 4) = v;
        }
    } else {
        const int cb = xb;
        const int64_t cblk = tile & (((int64_t)1 << (lo - cb)) - 1);
        const int64_t outer = tile >> (lo - cb);
        base = (outer << (kt + lo)) | (cblk << cb);
        const int per_row = 1 << (cb - 2);
        for (int i = tid; i < (1 << (TB - 2)); i += 256) {
            const int row = i / per_row, ch = i % per_row;
            *reinterpret_cast<uint4*>(lds + i * 4) =
                *reinterpret_cast<const uint4*>(pl + base + ((int64_t)row << lo) + ch * 4);
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
            uint32_t d[8], lo4[4], hi4[4];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                d[j] = lds[window_addr(lam, 8 * (lane >> 4) + j, w)];
            transpose4(d, lo4);
            transpose4(d + 4, hi4);
            i32x4 acc[kOzPack][2];
            const i32x4 zero = {0, 0, 0, 0};
#pragma unroll
            for (int q = 0; q < kOzPack; ++q) {
                const long b = (long)(((uint64_t)hi4[q] << 32) | lo4[q]);
                acc[q][0] = __builtin_amdgcn_mfma_i32_16x16x32_i8(a[0], b, zero, 0, 0, 0);
                acc[q][1] = __builtin_amdgcn_mfma_i32_16x16x32_i8(a[1], b, zero, 0, 0, 0);
            }
            // every lane's operand words are in registers before any write
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                uint32_t v0 = 0, v1 = 0;
#pragma unroll
                for (int q = 0; q < kOzPack; ++q) {
                    v0 |= (uint32_t)(uint8_t)(int8_t)reduce_mod(acc[q][0][r], p[q], magic[q])
                          << (8 * q);
                    v1 |= (uint32_t)(uint8_t)(int8_t)reduce_mod(acc[q][1][r], p[q], magic[q])
                          << (8 * q);
                }
                const int o = 4 * (lane >> 4) + r;
                lds[window_addr(lam, o, w)] = v0;
                lds[window_addr(lam, o + 16, w)] = v1;
            }
        }
        __syncthreads();
    }

    if (ROW) {
        for (int i = tid; i < (1 << (TB - 2)); i += 256)
            if (i * 4 < valid)
                *reinterpret_cast<uint4*>(pl + base + i * 4) =
                    *reinterpret_cast<const uint4*>(lds + i * 4);
    } else {
        const int per_row = 1 << (xb - 2);
        for (int i = tid; i < (1 << (TB - 2)); i += 256) {
            const int row = i / per_row, ch = i % per_row;
            *reinterpret_cast<uint4*>(pl + base + ((int64_t)row << lo) + ch * 4) =
                *reinterpret_cast<const uint4*>(lds + i * 4);
        }
    }
}

// ---- merge: CRT with a rounded quotient, exact 128-bit sum, scaling --------

template <int M>
__global__ void __launch_bounds__(256)
    oz_merge_kernel(double* __restrict__ re, double* __restrict__ im, int n, int64_t groups,
                    const int* __restrict__ exps, int64_t batch,
                    const uint32_t* __restrict__ words, int64_t plane_len, double c, OzConst k)
{
    constexpr int G = (M + kOzPack - 1) / kOzPack;
    double* const x = blockIdx.y ? im : re;
    const int* const ex = exps + blockIdx.y * batch;
    const uint32_t* const base = words + (int64_t)blockIdx.y * G * plane_len;
    for (int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x; g < groups;
         g += (int64_t)gridDim.x * 256) {
        const int64_t e0 = g * 8;
        uint32_t res[G][8];
#pragma unroll
        for (int grp = 0; grp < G; ++grp) {
            const uint4* const in =
                reinterpret_cast<const uint4*>(base + (int64_t)grp * plane_len + e0);
            const uint4 u0 = in[0], u1 = in[1];
            res[grp][0] = u0.x; res[grp][1] = u0.y; res[grp][2] = u0.z; res[grp][3] = u0.w;
            res[grp][4] = u1.x; res[grp][5] = u1.y; res[grp][6] = u1.z; res[grp][7] = u1.w;
        }
        const int sh = ex[e0 >> n] - kOzScaleBits;
        double y[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            // sum_j t_j (M / p_j) - q M in three 32-bit limbs with int64
            // accumulators (|t_j| <= 125, limbs < 2^32: no overflow)
            int64_t a0 = 0, a1 = 0, a2 = 0;
            double f = 0.0;
#pragma unroll
            for (int j = 0; j < M; ++j) {
                const int r = (int)(int8_t)(uint8_t)(res[j / kOzPack][i] >> (8 * (j % kOzPack)));
                const int t = reduce_mod(r * k.crt_c[j], k.p[j], k.magic[j]);
                f = fma((double)t, k.inv_pd[j], f);
                a0 += (int64_t)t * (uint32_t)k.crt_lo[j];
                a1 += (int64_t)t * (uint32_t)(k.crt_lo[j] >> 32);
                a2 += (int64_t)t * (int64_t)k.crt_hi[j];
            }
            const int64_t q = (int64_t)rint(f);
            a0 -= q * (int64_t)(uint32_t)k.m_lo;
            a1 -= q * (int64_t)(uint32_t)(k.m_lo >> 32);
            a2 -= q * (int64_t)k.m_hi;
            const __int128 Y = (__int128)a0 + ((__int128)a1 << 32) + ((__int128)a2 << 64);
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
    unsigned __int128 M = 1;
    for (int j = 0; j < k.m; ++j)
        M *= (unsigned)kOzPrimes[j];
    k.m_lo = (uint64_t)M;
    k.m_hi = (uint64_t)(M >> 64);
    for (int j = 0; j < kOzMaxModuli; ++j) {
        k.p[j] = kOzPrimes[j];
        k.magic[j] = (int)((1 << 20) / (double)kOzPrimes[j] + 0.5);
        k.inv_pd[j] = 1.0 / (double)kOzPrimes[j];
        if (j < k.m) {
            const unsigned __int128 cj = M / (unsigned)kOzPrimes[j];
            k.crt_lo[j] = (uint64_t)cj;
            k.crt_hi[j] = (uint64_t)(cj >> 64);
            k.crt_c[j] = mod_inverse((int)(cj % (unsigned)kOzPrimes[j]), kOzPrimes[j]);
        }
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
        // 128-byte row segments (32 words) while the tile stays <= 64 KiB,
        // and at least 2^9 words per tile
        int cb = k <= 9 ? 5 : 4;
        if (k + cb < 9)
            cb = 9 - k;
        passes[np++] = OzPass{0, lo, k, cb};
        lo += k;
    }
    *npasses = np;
}

size_t oz_workspace_layout(int64_t batch, int n, int comps, size_t* off_partial,
                           size_t* off_exps)
{
    const int G = (oz_num_moduli(n) + kOzPack - 1) / kOzPack;
    const size_t plane_len = (size_t)batch << n;
    const int sb = n < kSliceBits ? n : kSliceBits;
    const size_t slices = (size_t)1 << (n - sb);
    size_t off = (size_t)comps * G * plane_len * sizeof(uint32_t);
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
    uint32_t* const words = (uint32_t*)ws;
    const int G = (k.m + kOzPack - 1) / kOzPack;
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
                       re, im, n, groups, exps, batch, words, plane_len, k);
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
            const size_t lds = sizeof(uint32_t) << TB;
            if (q.row)
                hipLaunchKernelGGL(oz_pass_kernel<true>, dim3((unsigned)nt, comps * G), dim3(256),
                                   lds, stream, words, plane_len, G, t0, q.lo, q.kt, q.xb, nstage,
                                   w[0], mask[0], w[1], mask[1], k);
            else
                hipLaunchKernelGGL(oz_pass_kernel<false>, dim3((unsigned)nt, comps * G), dim3(256),
                                   lds, stream, words, plane_len, G, t0, q.lo, q.kt, q.xb, nstage,
                                   w[0], mask[0], w[1], mask[1], k);
            if ((e = hipGetLastError()) != hipSuccess)
                return e;
        }
    }

    // The merge kernel is compiled per modulus count (7..10).
    decltype(&oz_merge_kernel<7>) merge;
    switch (k.m) {
    case 7: merge = &oz_merge_kernel<7>; break;
    case 8: merge = &oz_merge_kernel<8>; break;
    case 9: merge = &oz_merge_kernel<9>; break;
    case 10: merge = &oz_merge_kernel<10>; break;
    default: return hipErrorInvalidValue;
    }
    hipLaunchKernelGGL(merge, dim3(stride_grid(groups), comps), dim3(256), 0, stream, re, im, n,
                       groups, exps, batch, words, plane_len, c, k);
    return hipGetLastError();
}

}  // namespace qse
