// Device helpers shared by the transform kernels (fwt_kernels.hip,
// fwt_onepass.hip): 16-byte vector types, butterflies, stages on register
// bits, and stages on lane bits across a wave64.  Internal; not installed.
//
// A stage on lane bit b pairs lane l with lane l ^ 2^b.  Lane bits 0 and 1
// cross with DPP quad permutes, 2 and 3 with ds_swizzle (bit 3 with a DPP
// row rotation instead, and bit 2 with a DPP row half-mirror in mirrored
// row tiles), and 4 and 5 with v_permlane16/32_swap, which exchange a lane
// bit with a register bit so the stage becomes a register butterfly (and a
// second swap restores the layout).  Lanes keep their own half of each pair
// with y = partner + s * x, s = +1 for the lower index and -1 for the
// upper: one rounding, exactly the sum or difference.  (fp32 stages on lane
// bits 0, 1 and 3 keep x + s * partner instead, the difference negated,
// and the kernel's final scaling removes the sign: fmac_dpp_regs.)
#pragma once

#include <hip/hip_runtime.h>

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

}  // namespace
}  // namespace qse
