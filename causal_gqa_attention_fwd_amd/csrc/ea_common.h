// ea_common.h -- device-side building blocks shared by the libeuler_attn kernels (gfx950).
//
// MFMA operand layouts used throughout (64-lane wavefront, lane l, half h = l >> 5):
//  * v_mfma_f32_32x32x16_bf16 (bf16) and v_mfma_f32_32x32x2_f32 (fp32) both compute a
//    32 x 32 fp32 tile C += A * B.  A lane supplies row (l & 31) of A and column (l & 31)
//    of B, KPL contraction elements each (8 for bf16, 1 for fp32).  Which contraction
//    index a (half, element) slot carries is our choice, as long as A and B agree.
//  * C: lane l holds column (l & 31); its register r (0..15) holds row
//    acc_row(r, h) = 8 * (r / 4) + 4 * h + (r % 4).
//
// Two contraction mappings are used:
//  * "split" (over a contiguous dimension of length L, e.g. head_dim): instruction s, half
//    h, element e  <->  index h * L/2 + s * KPL + e.  A lane's elements are one contiguous
//    run of L/2, so its operand is read with wide loads.
//  * "accumulator" (over the 32 rows of a C tile reused as an operand): instruction s,
//    half h, element e  <->  register r = s * KPL + e  <->  row acc_row(r, h).  The partner
//    operand is read from a row-major LDS tile whose rows are the contraction index with
//    load_rows_frag: for bf16, two ds_read_b64_tr_b16 transposing reads (each 16-lane group
//    reads a 4-row x 16-column block and every lane receives one column); for fp32, one
//    dword per instruction.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <climits>
#include <cmath>
#include <type_traits>

namespace ea {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <typename T>
struct Mfma;

template <>
struct Mfma<float> {
    typedef float frag;
    static constexpr int KPL = 1;
    __device__ static inline f32x16 mma(frag a, frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
};

template <>
struct Mfma<bf16> {
    typedef bf16x8 frag;
    static constexpr int KPL = 8;
    __device__ static inline f32x16 mma(frag a, frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};

// Row of a 32x32 accumulator held by register r of a lane in half h.
__device__ __host__ constexpr inline int acc_row(int r, int h) {
    return 8 * (r >> 2) + 4 * h + (r & 3);
}

// LDS slot of row k (0..31) of an accumulator-ordered operand: 16 * half + register.
__device__ __host__ constexpr inline int acc_slot(int k) {
    return 16 * ((k >> 2) & 1) + 4 * (k >> 3) + (k & 3);
}

// Fragment load of KPL contiguous elements from LDS or global memory.
template <typename T>
__device__ inline typename Mfma<T>::frag load_frag(const T* p);

template <>
__device__ inline float load_frag<float>(const float* p) {
    return *p;
}

template <>
__device__ inline bf16x8 load_frag<bf16>(const bf16* p) {
    return *reinterpret_cast<const bf16x8*>(p);
}

// Convert fp32 values (registers r0 .. r0+KPL-1 of an accumulator) into an operand fragment.
template <typename T>
__device__ inline typename Mfma<T>::frag acc_to_frag(const f32x16& c, int r0);

template <>
__device__ inline float acc_to_frag<float>(const f32x16& c, int r0) {
    return c[r0];
}

template <>
__device__ inline bf16x8 acc_to_frag<bf16>(const f32x16& c, int r0) {
    bf16x8 f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = (bf16)c[r0 + e];  // round to nearest even
    return f;
}

// Operand fragment for a contraction over 32 "accumulator"-ordered rows of a row-major LDS
// tile (row = contraction index, column = this lane's MFMA row or column):
//   lane l, half h = l >> 5, element e of instruction ps  <-  tile[row0 + acc_row(ps*KPL + e, h)]
//                                                               [col0 + (l & 31)].
template <typename T>
__device__ inline typename Mfma<T>::frag load_rows_frag(const T* tile, int stride, int row0,
                                                        int ps, int col0);

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

template <>
__device__ inline bf16x8 load_rows_frag<bf16>(const bf16* tile, int stride, int row0, int ps,
                                             int col0) {
    // ds_read_b64_tr_b16: within each group of 16 lanes, lane j supplies the address of a
    // 4-element chunk C_j; lane i receives C_{4e + i/4}[i % 4] as element e.  Lane j points
    // at row (4h + j/4) and columns 16*grp + 4*(j%4) .. +3, so lane i gets column 16*grp + i
    // of rows 4h + 0..3 (first read) and 8 + 4h + 0..3 (second read): exactly
    // acc_row(8*ps + e, h) for e = 0..7.
    const int lane = __lane_id();
    const int h = lane >> 5, grp = (lane >> 4) & 1, j = lane & 15;
    const bf16* p = tile + (row0 + 16 * ps + 4 * h + (j >> 2)) * stride + col0 + 16 * grp + 4 * (j & 3);
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 8 * stride));
    bf16x8 f;
    const bf16x4 a = __builtin_bit_cast(bf16x4, lo);
    const bf16x4 b = __builtin_bit_cast(bf16x4, hi);
    f[0] = a[0]; f[1] = a[1]; f[2] = a[2]; f[3] = a[3];
    f[4] = b[0]; f[5] = b[1]; f[6] = b[2]; f[7] = b[3];
    return f;
}

template <>
__device__ inline float load_rows_frag<float>(const float* tile, int stride, int row0, int ps,
                                             int col0) {
    const int lane = __lane_id();
    return tile[(row0 + acc_row(ps, lane >> 5)) * stride + col0 + (lane & 31)];
}

template <typename T>
__device__ inline float to_f32(T x) {
    return (float)x;
}

template <typename T>
__device__ inline T from_f32(float x) {
    return (T)x;
}

// 16-byte vector of I/O elements.
template <typename T>
struct Vec16 {
    static constexpr int N = 16 / sizeof(T);
    u32x4 raw;
    __device__ inline T get(int i) const {
        return reinterpret_cast<const T*>(&raw)[i];
    }
    __device__ inline void set(int i, T v) {
        reinterpret_cast<T*>(&raw)[i] = v;
    }
};

// Loads issued before a loop and first used inside it: the compiler's wait-count insertion
// cannot tell, inside the loop, whether such a load is still in flight, so it waits for every
// outstanding load (the loop's own prefetches included) at that first use, in every
// iteration.  settle(x) consumes x once at the call site, so the wait happens there, once.
template <typename T>
__device__ inline void settle(T& x) {
    asm volatile("" : "+v"(x));
}

template <typename T>
__device__ inline Vec16<T> ld16(const T* p) {
    Vec16<T> v;
    v.raw = *reinterpret_cast<const u32x4*>(p);
    return v;
}

template <typename T>
__device__ inline void st16(T* p, const Vec16<T>& v) {
    *reinterpret_cast<u32x4*>(p) = v.raw;
}

template <typename T>
__device__ inline Vec16<T> zero16() {
    Vec16<T> v;
    v.raw = u32x4{0u, 0u, 0u, 0u};
    return v;
}

__device__ inline f32x16 zero_acc() {
    f32x16 z;
#pragma unroll
    for (int r = 0; r < 16; ++r) z[r] = 0.0f;
    return z;
}

// Max and sum of x over the lane pair (l, l ^ 32), returned in both lanes: one
// v_permlane32_swap (the two 32-lane halves exchange x) and one VALU op, no LDS round trip.
// The swap leaves lane l < 32 with (x[l], x[l + 32]) and lane l >= 32 with (x[l - 32], x[l]),
// so both lanes of a pair combine the same two values in the same order.
__device__ inline float half_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ inline float half_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum of x over each aligned group of W lanes (W = 1, 2, 4, ..., 64) as a butterfly: partners
// one lane apart are added first, then two, four, ...  Every lane of a group ends with the same
// bits, and so does any code that adds the same W values pairwise in that order, across lanes
// or within one lane (floating-point addition is commutative).  Up to 16 lanes the exchanges
// are DPP lane permutations (quad permutes, then the mirror of 8 and of 16 lanes, which after
// the earlier levels hold the same value as the xor partner), so they cost no LDS access.
template <int W>
__device__ inline float group_sum(float x) {
    static_assert(W >= 1 && W <= 64 && (W & (W - 1)) == 0, "group width");
    auto dpp = [](float v, auto ctrl) {
        return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), decltype(ctrl)::value, 0xF, 0xF, true));
    };
    if constexpr (W >= 2) x += dpp(x, std::integral_constant<int, 0xB1>{});   // quad_perm 1,0,3,2
    if constexpr (W >= 4) x += dpp(x, std::integral_constant<int, 0x4E>{});   // quad_perm 2,3,0,1
    if constexpr (W >= 8) x += dpp(x, std::integral_constant<int, 0x141>{});  // row_half_mirror
    if constexpr (W >= 16) x += dpp(x, std::integral_constant<int, 0x140>{}); // row_mirror
    if constexpr (W >= 32) x += __shfl_xor(x, 16, 64);
    if constexpr (W >= 64) x = half_sum(x);
    return x;
}

// Dot product of two 16-byte chunks: one fused multiply-add per element, in element order,
// starting from zero.
template <typename T>
__device__ inline float dot16(const Vec16<T>& a, const Vec16<T>& b) {
    float acc = 0.0f;
#pragma unroll
    for (int e = 0; e < Vec16<T>::N; ++e) acc = __builtin_fmaf(to_f32(a.get(e)), to_f32(b.get(e)), acc);
    return acc;
}

// RoPE frequencies theta_i = base^(-2i/D), i < D/2 <= 128, computed on the host in double
// and passed by value to the kernels that rotate.
struct RopeFreq {
    double theta[128];
};

inline void fill_rope_freq(RopeFreq* f, int D, double base) {
    for (int i = 0; i < 128; ++i) f->theta[i] = (i < D / 2) ? pow(base, -2.0 * (double)i / (double)D) : 0.0;
}

// cos and sin of the RoPE angle phi = pos * theta: phi is formed and reduced modulo 2*pi in
// double (two-term 2*pi), and the reduced angle, |r| <= pi, goes to the hardware sine and
// cosine (v_sin_f32 / v_cos_f32, which take the angle in revolutions: x = r / (2 pi), formed
// in double, |x| <= 1/2).  Measured against the float64 oracle, the rotated values carry the
// same error as with the library sincosf of the reduced angle (fp32 rounding of the product).
__device__ inline void rope_cos_sin(double pos, double theta, float* c, float* s) {
    constexpr double kTwoPiHi = 6.283185307179586;       // nearest double to 2*pi
    constexpr double kTwoPiLo = 2.4492935982947064e-16;  // 2*pi - kTwoPiHi
    constexpr double kInvTwoPi = 0.15915494309189535;
    const double phi = pos * theta;
    const double n = rint(phi * kInvTwoPi);
    double r = fma(-n, kTwoPiHi, phi);
    r = fma(-n, kTwoPiLo, r);
    const float x = (float)(r * kInvTwoPi);
    *s = __builtin_amdgcn_sinf(x);
    *c = __builtin_amdgcn_cosf(x);
}

// Rotation of one RoPE pair (x0, x1) by the angle with cosine c and sine s:
//   y0 = x0 c - x1 s,   y1 = x0 s + x1 c.
// The evaluation order is fixed (one product, then one fused multiply-add per output), so
// every kernel that rotates a pair rounds it the same way whatever the compiler would have
// contracted; the inverse rotation passes -s.
__device__ inline void rope_rotate(float x0, float x1, float c, float s, float* y0, float* y1) {
    *y0 = __builtin_fmaf(x0, c, -(x1 * s));
    *y1 = __builtin_fmaf(x0, s, x1 * c);
}

}  // namespace ea
