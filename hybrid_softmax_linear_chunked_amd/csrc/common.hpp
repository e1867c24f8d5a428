// common.hpp -- shared device helpers for the gfx950 (CDNA4) ReHyAt kernels.
//
// Matrix-core conventions used by every kernel (32x32 MFMA tiles, wave64):
//   lane l = 32*h + col, h in {0,1}
//   A operand (M x K): lane holds row m = col and EPL consecutive contraction slots
//                      h*EPL .. h*EPL+EPL-1 of the instruction's K range.
//   B operand (K x N): lane holds column n = col and the same slots.
//   C/D (32x32 fp32, 16 registers): lane holds column n = col; register r holds row
//                      crow(r, h) = (r/4)*8 + h*4 + (r%4).
// A product only pairs slot (h, e) of A with slot (h, e) of B, so a contraction index can
// be assigned to slots in any order as long as both operands use the same assignment.
// This lets a C tile (one lane per output column, 16 rows in registers) be fed straight
// back as the B operand of the next product: register r of lane-half h becomes slot
// (h, r % EPL) of instruction r / EPL, i.e. contraction index crow(r, h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rehyat {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

template <class T>
struct Mfma;

// v_mfma_f32_32x32x16_bf16: 32x32 output, contraction 16 per instruction, 8 bf16 per lane.
template <>
struct Mfma<bf16> {
    static constexpr int KS = 16;
    static constexpr int EPL = 8;
    using frag = bf16x8;
    __device__ static inline f32x16 mma(frag a, frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    __device__ static inline frag load(const bf16* p) { return *reinterpret_cast<const frag*>(p); }
    // 8 fp32 values -> operand (round to nearest even)
    __device__ static inline frag pack(const float* x) {
        frag f;
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = (bf16)x[e];
        return f;
    }
};

// v_mfma_f32_32x32x2_f32: contraction 2 per instruction, one fp32 per lane.
template <>
struct Mfma<float> {
    static constexpr int KS = 2;
    static constexpr int EPL = 1;
    using frag = float;
    __device__ static inline f32x16 mma(frag a, frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
    __device__ static inline frag load(const float* p) { return *p; }
    __device__ static inline frag pack(const float* x) { return x[0]; }
};

__host__ __device__ constexpr int crow(int r, int h) { return (r / 4) * 8 + h * 4 + (r % 4); }

// Position of contraction index kk (0..31 within a 32-block) in "slot order": the order
// in which a lane reads EPL consecutive elements for instruction t, lane-half h.
template <int EPL>
__host__ __device__ constexpr int slot_pos(int kk) {
    int r = (kk / 8) * 4 + (kk % 4);
    int h = (kk / 4) % 2;
    return (r / EPL) * 2 * EPL + h * EPL + (r % EPL);
}

__device__ inline f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.f;
    return z;
}

// Feature index of phi entry (j, power pw) -- ReHyAt blog section 2.2.2: u is split into
// P contiguous parts (the first Dphi mod P parts one longer), part pi contributes
// [u_pi^1 | .. | u_pi^P], parts concatenated in order.
__host__ __device__ inline int feat_index(int j, int pw, int Dphi, int P) {
    const int q = Dphi / P, r = Dphi % P;
    int part, start;
    if (j < r * (q + 1)) {
        part = j / (q + 1);
        start = part * (q + 1);
    } else {
        part = r + (j - r * (q + 1)) / q;
        start = r * (q + 1) + (part - r) * q;
    }
    const int len = q + (part < r ? 1 : 0);
    return P * start + (pw - 1) * len + (j - start);
}

// Inverse of feat_index: feature f -> (j, power).
__host__ __device__ inline void feat_split(int f, int Dphi, int P, int& j, int& pw) {
    const int q = Dphi / P, r = Dphi % P;
    int start = 0;
    for (int part = 0; part < P; ++part) {
        const int len = q + (part < r ? 1 : 0);
        if (f < P * (start + len)) {
            const int off = f - P * start;
            pw = off / len + 1;
            j = start + off % len;
            return;
        }
        start += len;
    }
    j = 0;
    pw = 1;
}

// softplus(x) = log(1 + e^x), split so neither term overflows.
__device__ inline float softplus(float x) { return fmaxf(x, 0.f) + log1pf(__expf(-fabsf(x))); }

// softplus for the bf16 path: the same split with the hardware base-2 exp and log
// (v_exp_f32, v_log_f32).  The error of log2(1 + e) near 1 is far below the bf16 rounding
// the features get before their product; fp32 inputs keep the log1p form.
template <class T>
__device__ inline float softplus_fast(float x) {
    if constexpr (sizeof(T) == 2) {
        const float e = __builtin_amdgcn_exp2f(-fabsf(x) * 1.4426950408889634f);
        return fmaxf(x, 0.f) + __builtin_amdgcn_logf(1.f + e) * 0.6931471805599453f;
    } else {
        return softplus(x);
    }
}

// Exchange with the lane 32 positions away (the other half of the wave).
__device__ inline float other_half(float x) { return __shfl_xor(x, 32); }

// max(x[l], x[l ^ 32]) for every lane l, on the VALU: v_permlane32_swap exchanges the upper
// half of its first operand with the lower half of its second, so with both operands = x
// the two results hold x[l % 32] and x[32 + l % 32].
__device__ inline float pair_max(float x) {
    const int xi = __float_as_int(x);
    const auto r = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
    return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}

template <class T>
__device__ inline T from_float(float x);
template <>
__device__ inline float from_float<float>(float x) { return x; }
template <>
__device__ inline bf16 from_float<bf16>(float x) { return (bf16)x; }

}  // namespace rehyat
