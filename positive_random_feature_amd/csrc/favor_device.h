// Device-side building blocks for the gfx950 FAVOR+ kernels.
//
// Matrix-core conventions (v_mfma_f32_16x16x32_bf16, 64-lane wave, lane
// l = 16*g + r with r = l % 16, g = l / 16):
//   A (16 x 32):  lane (r, g) holds A[r][8g + j],     j = 0..7
//   B (32 x 16):  lane (r, g) holds B[8g + j][r]
//   D (16 x 16):  lane (r, g) holds D[4g + i][r],     i = 0..3
// A reduction only needs A and B to agree on which k each (g, j) slot means,
// so every contraction below picks its own k order.  Two D tiles stacked
// along M (rows 0..15 and 16..31) give each lane the 8 rows
// {4g..4g+3, 16+4g..16+4g+3}; that set is used directly as the k slots of the
// next contraction ("kappa order"), which lets a D tile feed the next MFMA
// without any data movement whenever the next MFMA contracts over D's rows.
//
// fp32 operands use the same register layout: a 32-deep contraction is eight
// v_mfma_f32_16x16x4_f32 where step j takes slot j of every lane.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace favor {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();
// Lazy stabiliser threshold (log2 units): a running reference is only raised
// when new exponents exceed it by more than this, so features stay <= 2^kTau.
constexpr float kTau = 8.0f;

template <typename T> struct OperandOf;
template <> struct OperandOf<bf16> { using type = bf16x8; };
template <> struct OperandOf<float> { using type = f8; };
template <typename T> using vec8 = typename OperandOf<T>::type;

__device__ __forceinline__ f4 mma32(bf16x8 a, bf16x8 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f4 mma32(f8 a, f8 b, f4 c) {
#pragma unroll
    for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], c, 0, 0, 0);
    return c;
}

__device__ __forceinline__ f4 f4splat(float x) { return f4{x, x, x, x}; }

// Pack two D tiles' 4-element columns into one 8-slot operand (kappa order).
__device__ __forceinline__ bf16x8 pack8(bf16, f4 lo, f4 hi) {
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r[i] = (bf16)lo[i];
        r[4 + i] = (bf16)hi[i];
    }
    return r;
}
__device__ __forceinline__ f8 pack8(float, f4 lo, f4 hi) {
    f8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r[i] = lo[i];
        r[4 + i] = hi[i];
    }
    return r;
}
template <typename T> __device__ __forceinline__ vec8<T> pack8t(f4 lo, f4 hi) { return pack8(T(), lo, hi); }

template <typename T> __device__ __forceinline__ vec8<T> splat8(float x) {
    vec8<T> r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = (T)x;
    return r;
}
template <typename T> __device__ __forceinline__ vec8<T> zero8() { return splat8<T>(0.0f); }

template <typename T> __device__ __forceinline__ float to_f(T x) { return (float)x; }

// 8 consecutive elements from global memory (16 B for bf16, 32 B for fp32).
__device__ __forceinline__ bf16x8 load8(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ f8 load8(const float* p) {
    const float4* q = reinterpret_cast<const float4*>(p);
    float4 a = q[0], b = q[1];
    return f8{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
}

// Lane exchanges (ds_bpermute through __shfl_xor).
// Sum / max over the four lanes r, r+16, r+32, r+48 (the lanes holding one
// token column in B-operand layout).
__device__ __forceinline__ float col_sum(float x) {
    x += __shfl_xor(x, 16);
    return x + __shfl_xor(x, 32);
}
__device__ __forceinline__ float col_max(float x) {
    x = __builtin_fmaxf(x, __shfl_xor(x, 16));
    return __builtin_fmaxf(x, __shfl_xor(x, 32));
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) x = __builtin_fmaxf(x, __shfl_xor(x, o));
    return col_max(x);
}

__device__ __forceinline__ float exp2f_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Store 4 consecutive output elements.
__device__ __forceinline__ void store4(bf16* p, f4 v) {
    bf16x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = (bf16)v[i];
    *reinterpret_cast<bf16x4*>(p) = r;
}
__device__ __forceinline__ void store4(float* p, f4 v) { *reinterpret_cast<float4*>(p) = float4{v[0], v[1], v[2], v[3]}; }

}  // namespace favor
