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

// compile-time integer, to pick a specialised code path from a run-time value
template <int N> struct IntC { static constexpr int value = N; };

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

// Sum of squares of 8 elements: bf16 pairs through v_dot2c_f32_bf16 (the
// products of bf16 values are exact in fp32), fp32 through fused multiply-adds.
__device__ __forceinline__ float sumsq8(bf16x8 x) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
        const bf16x2 p{x[j], x[j + 1]};
        s = __builtin_amdgcn_fdot2_f32_bf16(p, p, s, false);
    }
    return s;
}
__device__ __forceinline__ float sumsq8(f8 x) {
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) s += x[j] * x[j];
    return s;
}

// 8 consecutive elements from global memory (16 B for bf16, 32 B for fp32).
__device__ __forceinline__ bf16x8 load8(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ f8 load8(const float* p) {
    const float4* q = reinterpret_cast<const float4*>(p);
    float4 a = q[0], b = q[1];
    return f8{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
}

// The same loads through an explicitly global pointer: when a pointer's
// address space cannot be inferred (e.g. picked from an array at run time)
// the compiler emits flat loads, which also count against the LDS wait
// counter and so serialise with every later LDS access.
typedef __attribute__((address_space(1))) const bf16x8 gbf16x8;
typedef __attribute__((address_space(1))) const f4 gf4;
__device__ __forceinline__ bf16x8 gload8(const bf16* p) { return *(gbf16x8*)(p); }
__device__ __forceinline__ f8 gload8(const float* p) {
    const f4 a = ((gf4*)(p))[0], b = ((gf4*)(p))[1];
    return f8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

template <typename V> __device__ __forceinline__ V gload_vec(const V* p) {
    return *(__attribute__((address_space(1))) const V*)(p);
}

// Workgroup copy of n 16-byte vectors from global memory straight into LDS
// (global_load_lds_dwordx4: no registers, every load of every thread in
// flight at once).  Each wave instruction fills 1 KB of consecutive LDS from
// a wave-uniform base (the lane offset is implicit).  The data is in LDS only
// after lds_dma_wait() and a barrier.
template <int NTHR, typename V>
__device__ __forceinline__ void copy_to_lds_async(V* dst, const V* src, int n) {
    static_assert(sizeof(V) % 16 == 0, "16-byte vectors");
    constexpr int P = sizeof(V) / 16;  // 16-byte pieces per vector
    typedef __attribute__((address_space(3))) void* lds_ptr;
    const int n16 = n * P;
    const int lane = threadIdx.x & 63;
    const char* s8 = reinterpret_cast<const char*>(src);
    char* d8 = reinterpret_cast<char*>(dst);
    for (int e = threadIdx.x; e < n16; e += NTHR)
        __builtin_amdgcn_global_load_lds(s8 + 16 * (size_t)e, (lds_ptr)(d8 + 16 * (size_t)(e - lane)), 16, 0, 0);
}
// Completion of this thread's LDS-direct loads (and of everything else it
// has outstanding).
__device__ __forceinline__ void lds_dma_wait() { __builtin_amdgcn_s_waitcnt(0); }

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

// DPP lane permutations inside rows of 16 lanes (no LDS traffic).  Every
// permutation used here gives each lane a valid source lane, so the
// out-of-range value (bound_ctrl: zero) never appears; with no old value to
// keep, the compiler folds the permutation into the instruction that uses it
// (one v_add_f32_dpp / v_max_f32_dpp instead of a copy, a move and the op).
template <int CTRL> __device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7 - i within 8 lanes
constexpr int kDppMirror = 0x140;      // lane i <-> 15 - i within 16 lanes

// Sum over N consecutive lanes (N = 2, 4, 8, 16; groups aligned to N); every
// lane of a group gets the group's sum.
template <int N> __device__ __forceinline__ float group_sum(float x) {
    if (N >= 2) x += dpp<kDppXor1>(x);
    if (N >= 4) x += dpp<kDppXor2>(x);
    if (N >= 8) x += dpp<kDppHalfMirror>(x);
    if (N >= 16) x += dpp<kDppMirror>(x);
    return x;
}

// Max over the whole wave, uniform result (rows reduced with DPP, then the
// four row results combined through scalar reads).
__device__ __forceinline__ float wave_max_uniform(float x) {
    x = __builtin_fmaxf(x, dpp<kDppXor1>(x));
    x = __builtin_fmaxf(x, dpp<kDppXor2>(x));
    x = __builtin_fmaxf(x, dpp<kDppHalfMirror>(x));
    x = __builtin_fmaxf(x, dpp<kDppMirror>(x));
    const float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 0));
    const float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 16));
    const float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 32));
    const float d = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 48));
    return __builtin_fmaxf(__builtin_fmaxf(a, b), __builtin_fmaxf(c, d));
}

__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) x = __builtin_fmaxf(x, __shfl_xor(x, o));
    return col_max(x);
}

__device__ __forceinline__ float exp2f_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Feature nonlinearity applied to a projected value: 2^x for the positive
// (softmax-kernel) features, whose exponent x is already in log2 units and
// shifted; max(x, 0) for the generalised ReLU features (x = log2(e) omega.x,
// a constant factor that cancels in normalised attention).
// ReLU features take the IEEE 754-2019 maximum (v_maximum3_f32 on gfx950):
// unlike fmax it keeps a NaN projection NaN, as max(NaN, 0) in the exact
// formula, and still maps the -inf of masked rows to 0.
template <bool RELU> __device__ __forceinline__ float feat(float x) {
    if constexpr (RELU) return __builtin_elementwise_maximum(x, 0.0f);
    else return exp2f_fast(x);
}

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// gfx950 LDS transpose read (ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane s supplies the address of a 4-element chunk M[s][0..3]; lane i
// receives {M[4j + i/4][i % 4] : j = 0..3}.
__device__ __forceinline__ bf16x4 lds_read_tr16(const bf16* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}

// Row-major LDS tile of 32 rows; rows padded by 16 bytes so that 16 lanes
// reading 16-byte pieces of 16 consecutive rows hit distinct banks.
template <typename T, int COLS> struct LdsTile {
    static constexpr int RS = COLS + 16 / (int)sizeof(T);  // row stride, elements
    static constexpr int ELEMS = 32 * RS;
};

// Operand holding, for column `col` (= col0 + r), the 8 rows in kappa order
// {4g..4g+3, 16+4g..16+4g+3} of a row-major 32-row LDS tile: the B operand of
// a contraction over the tile's rows.  bf16: two transpose reads (lane
// (q, s = 4j + c) points at row 4q + j, columns col0 + 4c..+3).
template <int RS>
__device__ __forceinline__ bf16x8 kappa_col(const bf16* tile, int col0, int lane) {
    const int q = lane >> 4, s = lane & 15;
    const bf16* p0 = tile + (4 * q + (s >> 2)) * RS + col0 + 4 * (s & 3);
    const bf16x4 lo = lds_read_tr16(p0);
    const bf16x4 hi = lds_read_tr16(p0 + 16 * RS);
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
template <int RS>
__device__ __forceinline__ f8 kappa_col(const float* tile, int col0, int lane) {
    const int r = lane & 15, g = lane >> 4;
    const float* p = tile + col0 + r;
    f8 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[i] = p[(4 * g + i) * RS];
        v[4 + i] = p[(16 + 4 * g + i) * RS];
    }
    return v;
}

// Store 4 consecutive elements (one D-tile column quad) into LDS.
__device__ __forceinline__ void lds_store4(bf16* p, f4 v) {
    bf16x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = (bf16)v[i];
    *reinterpret_cast<bf16x4*>(p) = r;
}
__device__ __forceinline__ void lds_store4(float* p, f4 v) { *reinterpret_cast<float4*>(p) = float4{v[0], v[1], v[2], v[3]}; }

// Store 4 consecutive output elements.
__device__ __forceinline__ void store4(bf16* p, f4 v) {
    bf16x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = (bf16)v[i];
    *reinterpret_cast<bf16x4*>(p) = r;
}
__device__ __forceinline__ void store4(float* p, f4 v) { *reinterpret_cast<float4*>(p) = float4{v[0], v[1], v[2], v[3]}; }

// Load 4 consecutive elements as fp32.
__device__ __forceinline__ f4 load4f(const bf16* p) {
    const bf16x4 x = *reinterpret_cast<const bf16x4*>(p);
    return f4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
}
__device__ __forceinline__ f4 load4f(const float* p) { return *reinterpret_cast<const f4*>(p); }

}  // namespace favor
