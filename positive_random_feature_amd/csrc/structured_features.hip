// Positive (or ReLU) random features over the structured Hadamard projection
// without materialising it (favor_features_hadamard in include/favor.h).
//
// paperlayer.ai summary of arXiv:2009.14794v4, B.3 (implementation
// trade-offs): structured ORFs let the features be built with fast transforms
// in O(L m log d) time instead of a dense projection.  Block b of the
// projection is sqrt(d) H S1 H S2 H S3 (H the normalised Sylvester-Hadamard
// matrix, S_t diagonal +-1), so its rows applied to x are
//     (1/d) Hu S1 Hu S2 Hu S3 x,   Hu = sqrt(d) H (entries +-1),
// three unnormalised Walsh-Hadamard transforms of length d with sign flips
// between them: d log2 d additions each instead of d^2 multiply-adds.
//
// One thread per token: x stays in registers in its input type, each block's
// transform runs in fp32 registers, and the features of a block go through
// an LDS tile so that each wave writes whole output rows.  The signs are the
// ones favor_hadamard_omega draws (Philox4x64-10, key (seed, 0), counter
// (0, b, h, 2 + t) for diagonal t; entry j flips when bit j % 64 of output
// word j / 64 is set), computed once per workgroup.
#include "favor_device.h"
#include "favor_kernels.h"
#include "philox_device.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace favor {
namespace {

using favor_rng::Words;
using favor_rng::philox4x64_10;

constexpr int kTokWave = 64;
constexpr int kWavesHf = 4;
constexpr int kMaxBlocksHf = 512 / 16;  // m <= 512, d >= 16

template <int D>
struct HfSmem {
    static constexpr int RS = D + 4;  // tile row stride (floats)
    static constexpr size_t SIGNS = sizeof(uint32_t) * (size_t)kMaxBlocksHf * 3 * 4;
    static constexpr size_t BYTES = SIGNS + sizeof(float) * (size_t)kWavesHf * kTokWave * RS;
};

// Unnormalised Walsh-Hadamard transform in place (Sylvester order).
template <int D>
__device__ __forceinline__ void wht(float (&v)[D]) {
#pragma unroll
    for (int len = 1; len < D; len <<= 1)
#pragma unroll
        for (int i = 0; i < D; i += 2 * len)
#pragma unroll
            for (int j = 0; j < len; ++j) {
                const float a = v[i + j], b = v[i + j + len];
                v[i + j] = a + b;
                v[i + j + len] = a - b;
            }
}

// Sign flips by a diagonal held as four wave-uniform 32-bit words.
template <int D>
__device__ __forceinline__ void flip(float (&v)[D], const uint32_t (&w)[4]) {
#pragma unroll
    for (int j = 0; j < D; ++j)
        v[j] = __uint_as_float(__float_as_uint(v[j]) ^ (((w[j / 32] >> (j % 32)) & 1u) << 31));
}

template <int D>
__device__ __forceinline__ void load_diag(const uint32_t* sg, int b, int t, uint32_t (&w)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = __builtin_amdgcn_readfirstlane(sg[(b * 3 + t) * 4 + i]);
}

// Projection of block b: v = (1/d) Hu S1 Hu S2 Hu S3 x.
template <typename T, int D>
__device__ __forceinline__ void project_block(const vec8<T> (&xv)[D / 8], const uint32_t* sg, int b, float (&v)[D]) {
#pragma unroll
    for (int c = 0; c < D / 8; ++c)
#pragma unroll
        for (int i = 0; i < 8; ++i) v[8 * c + i] = to_f(xv[c][i]);
    uint32_t w[4];
#pragma unroll
    for (int t = 2; t >= 0; --t) {
        load_diag<D>(sg, b, t, w);
        flip<D>(v, w);
        wht<D>(v);
    }
#pragma unroll
    for (int j = 0; j < D; ++j) v[j] *= 1.0f / D;
}

template <typename T, int D, bool RELU>
__global__ __launch_bounds__(kWavesHf * 64) void hadamard_features_kernel(const T* __restrict__ x,
                                                                         unsigned long long seed, int per_head,
                                                                         float* __restrict__ phi,
                                                                         float* __restrict__ log_scale, int H, int L,
                                                                         int m, int stabilize) {
    using SM = HfSmem<D>;
    extern __shared__ __attribute__((aligned(16))) char smem_raw[];
    uint32_t* sg = reinterpret_cast<uint32_t*>(smem_raw);
    float* tile_all = reinterpret_cast<float*>(smem_raw + SM::SIGNS);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int bh = blockIdx.y, h = bh % H;
    const int nb = (m + D - 1) / D;
    const int t0w = blockIdx.x * (kWavesHf * kTokWave) + w * kTokWave;
    const int row = t0w + lane;
    const bool ok = row < L;
    const size_t grow = (size_t)bh * L + row;

    // the diagonals of this head's blocks: one Philox call each
    for (int e = threadIdx.x; e < 3 * nb; e += blockDim.x) {
        const int b = e / 3, t = e % 3;
        const Words o = philox4x64_10(Words{{0, (uint64_t)b, (uint64_t)(per_head ? h : 0), (uint64_t)(2 + t)}}, seed, 0);
        uint32_t* d = sg + (size_t)(b * 3 + t) * 4;
        d[0] = (uint32_t)o.w[0];
        d[1] = (uint32_t)(o.w[0] >> 32);
        d[2] = (uint32_t)o.w[1];
        d[3] = (uint32_t)(o.w[1] >> 32);
    }
    vec8<T> xv[D / 8];
    float ss = 0.0f;
#pragma unroll
    for (int c = 0; c < D / 8; ++c) {
        xv[c] = ok ? load8(x + grow * D + 8 * c) : zero8<T>();
#pragma unroll
        for (int i = 0; i < 8; ++i) ss += to_f(xv[c][i]) * to_f(xv[c][i]);
    }
    __syncthreads();

    float s = 0.0f;  // stabiliser, natural-log units
    if (!RELU && stabilize) {
        float mx = kNegInf;
        for (int b = 0; b < nb; ++b) {
            float v[D];
            project_block<T, D>(xv, sg, b, v);
            const int rows = min(D, m - b * D);
#pragma unroll
            for (int j = 0; j < D; ++j)
                if (j < rows) mx = __builtin_fmaxf(mx, v[j]);
        }
        s = mx - 0.5f * ss;
    }
    if (stabilize && ok && log_scale) log_scale[grow] = RELU ? 0.0f : s;
    // positive: phi = 2^(log2(e) p + off); ReLU: phi = rscale max(p, 0)
    const float off = -kLog2e * (0.5f * ss + s) - 0.5f * __builtin_log2f((float)m);
    const float rscale = 1.0f / __builtin_sqrtf((float)m);
    float* tile = tile_all + (size_t)w * kTokWave * SM::RS;
    for (int b = 0; b < nb; ++b) {
        float v[D];
        project_block<T, D>(xv, sg, b, v);
        float* tr = tile + (size_t)lane * SM::RS;
#pragma unroll
        for (int j = 0; j < D; j += 4) {
            f4 e;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                e[i] = RELU ? rscale * feat<true>(v[j + i]) : exp2f_fast(__builtin_fmaf(kLog2e, v[j + i], off));
            *reinterpret_cast<f4*>(tr + j) = e;
        }
        __syncthreads();
        // the wave writes its 64 token rows: rows / 4 lanes per row
        const int rows = min(D, m - b * D);
        const int per_row = rows / 4;
        for (int idx = lane; idx < kTokWave * per_row; idx += 64) {
            const int rr = idx / per_row, c4 = idx % per_row;
            if (t0w + rr < L)
                *reinterpret_cast<f4*>(phi + ((size_t)bh * L + t0w + rr) * m + (size_t)b * D + 4 * c4) =
                    *reinterpret_cast<const f4*>(tile + (size_t)rr * SM::RS + 4 * c4);
        }
        __syncthreads();
    }
}

template <typename T, int D, bool RELU>
hipError_t launch_hf(const HadamardFeaturesArgs& a) {
    constexpr size_t bytes = HfSmem<D>::BYTES;
    static_assert(bytes <= kMaxLds, "hadamard features LDS");
    auto kern = hadamard_features_kernel<T, D, RELU>;
    (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    const int per_wg = kWavesHf * kTokWave;
    const dim3 grid((a.L + per_wg - 1) / per_wg, a.B * a.H);
    hipLaunchKernelGGL(kern, grid, dim3(kWavesHf * 64), bytes, a.stream, static_cast<const T*>(a.x), a.seed,
                       a.omega_per_head, a.phi, a.log_scale, a.H, a.L, a.m, a.stabilize);
    return hipGetLastError();
}

template <typename T, bool RELU>
hipError_t launch_hf_d(const HadamardFeaturesArgs& a) {
    switch (a.D) {
        case 16: return launch_hf<T, 16, RELU>(a);
        case 32: return launch_hf<T, 32, RELU>(a);
        case 64: return launch_hf<T, 64, RELU>(a);
        default:
            if constexpr (sizeof(T) == 2) return launch_hf<T, 128, RELU>(a);
            return hipErrorInvalidValue;  // fp32 with d = 128 is rejected by argument validation
    }
}

}  // namespace

hipError_t launch_hadamard_features(const HadamardFeaturesArgs& a) {
    if (a.dtype_bytes == 2) return a.relu ? launch_hf_d<bf16, true>(a) : launch_hf_d<bf16, false>(a);
    return a.relu ? launch_hf_d<float, true>(a) : launch_hf_d<float, false>(a);
}

}  // namespace favor
