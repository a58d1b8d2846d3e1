// Structured (Hadamard) orthogonal random projections generated on the
// device (favor_hadamard_omega in include/favor.h).
//
// paperlayer.ai summary of arXiv:2009.14794v4, A.2 (ORF bullet) and B.3
// (space and time trade-offs): Hadamard ORFs are orthogonal random features
// that need only O(m) random numbers, at the price of a small bias that
// vanishes as d grows.  Each d x d block here is sqrt(d) H S1 H S2 H S3,
// with H the normalised Sylvester-Hadamard matrix and S_t diagonal +-1
// matrices; its rows are orthogonal with norm sqrt(d).  The projection is
// materialised ([H, m, d] fp32) and used by the matrix-core projection like
// any other.  favor_features_hadamard applies the same blocks as fast
// Walsh-Hadamard transforms instead; measured on MI355X for stabilised bf16
// features of 131072 tokens (m = 4d), the dense matrix-core product is the
// faster one at every d: 14 against 18 us at d = 16, 42 against 61 us at
// d = 64, 128 against 178 us at d = 128.  The attention kernels keep the
// dense projection.
//
// Signs: Philox4x64 with 10 rounds (Salmon, Moraes, Dror, Shaw, SC'11), key
// (seed, 0); diagonal t of block b of head h reads counter (0, b, h, 2 + t),
// entry j is -1 when bit j % 64 of output word j / 64 is set.
#include "../../include/favor.h"
#include "philox_device.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

using favor_rng::Words;
using favor_rng::philox4x64_10;

// Unnormalised Walsh-Hadamard transform of a row vector, in place (the
// Sylvester matrix is symmetric, so v H = H v).
template <int D>
__device__ __forceinline__ void fwht(float (&v)[D]) {
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

// One thread per (head, row): row i of block b is e_i^T sqrt(d) H S1 H S2 H S3,
// built from the unnormalised matrix Hu = sqrt(d) H as (1/d) e_i^T Hu S1 Hu S2 Hu S3.
// Every intermediate is an integer of magnitude <= d^3, so the result is
// exact in fp32.
template <int D>
__global__ __launch_bounds__(64) void hadamard_omega_kernel(unsigned long long seed, int n_heads, int m,
                                                            float* __restrict__ omega) {
    const long long idx = (long long)blockIdx.x * 64 + threadIdx.x;
    if (idx >= (long long)n_heads * m) return;
    const int h = (int)(idx / m), row = (int)(idx % m);
    const int b = row / D, i = row % D;
    float v[D];
#pragma unroll
    for (int j = 0; j < D; ++j) v[j] = (__popc(i & j) & 1) ? -1.0f : 1.0f;
#pragma unroll
    for (int t = 0; t < 3; ++t) {
        const Words w = philox4x64_10(Words{{0, (uint64_t)b, (uint64_t)h, (uint64_t)(2 + t)}}, seed, 0);
#pragma unroll
        for (int j = 0; j < D; ++j)
            if ((w.w[j / 64] >> (j % 64)) & 1) v[j] = -v[j];
        if (t < 2) fwht<D>(v);
    }
    float* dst = omega + (size_t)idx * D;
#pragma unroll
    for (int j = 0; j < D; j += 4)
        *reinterpret_cast<float4*>(dst + j) = float4{v[j] / D, v[j + 1] / D, v[j + 2] / D, v[j + 3] / D};
}

}  // namespace

extern "C" favor_status favor_hadamard_omega(unsigned long long seed, int n_heads, int m, int d, float* omega,
                                             void* stream) {
    if (!omega || ((uintptr_t)omega % 16) != 0 || n_heads < 1 || m < 1) return FAVOR_ERR_INVALID_ARG;
    if (d != 16 && d != 32 && d != 64 && d != 128) return FAVOR_ERR_UNSUPPORTED;
    // n_heads * m * d < 2^31; n_heads * m < 2^62 cannot overflow, and the
    // bound is checked before the last factor
    if ((long long)n_heads * m >= (1LL << 31) / d) return FAVOR_ERR_UNSUPPORTED;
    const long long rows = (long long)n_heads * m;
    const dim3 grid((unsigned)((rows + 63) / 64));
    hipStream_t st = static_cast<hipStream_t>(stream);
    switch (d) {
        case 16: hipLaunchKernelGGL(hadamard_omega_kernel<16>, grid, dim3(64), 0, st, seed, n_heads, m, omega); break;
        case 32: hipLaunchKernelGGL(hadamard_omega_kernel<32>, grid, dim3(64), 0, st, seed, n_heads, m, omega); break;
        case 64: hipLaunchKernelGGL(hadamard_omega_kernel<64>, grid, dim3(64), 0, st, seed, n_heads, m, omega); break;
        default: hipLaunchKernelGGL(hadamard_omega_kernel<128>, grid, dim3(64), 0, st, seed, n_heads, m, omega); break;
    }
    return hipGetLastError() == hipSuccess ? FAVOR_OK : FAVOR_ERR_HIP;
}
