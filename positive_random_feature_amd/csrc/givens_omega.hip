// Structured (Givens) orthogonal random projections generated on the device
// (favor_givens_omega in include/favor.h).
//
// paperlayer.ai summary of arXiv:2009.14794v4, A.2 (ORF bullet) and B.3
// (space and time trade-offs): Givens ORFs are orthogonal random features
// that keep O(m log d) random numbers, at the price of a small bias that
// vanishes as d grows.  Each d x d block here is a product of K random plane
// rotations applied to the identity (K = d ceil(log2 d) by default, the
// order of steps after which such a walk is close to a uniformly random
// rotation); row r is then scaled to an independent chi(d) length, the one
// the Gram-Schmidt generator gives row r of the same block.  The block is
// computed in fp64 in LDS and rounded to fp32 once.
//
// Random numbers: Philox4x64-10, key (seed, 0).  Rotation k of block b of
// head h reads counter (k, b, h, 5): coordinates i = floor(d w0hi / 2^32),
// j' = floor((d - 1) w1hi / 2^32), j = j' + (j' >= i) (whi = w >> 32), angle
// 2 pi ((w2 >> 11) + 1) 2^-53.  Row lengths: the norm of normals
// r d .. r d + d - 1 of counter stream (b, h, 1), four normals per counter
// (j, b, h, 1) by Box-Muller on 53-bit uniforms.
#include "../../include/favor.h"
#include "philox_device.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

using favor_rng::Words;
using favor_rng::philox4x64_10;

constexpr int kMaxD = 128;
constexpr int kRotChunk = 256;  // rotations drawn per round, one per thread
constexpr int kThreads = 256;
constexpr int kMaxRotations = 1 << 24;

__device__ __forceinline__ double unit53(uint64_t w) { return ((double)(w >> 11) + 1.0) * 0x1p-53; }

// Normal number e of counter stream (b, h, 1) (Box-Muller, as the host
// Gram-Schmidt generator draws it).
__device__ double stream_normal(unsigned long long seed, int b, int h, long long e) {
    const Words w = philox4x64_10(Words{{(uint64_t)(e / 4), (uint64_t)b, (uint64_t)h, 1}}, seed, 0);
    const int k = (int)(e % 4);
    const double ua = unit53(w.w[k < 2 ? 0 : 2]), ub = unit53(w.w[k < 2 ? 1 : 3]);
    const double r = sqrt(-2.0 * log(ua));
    const double t = 6.283185307179586 * ub;
    return (k % 2 == 0) ? r * cos(t) : r * sin(t);
}

// One workgroup per (block, head).  LDS: the block q[d][d] (fp64, row-major),
// the row lengths, and one round of rotation parameters.  Thread c < d owns
// column c: a rotation of rows (i, j) changes each column independently, so
// the rotations of a round are applied without barriers between them.
__global__ __launch_bounds__(kThreads) void givens_omega_kernel(unsigned long long seed, int m, int d, int count,
                                                                float* __restrict__ omega) {
    extern __shared__ double smem[];
    double* q = smem;                      // [d][d]
    double* len = q + (size_t)d * d;       // [d]
    double* rc = len + kMaxD;              // [kRotChunk] cos
    double* rs = rc + kRotChunk;           // [kRotChunk] sin
    int* ri = reinterpret_cast<int*>(rs + kRotChunk);  // [kRotChunk]
    int* rj = ri + kRotChunk;                          // [kRotChunk]
    const int b = blockIdx.x, h = blockIdx.y, t = threadIdx.x;

    for (int e = t; e < d * d; e += kThreads) q[e] = (e / d == e % d) ? 1.0 : 0.0;
    for (int r = t; r < d; r += kThreads) {
        double ss = 0.0;
        for (int c = 0; c < d; ++c) {
            const double z = stream_normal(seed, b, h, (long long)r * d + c);
            ss += z * z;
        }
        len[r] = sqrt(ss);
    }
    for (int k0 = 0; k0 < count; k0 += kRotChunk) {
        const int n = min(kRotChunk, count - k0);
        __syncthreads();  // the previous round's parameters are no longer read
        if (t < n) {
            const Words w = philox4x64_10(Words{{(uint64_t)(k0 + t), (uint64_t)b, (uint64_t)h, 5}}, seed, 0);
            const int i = (int)(((uint64_t)d * (w.w[0] >> 32)) >> 32);
            const int jp = (int)(((uint64_t)(d - 1) * (w.w[1] >> 32)) >> 32);
            const double th = 6.283185307179586 * unit53(w.w[2]);
            ri[t] = i;
            rj[t] = jp + (jp >= i ? 1 : 0);
            rc[t] = cos(th);
            rs[t] = sin(th);
        }
        __syncthreads();
        if (t < d) {
            for (int u = 0; u < n; ++u) {
                double* a = q + (size_t)ri[u] * d + t;
                double* bb = q + (size_t)rj[u] * d + t;
                const double x = *a, y = *bb, c = rc[u], s = rs[u];
                *a = c * x - s * y;
                *bb = s * x + c * y;
            }
        }
    }
    __syncthreads();
    const int rows = min(d, m - b * d);
    float* dst = omega + ((size_t)h * m + (size_t)b * d) * d;
    for (int e = t; e < rows * d; e += kThreads) dst[e] = (float)(q[e] * len[e / d]);
}

}  // namespace

extern "C" favor_status favor_givens_omega(unsigned long long seed, int n_heads, int m, int d, int rotations,
                                           float* omega, void* stream) {
    if (!omega || ((uintptr_t)omega % 16) != 0 || n_heads < 1 || m < 1) return FAVOR_ERR_INVALID_ARG;
    if (rotations < 0 || rotations > kMaxRotations) return FAVOR_ERR_INVALID_ARG;
    if (d < 2 || d > kMaxD || n_heads > 65535) return FAVOR_ERR_UNSUPPORTED;
    // n_heads * m * d < 2^31, checked before the last factor
    if ((long long)n_heads * m >= (1LL << 31) / d) return FAVOR_ERR_UNSUPPORTED;
    int log2d = 0;
    while ((1 << log2d) < d) ++log2d;  // ceil(log2 d), >= 1 for d >= 2
    const int count = rotations > 0 ? rotations : d * log2d;
    const int nb = (m + d - 1) / d;
    const size_t lds = sizeof(double) * ((size_t)d * d + kMaxD + 2 * kRotChunk) + sizeof(int) * 2 * kRotChunk;
    (void)hipFuncSetAttribute((const void*)givens_omega_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL(givens_omega_kernel, dim3(nb, n_heads), dim3(kThreads), lds, static_cast<hipStream_t>(stream), seed,
                       m, d, count, omega);
    return hipGetLastError() == hipSuccess ? FAVOR_OK : FAVOR_ERR_HIP;
}
