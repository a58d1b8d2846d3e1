// Philox4x64 with 10 rounds (Salmon, Moraes, Dror, Shaw, "Parallel random
// numbers: as easy as 1, 2, 3", SC'11) for device code: the counter-based
// generator the projection generators draw their random numbers from.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace favor_rng {

struct Words {
    uint64_t w[4];
};

__device__ inline Words philox4x64_10(Words c, uint64_t k0, uint64_t k1) {
    const uint64_t M0 = 0xD2E7470EE14C6C93ULL, M1 = 0xCA5A826395121157ULL;
    const uint64_t W0 = 0x9E3779B97F4A7C15ULL, W1 = 0xBB67AE8584CAA73BULL;
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += W0;
            k1 += W1;
        }
        const uint64_t hi0 = __umul64hi(M0, c.w[0]), lo0 = M0 * c.w[0];
        const uint64_t hi1 = __umul64hi(M1, c.w[2]), lo1 = M1 * c.w[2];
        Words n;
        n.w[0] = hi1 ^ c.w[1] ^ k0;
        n.w[1] = lo1;
        n.w[2] = hi0 ^ c.w[3] ^ k1;
        n.w[3] = lo0;
        c = n;
    }
    return c;
}

}  // namespace favor_rng
