// Seeded orthogonal random projections on the host (see favor_orf_omega in
// include/favor.h).
//
// "Performer" digest (irregular6612.github.io), core components: the rows of
// the Gaussian projection are orthogonalised by Gram-Schmidt, block by block
// when m > d; paperlayer.ai summary of arXiv:2009.14794v4, A.2: the
// construction keeps every row marginally Gaussian.  Each row is therefore
// given the length of an independent N(0, I_d) vector.
//
// Random numbers: Philox4x64 with 10 rounds (Salmon, Moraes, Dror, Shaw,
// "Parallel random numbers: as easy as 1, 2, 3", SC'11), turned into normals
// with the Box-Muller transform.
#include "../../include/favor.h"

#include <cmath>
#include <cstdint>
#include <vector>

namespace {

typedef unsigned __int128 u128;

struct Ctr {
    uint64_t w[4];
};

Ctr philox4x64_10(Ctr c, uint64_t k0, uint64_t k1) {
    const uint64_t M0 = 0xD2E7470EE14C6C93ULL, M1 = 0xCA5A826395121157ULL;
    const uint64_t W0 = 0x9E3779B97F4A7C15ULL, W1 = 0xBB67AE8584CAA73BULL;
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += W0;
            k1 += W1;
        }
        const u128 p0 = (u128)M0 * c.w[0];
        const u128 p1 = (u128)M1 * c.w[2];
        const uint64_t hi0 = (uint64_t)(p0 >> 64), lo0 = (uint64_t)p0;
        const uint64_t hi1 = (uint64_t)(p1 >> 64), lo1 = (uint64_t)p1;
        Ctr n;
        n.w[0] = hi1 ^ c.w[1] ^ k0;
        n.w[1] = lo1;
        n.w[2] = hi0 ^ c.w[3] ^ k1;
        n.w[3] = lo0;
        c = n;
    }
    return c;
}

// n standard normals of stream (a, b, c): call j uses counter (j, a, b, c).
void normals(uint64_t seed, uint64_t a, uint64_t b, uint64_t c, int n, double* out) {
    const double two_pi = 6.283185307179586;
    for (int j = 0; 4 * j < n; ++j) {
        const Ctr w = philox4x64_10(Ctr{{(uint64_t)j, a, b, c}}, seed, 0);
        double u[4];
        for (int i = 0; i < 4; ++i) u[i] = ((double)(w.w[i] >> 11) + 1.0) * 0x1p-53;
        const double r01 = std::sqrt(-2.0 * std::log(u[0]));
        const double r23 = std::sqrt(-2.0 * std::log(u[2]));
        const double t01 = two_pi * u[1], t23 = two_pi * u[3];
        const double z[4] = {r01 * std::cos(t01), r01 * std::sin(t01), r23 * std::cos(t23), r23 * std::sin(t23)};
        for (int i = 0; i < 4 && 4 * j + i < n; ++i) out[4 * j + i] = z[i];
    }
}

}  // namespace

extern "C" favor_status favor_orf_omega(unsigned long long seed, int n_heads, int m, int d, float* omega_host) {
    if (!omega_host || n_heads < 1 || m < 1 || d < 1) return FAVOR_ERR_INVALID_ARG;
    const int nb = (m + d - 1) / d;
    std::vector<double> blk((size_t)d * d), len((size_t)d * d);
    for (int h = 0; h < n_heads; ++h) {
        for (int b = 0; b < nb; ++b) {
            normals(seed, (uint64_t)b, (uint64_t)h, 0, d * d, blk.data());
            normals(seed, (uint64_t)b, (uint64_t)h, 1, d * d, len.data());
            const int rows = (b == nb - 1) ? m - b * d : d;
            for (int i = 0; i < rows; ++i) {
                double* u = &blk[(size_t)i * d];
                for (int j = 0; j < i; ++j) {  // modified Gram-Schmidt, rows in order
                    const double* e = &blk[(size_t)j * d];
                    double dot = 0.0;
                    for (int c = 0; c < d; ++c) dot += u[c] * e[c];
                    for (int c = 0; c < d; ++c) u[c] -= dot * e[c];
                }
                double nrm = 0.0;
                for (int c = 0; c < d; ++c) nrm += u[c] * u[c];
                nrm = std::sqrt(nrm);
                for (int c = 0; c < d; ++c) u[c] /= nrm;
                double l2 = 0.0;
                for (int c = 0; c < d; ++c) l2 += len[(size_t)i * d + c] * len[(size_t)i * d + c];
                const double l = std::sqrt(l2);
                float* dst = omega_host + ((size_t)h * m + (size_t)b * d + i) * d;
                for (int c = 0; c < d; ++c) dst[c] = (float)(u[c] * l);
            }
        }
    }
    return FAVOR_OK;
}
