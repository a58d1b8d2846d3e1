// gfx950 kernels for FAVOR+ attention.
//
// Pages: "Performer — 랜덤 특징으로 어텐션을 다시 생각하기" (digest of
// *Rethinking Attention with Performers*): Methods, core components, key
// formulas; Su Jianlin, "From Performer to Linear Attention": Simple
// Derivation; paperlayer.ai summary of arXiv:2009.14794v4: sections 2, A.2,
// B.3.
//
// Features phi(x)_i = m^-1/2 exp(omega_i.x - |x|^2/2) are built in base 2:
// omega is pre-scaled by log2(e) and rounded to the operand type when packed,
// the projection runs on the matrix cores with its accumulator initialised to
// -log2(e)|x|^2/2 (plus stabiliser offsets), and one v_exp_f32 finishes each
// feature.  The m^-1/2 factor cancels in normalised attention and is applied
// only by the features kernel.  Stabilisers (per query row, and one shift
// common to all keys of a head, applied per feature group with exact
// rescaling) cancel between numerator and denominator because a per-query
// factor and a factor common to all keys leave the normalised output
// unchanged (Simple Derivation).
//
// Kernels:
//   pack_omega      omega fp32 -> log2(e)*omega in operand order (per head)
//   kv_partial      per (head, segment, feature group): sum_s phi(k_s)[v_s | 1]
//                   with a running key shift per wave
//   merge_scan      per (head, 32-feature block): total over segments
//                   (bidirectional) or exclusive prefix (causal carry-in)
//   bidir_out       phi(q) . [KV | z] for tiles of 64 queries per wave
//   causal_chunk    per (head, segment): chunked scan, 32 tokens per step
//   features        phi(x) written to memory (diagnostic / API)
#include "favor_device.h"
#include "favor_kernels.h"

#include <algorithm>

namespace favor {

// ---------------------------------------------------------------------------
// omega packing: A-operand order for the projection D[F x T] = Omega'[F x d] X^T.
// Entry ((ft * KSD + ks) * 64 + lane) holds Omega'[16 ft + r][32 ks + 8 g + j].
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void pack_omega_kernel(const float* __restrict__ omega, vec8<T>* __restrict__ out,
                                                         int n_heads, int m) {
    constexpr int KSD = D < 32 ? 1 : D / 32;
    const int nft = m / 16;
    const long long per_head = (long long)nft * KSD * 64;
    const long long total = per_head * n_heads;
    for (long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (long long)gridDim.x * blockDim.x) {
        const int lane = (int)(idx % 64);
        const long long rest = idx / 64;
        const int ks = (int)(rest % KSD);
        const int ft = (int)((rest / KSD) % nft);
        const int h = (int)(rest / ((long long)KSD * nft));
        const int r = lane & 15, g = lane >> 4;
        const int f = 16 * ft + r;
        vec8<T> v;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int c = 32 * ks + 8 * g + j;
            const float x = c < D ? omega[((size_t)h * m + f) * D + c] * kLog2e : 0.0f;
            v[j] = (T)x;
        }
        out[idx] = v;
    }
}

// ---------------------------------------------------------------------------
// Tile staging helpers (LDS).
// Key tile: rows of 32 tokens x D, row stride KS_STRIDE elements (padded).
// Value tile, transposed: Vt[dim][token], row stride VT_STRIDE elements.
// ---------------------------------------------------------------------------
template <typename T, int D> struct Tiles {
    static constexpr int KS_STRIDE = D + 16 / (int)sizeof(T);  // rows padded by 16 B
    static constexpr int VT_STRIDE = 36;                       // 8-B (bf16) / 16-B (fp32) aligned rows
    static constexpr int K_ELEMS = 32 * KS_STRIDE;
    static constexpr int V_ELEMS = D * VT_STRIDE;
};

// Cooperative load of 32 rows starting at token t0 (rows >= t_end are zero)
// into the key tile (natural layout) and/or the transposed value tile.
template <typename T, int D, bool KEYS, bool VALS>
__device__ __forceinline__ void stage_tiles(const T* __restrict__ kbase, const T* __restrict__ vbase, int t0, int t_end,
                                            T* __restrict__ ks_lds, T* __restrict__ vt_lds) {
    using TL = Tiles<T, D>;
    constexpr int CPR = D / 8;  // 8-element chunks per row
    for (int item = threadIdx.x; item < 32 * CPR; item += blockDim.x) {
        const int tok = item / CPR, c = item % CPR;
        const int t = t0 + tok;
        const bool ok = t < t_end;
        if (KEYS) {
            vec8<T> x = ok ? load8(kbase + (size_t)t * D + 8 * c) : zero8<T>();
            *reinterpret_cast<vec8<T>*>(ks_lds + tok * TL::KS_STRIDE + 8 * c) = x;
        }
        if (VALS) {
            vec8<T> x = ok ? load8(vbase + (size_t)t * D + 8 * c) : zero8<T>();
#pragma unroll
            for (int j = 0; j < 8; ++j) vt_lds[(8 * c + j) * TL::VT_STRIDE + tok] = x[j];
        }
    }
}

// Key/query operand for 16 tokens (rows 16*tt + r of the staged tile), dims
// 32*ks + 8g .. +7, zero beyond D.
template <typename T, int D>
__device__ __forceinline__ vec8<T> tile_operand(const T* __restrict__ ks_lds, int row, int ks, int g) {
    using TL = Tiles<T, D>;
    if (D < 32 && g >= D / 8) return zero8<T>();
    return *reinterpret_cast<const vec8<T>*>(ks_lds + row * TL::KS_STRIDE + 32 * ks + 8 * g);
}

// Two runs of 4 elements at [4g, 4g+4) and [16+4g, 20+4g) of an LDS row.
template <typename T> __device__ __forceinline__ vec8<T> kappa_read(const T* row, int g);
template <> __device__ __forceinline__ bf16x8 kappa_read<bf16>(const bf16* row, int g) {
    const bf16x4 lo = *reinterpret_cast<const bf16x4*>(row + 4 * g);
    const bf16x4 hi = *reinterpret_cast<const bf16x4*>(row + 16 + 4 * g);
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
template <> __device__ __forceinline__ f8 kappa_read<float>(const float* row, int g) {
    const float4 lo = *reinterpret_cast<const float4*>(row + 4 * g);
    const float4 hi = *reinterpret_cast<const float4*>(row + 16 + 4 * g);
    return f8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
}

// Value operand in kappa order: tokens {4g..4g+3, 16+4g..16+4g+3}, dim `dim`.
template <typename T, int D>
__device__ __forceinline__ vec8<T> vt_operand(const T* __restrict__ vt_lds, int dim, int g) {
    using TL = Tiles<T, D>;
    return kappa_read<T>(vt_lds + dim * TL::VT_STRIDE, g);
}

// ---------------------------------------------------------------------------
// kv_partial: one workgroup per (segment, head, feature group of <= 256).
// Wave w owns FW = 32 features.  Per 32-token tile: projection D[T x F] =
// K[T x d] Omega'^T, a running shift M (max over this wave's exponents, raised
// lazily), phi in kappa order as the A operand, and [V | 1] from LDS.
// Output: partial[bh][seg][f][0..D] (column D = sum of phi) and pmax[bh][seg][f/32].
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(512) void kv_partial_kernel(const T* __restrict__ k, const T* __restrict__ v,
                                                         const vec8<T>* __restrict__ ompack, long long om_head_vecs,
                                                         float* __restrict__ partial, float* __restrict__ pmax, int H,
                                                         int L, int m, int seg_len, int nseg_stride) {
    using TL = Tiles<T, D>;
    constexpr int KSD = D < 32 ? 1 : D / 32;
    constexpr int NT = D / 16 + 1;  // value tiles + the ones tile
    constexpr int FW = 32;
    constexpr int NFT = FW / 16;
    __shared__ __attribute__((aligned(16))) T ks_lds[TL::K_ELEMS];
    __shared__ __attribute__((aligned(16))) T vt_lds[TL::V_ELEMS];

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, r = lane & 15, g = lane >> 4;
    const int seg = blockIdx.x, bh = blockIdx.y;
    const int h = bh % H;
    const int f0 = blockIdx.z * 256 + w * FW;  // first feature of this wave
    // The last feature group may have fewer than 8 waves' worth of features:
    // the spare waves still stage tiles and meet every barrier, but load,
    // compute and write nothing.
    const bool active = f0 < m;
    const int fa = active ? f0 : 0;
    const int t_begin = seg * seg_len;
    const int t_end = min(L, t_begin + seg_len);
    const size_t xbase = (size_t)bh * L * D;
    const vec8<T>* omh = ompack + (size_t)(om_head_vecs ? h : 0) * (size_t)om_head_vecs;

    vec8<T> om[NFT][KSD];
#pragma unroll
    for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) om[ft][ks] = omh[((size_t)(fa / 16 + ft) * KSD + ks) * 64 + lane];

    f4 kv[NFT][NT];
#pragma unroll
    for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) kv[ft][nt] = f4splat(0.0f);
    float M = kNegInf;

    for (int t0 = t_begin; t0 < t_end; t0 += 32) {
        __syncthreads();
        stage_tiles<T, D, true, true>(k + xbase, v + xbase, t0, t_end, ks_lds, vt_lds);
        __syncthreads();
        if (!active) continue;
        // key operands (rows T = 16tt + r) and accumulator init -log2e |k|^2 / 2
        vec8<T> xk[2][KSD];
        float cx[2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            float ss = 0.0f;
#pragma unroll
            for (int ks = 0; ks < KSD; ++ks) {
                xk[tt][ks] = tile_operand<T, D>(ks_lds, 16 * tt + r, ks, g);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float x = to_f(xk[tt][ks][j]);
                    ss += x * x;
                }
            }
            ss = col_sum(ss);
            cx[tt] = (t0 + 16 * tt + r < t_end) ? -0.5f * kLog2e * ss : kNegInf;
        }
        f4 p[2][NFT];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            f4 init;
#pragma unroll
            for (int i = 0; i < 4; ++i) init[i] = __shfl(cx[tt], 4 * g + i);
#pragma unroll
            for (int ft = 0; ft < NFT; ++ft) {
                p[tt][ft] = init;
#pragma unroll
                for (int ks = 0; ks < KSD; ++ks) p[tt][ft] = mma32(xk[tt][ks], om[ft][ks], p[tt][ft]);
            }
        }
        float tm = kNegInf;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
                for (int i = 0; i < 4; ++i) tm = __builtin_fmaxf(tm, p[tt][ft][i]);
        tm = wave_max(tm);
        if (tm > M + kTau) {
            const float sc = exp2f_fast(M - tm);
#pragma unroll
            for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) kv[ft][nt] *= sc;
            M = tm;
        }
        vec8<T> a[NFT];
#pragma unroll
        for (int ft = 0; ft < NFT; ++ft) {
            f4 e0, e1;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                e0[i] = exp2f_fast(p[0][ft][i] - M);
                e1[i] = exp2f_fast(p[1][ft][i] - M);
            }
            a[ft] = pack8t<T>(e0, e1);
        }
#pragma unroll
        for (int nt = 0; nt < NT - 1; ++nt) {
            const vec8<T> vb = vt_operand<T, D>(vt_lds, 16 * nt + r, g);
#pragma unroll
            for (int ft = 0; ft < NFT; ++ft) kv[ft][nt] = mma32(a[ft], vb, kv[ft][nt]);
        }
        const vec8<T> ones = splat8<T>(1.0f);
#pragma unroll
        for (int ft = 0; ft < NFT; ++ft) kv[ft][NT - 1] = mma32(a[ft], ones, kv[ft][NT - 1]);
    }

    if (!active) return;
    float* pp = partial + ((size_t)bh * nseg_stride + seg) * (size_t)m * (D + 1);
#pragma unroll
    for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int f = f0 + 16 * ft + 4 * g + i;
#pragma unroll
            for (int nt = 0; nt < NT - 1; ++nt) pp[(size_t)f * (D + 1) + 16 * nt + r] = kv[ft][nt][i];
            if (r == 0) pp[(size_t)f * (D + 1) + D] = kv[ft][NT - 1][i];
        }
    if (lane == 0) pmax[((size_t)bh * nseg_stride + seg) * (m / 32) + f0 / 32] = M;
}

// ---------------------------------------------------------------------------
// merge_scan: one workgroup per (32-feature block, head).
// mode 0 (bidirectional): sum over nseg partials, rescaled to the block's max;
//   writes the packed A operand of the output contraction
//   (kvpack[bh][mt][fb][lane], kappa order over the block's 32 features;
//   mt = D/16 is the z row replicated) and mmax[bh][fb].
// mode 1 (causal): exclusive prefix over segments, carry[bh][s][f][0..D] fp32,
//   scaled to cmax[bh][s][fb] = the running key shift including segment s.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void merge_scan_kernel(const float* __restrict__ partial, const float* __restrict__ pmax,
                                                         int m, int nseg, int nseg_stride, int mode,
                                                         vec8<T>* __restrict__ kvpack, float* __restrict__ mmax,
                                                         float* __restrict__ carry, float* __restrict__ cmax, int nout) {
    constexpr int D1 = D + 1;
    const int fb = blockIdx.x, bh = blockIdx.y;
    const int nfb = m / 32;
    const float* pb = partial + (size_t)bh * nseg_stride * m * D1;
    const float* pm = pmax + (size_t)bh * nseg_stride * nfb;
    if (mode == 0) {
        __shared__ float merged[32 * D1];
        float Ms = kNegInf;
        for (int s = 0; s < nseg; ++s) Ms = __builtin_fmaxf(Ms, pm[(size_t)s * nfb + fb]);
        for (int e = threadIdx.x; e < 32 * D1; e += blockDim.x) {
            const int f = 32 * fb + e / D1, c = e % D1;
            float acc = 0.0f;
            for (int s = 0; s < nseg; ++s) {
                const float ms = pm[(size_t)s * nfb + fb];
                if (ms != kNegInf) acc += exp2f_fast(ms - Ms) * pb[((size_t)s * m + f) * D1 + c];
            }
            merged[e] = acc;
        }
        __syncthreads();
        // pack: entry (mt, lane) holds rows dim = 16 mt + r (or z), k = kappa(g, j)
        constexpr int NMT = D / 16 + 1;
        for (int e = threadIdx.x; e < NMT * 64; e += blockDim.x) {
            const int mt = e / 64, lane = e % 64, r = lane & 15, g = lane >> 4;
            const int col = mt < NMT - 1 ? 16 * mt + r : D;
            vec8<T> v;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int fl = j < 4 ? 4 * g + j : 16 + 4 * g + (j - 4);
                v[j] = (T)merged[fl * D1 + col];
            }
            kvpack[(((size_t)bh * NMT + mt) * nfb + fb) * 64 + lane] = v;
        }
        if (threadIdx.x == 0) mmax[(size_t)bh * nfb + fb] = Ms;
    } else {
        // carry[s] = sum_{s' < s} partial[s'], scaled to Mincl[s] = max_{s' <= s} pmax[s']:
        // every key of segment s has exponents <= Mincl[s] + kTau, so the
        // chunk kernel can use Mincl[s] as a fixed key shift.
        float* cb = carry + (size_t)bh * nout * m * D1;
        for (int e = threadIdx.x; e < 32 * D1; e += blockDim.x) {
            const int f = 32 * fb + e / D1, c = e % D1;
            float acc = 0.0f, Mrun = kNegInf;
            for (int s = 0; s < nout; ++s) {
                const float ms = pm[(size_t)s * nfb + fb];
                if (ms > Mrun) {
                    acc = (Mrun == kNegInf) ? 0.0f : acc * exp2f_fast(Mrun - ms);
                    Mrun = ms;
                }
                cb[((size_t)s * m + f) * D1 + c] = acc;
                if (ms != kNegInf) acc += exp2f_fast(ms - Mrun) * pb[((size_t)s * m + f) * D1 + c];
            }
        }
        if (threadIdx.x == 0) {
            float Mrun = kNegInf;
            for (int s = 0; s < nout; ++s) {
                Mrun = __builtin_fmaxf(Mrun, pm[(size_t)s * nfb + fb]);
                cmax[((size_t)bh * nout + s) * nfb + fb] = Mrun;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// bidir_out: workgroup = 8 waves x 64 queries.  The projection operands
// (omega') and the output operands ([KV | z]^T) of the head are staged once in
// LDS.  Each wave loops over 32-feature chunks: project its 4 query tiles
// (D[F x T], lanes own token columns), keep a lazy per-query shift, exponentiate
// into the B operand and accumulate out^T[dims | z][T] on the matrix cores.
// ---------------------------------------------------------------------------
template <typename T, int D, bool OM_LDS, bool KV_LDS>
__global__ __launch_bounds__(512) void bidir_out_kernel(const T* __restrict__ q, const vec8<T>* __restrict__ ompack,
                                                        long long om_head_vecs, const vec8<T>* __restrict__ kvpack,
                                                        const float* __restrict__ mmax, T* __restrict__ out, int H,
                                                        int L, int m) {
    constexpr int KSD = D < 32 ? 1 : D / 32;
    constexpr int NMT = D / 16 + 1;
    constexpr int NTT = D >= 128 ? 2 : 4;  // query tiles per wave
    extern __shared__ __attribute__((aligned(16))) char smem_raw[];
    const int nft = m / 16, nfb = m / 32;
    vec8<T>* kv_stage = reinterpret_cast<vec8<T>*>(smem_raw);
    vec8<T>* om_stage = kv_stage + (KV_LDS ? (size_t)NMT * nfb * 64 : 0);

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, r = lane & 15, g = lane >> 4;
    const int bh = blockIdx.y, h = bh % H;
    const vec8<T>* omh = ompack + (size_t)(om_head_vecs ? h : 0) * (size_t)om_head_vecs;
    const vec8<T>* kvh = kvpack + (size_t)bh * NMT * nfb * 64;
    if (OM_LDS)
        for (int e = threadIdx.x; e < nft * KSD * 64; e += blockDim.x) om_stage[e] = omh[e];
    if (KV_LDS)
        for (int e = threadIdx.x; e < NMT * nfb * 64; e += blockDim.x) kv_stage[e] = kvh[e];
    const vec8<T>* om_lds = OM_LDS ? om_stage : omh;
    const vec8<T>* kv_lds = KV_LDS ? kv_stage : kvh;
    float Mstar = kNegInf;
    for (int fb = 0; fb < nfb; ++fb) Mstar = __builtin_fmaxf(Mstar, mmax[(size_t)bh * nfb + fb]);
    __syncthreads();

    const int tbase = (blockIdx.x * (blockDim.x >> 6) + w) * (16 * NTT);
    if (tbase >= L) return;
    const size_t xbase = (size_t)bh * L * D;
    vec8<T> xq[NTT][KSD];
    float cq[NTT];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) {
        const int t = tbase + 16 * tt + r;
        const bool ok = t < L;
        float ss = 0.0f;
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) {
            const bool in = ok && (D >= 32 || g < D / 8);
            xq[tt][ks] = in ? load8(q + xbase + (size_t)t * D + 32 * ks + 8 * g) : zero8<T>();
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float x = to_f(xq[tt][ks][j]);
                ss += x * x;
            }
        }
        cq[tt] = -0.5f * kLog2e * col_sum(ss);
    }
    f4 acc[NMT][NTT];
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) acc[mt][tt] = f4splat(0.0f);
    float sref[NTT];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) sref[tt] = kNegInf;

    for (int fb = 0; fb < nfb; ++fb) {
        const float mb = mmax[(size_t)bh * nfb + fb];
        const float off = (mb == kNegInf) ? kNegInf : mb - Mstar;  // per-block key shift, <= 0
        f4 p[NTT][2];
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) p[tt][hh] = f4splat(cq[tt] + off);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int ks = 0; ks < KSD; ++ks) {
                const vec8<T> a = om_lds[((size_t)(2 * fb + hh) * KSD + ks) * 64 + lane];
#pragma unroll
                for (int tt = 0; tt < NTT; ++tt) p[tt][hh] = mma32(a, xq[tt][ks], p[tt][hh]);
            }
        vec8<T> b[NTT];
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) {
            float cm = kNegInf;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int i = 0; i < 4; ++i) cm = __builtin_fmaxf(cm, p[tt][hh][i]);
            cm = col_max(cm);
            const bool raise = cm > sref[tt] + kTau;
            if (__builtin_amdgcn_ballot_w64(raise)) {
                const float sc = raise ? ((sref[tt] == kNegInf) ? 0.0f : exp2f_fast(sref[tt] - cm)) : 1.0f;
#pragma unroll
                for (int mt = 0; mt < NMT; ++mt) acc[mt][tt] *= sc;
                if (raise) sref[tt] = cm;
            }
            f4 e0, e1;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                e0[i] = exp2f_fast(p[tt][0][i] - sref[tt]);
                e1[i] = exp2f_fast(p[tt][1][i] - sref[tt]);
            }
            b[tt] = pack8t<T>(e0, e1);
        }
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) {
            const vec8<T> a = kv_lds[((size_t)mt * nfb + fb) * 64 + lane];
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt) acc[mt][tt] = mma32(a, b[tt], acc[mt][tt]);
        }
    }
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) {
        const int t = tbase + 16 * tt + r;
        if (t >= L) continue;
        const float inv = 1.0f / acc[NMT - 1][tt][0];
#pragma unroll
        for (int mt = 0; mt < NMT - 1; ++mt) store4(out + xbase + (size_t)t * D + 16 * mt + 4 * g, acc[mt][tt] * inv);
    }
}

// ---------------------------------------------------------------------------
// causal_chunk: one workgroup per (segment, head); wave w owns features
// [64w, 64w + 64) and keeps its slice of the state G = sum phi(k) [v | 1]^T in
// registers (D layout: rows = features, columns = value dims / z).  Per chunk
// of 32 tokens:
//   1. stage K, Q (natural) and V (transposed) tiles in LDS;
//   2. project Q and K (D[F x T]); query shift = per-token max over the wave's
//      features; key shift M = fixed for the segment (from the partial pass:
//      no key of the segment exceeds it by more than kTau);
//   3. intra-chunk S^T[T_k x T_q] = phi(K) phi(Q)^T over the wave's features,
//      masked to T_k <= T_q;
//   4. partial numerator/denominator over this wave's features:
//      out^T = G^T phi(Q)^T + [V | 1]^T S^T, written to LDS with its log-scale;
//   5. G += phi(K)^T [V | 1] (phi(K) re-read transposed from LDS);
//   6. the workgroup sums the waves' partials (rescaled to a common scale)
//      and writes the outputs.
// The state starts from the exclusive prefix of earlier segments (carry).
// ---------------------------------------------------------------------------
template <typename T, int D, int FW_>
struct CausalSmem {
    using TL = Tiles<T, D>;
    static constexpr int FW = FW_;
    static constexpr int PT_STRIDE = 32 + 8;        // phi(K)^T rows (features) x 32 tokens (+pad)
    static constexpr int PART_STRIDE = D + 4;       // partial rows: 32 tokens x (D + 1) (+pad)
    static size_t bytes(int W) {
        size_t b = 0;
        b += sizeof(T) * (size_t)TL::K_ELEMS * 2;   // K and Q tiles
        b += sizeof(T) * (size_t)TL::V_ELEMS;       // V^T tile
        b += sizeof(T) * (size_t)W * FW * PT_STRIDE;  // per-wave phi(K)^T
        b += sizeof(float) * (size_t)W * 32 * PART_STRIDE;  // partials for the 32 queries
        b += sizeof(float) * (size_t)W * 32;        // partial log-scales
        return b;
    }
};

template <typename T, int D, int FW_, int MAXW>
__global__ __launch_bounds__(64 * MAXW) void causal_chunk_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                           const T* __restrict__ v, const vec8<T>* __restrict__ ompack,
                                                           long long om_head_vecs, const float* __restrict__ carry,
                                                           const float* __restrict__ cmax, T* __restrict__ out, int H,
                                                           int L, int m, int seg_len, int nseg) {
    using TL = Tiles<T, D>;
    using SM = CausalSmem<T, D, FW_>;
    constexpr int KSD = D < 32 ? 1 : D / 32;
    constexpr int NT = D / 16 + 1;
    constexpr int FW = SM::FW;
    constexpr int NFT = FW / 16;
    constexpr int KSF = FW / 32;
    constexpr int D1 = D + 1;
    extern __shared__ __attribute__((aligned(16))) char smem_raw[];
    const int W = blockDim.x >> 6;
    T* kt_lds = reinterpret_cast<T*>(smem_raw);
    T* qt_lds = kt_lds + TL::K_ELEMS;
    T* vt_lds = qt_lds + TL::K_ELEMS;
    T* pt_lds = vt_lds + TL::V_ELEMS;
    float* part = reinterpret_cast<float*>(pt_lds + (size_t)W * FW * SM::PT_STRIDE);
    float* plam = part + (size_t)W * 32 * SM::PART_STRIDE;

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, r = lane & 15, g = lane >> 4;
    const int seg = blockIdx.x, bh = blockIdx.y, h = bh % H;
    const int f0 = w * FW;
    const int nfb = m / 32;
    const int t_begin = seg * seg_len;
    const int t_end = min(L, t_begin + seg_len);
    const size_t xbase = (size_t)bh * L * D;
    const vec8<T>* omh = ompack + (size_t)(om_head_vecs ? h : 0) * (size_t)om_head_vecs;
    T* ptw = pt_lds + (size_t)w * FW * SM::PT_STRIDE;

    // state from the carry-in, rescaled to one fixed key shift per wave
    float M = kNegInf;
    const float* cm = cmax + ((size_t)bh * nseg + seg) * nfb;
#pragma unroll
    for (int b = 0; b < KSF; ++b) M = __builtin_fmaxf(M, cm[f0 / 32 + b]);
    f4 G[NFT][NT];
    {
        const float* cb = carry + ((size_t)bh * nseg + seg) * (size_t)m * D1;
#pragma unroll
        for (int ft = 0; ft < NFT; ++ft) {
            const float mb = cm[(f0 + 16 * ft) / 32];
            const float sc = (mb == kNegInf) ? 0.0f : exp2f_fast(mb - M);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int f = f0 + 16 * ft + 4 * g + i;
                    const int c = nt < NT - 1 ? 16 * nt + r : D;
                    G[ft][nt][i] = sc * cb[(size_t)f * D1 + c];
                }
        }
    }

    for (int t0 = t_begin; t0 < t_end; t0 += 32) {
        __syncthreads();
        stage_tiles<T, D, true, true>(k + xbase, v + xbase, t0, t_end, kt_lds, vt_lds);
        stage_tiles<T, D, true, false>(q + xbase, nullptr, t0, t_end, qt_lds, nullptr);
        __syncthreads();
        // Re-read the projection operands from memory every chunk (they stay in
        // cache) instead of pinning FW x D values in registers for the loop.
        const vec8<T>* omc = omh;
        asm volatile("" : "+s"(omc));

        // ---- queries: projection, per-token shift over this wave's features
        vec8<T> bq[2][KSF];
        float sq[2];
        {
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                vec8<T> x[KSD];
                float ss = 0.0f;
#pragma unroll
                for (int ks = 0; ks < KSD; ++ks) {
                    x[ks] = tile_operand<T, D>(qt_lds, 16 * tt + r, ks, g);
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const float xv = to_f(x[ks][j]);
                        ss += xv * xv;
                    }
                }
                const float c = -0.5f * kLog2e * col_sum(ss);
                f4 pq[NFT];
#pragma unroll
                for (int ft = 0; ft < NFT; ++ft) {
                    pq[ft] = f4splat(c);
#pragma unroll
                    for (int ks = 0; ks < KSD; ++ks)
                        pq[ft] = mma32(omc[((size_t)(f0 / 16 + ft) * KSD + ks) * 64 + lane], x[ks], pq[ft]);
                }
                float mx = kNegInf;
#pragma unroll
                for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
                    for (int i = 0; i < 4; ++i) mx = __builtin_fmaxf(mx, pq[ft][i]);
                mx = col_max(mx);
                sq[tt] = mx;
#pragma unroll
                for (int kf = 0; kf < KSF; ++kf) {
                    f4 e0, e1;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        e0[i] = exp2f_fast(pq[2 * kf][i] - mx);
                        e1[i] = exp2f_fast(pq[2 * kf + 1][i] - mx);
                    }
                    bq[tt][kf] = pack8t<T>(e0, e1);
                }
            }
        }
        // ---- keys: projection and features with the segment's fixed shift M
        vec8<T> ak[2][KSF];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            f4 pk[NFT];
            {
                vec8<T> x[KSD];
                float ss = 0.0f;
#pragma unroll
                for (int ks = 0; ks < KSD; ++ks) {
                    x[ks] = tile_operand<T, D>(kt_lds, 16 * tt + r, ks, g);
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const float xv = to_f(x[ks][j]);
                        ss += xv * xv;
                    }
                }
                const float c = (t0 + 16 * tt + r < t_end) ? -0.5f * kLog2e * col_sum(ss) - M : kNegInf;
#pragma unroll
                for (int ft = 0; ft < NFT; ++ft) {
                    pk[ft] = f4splat(c);
#pragma unroll
                    for (int ks = 0; ks < KSD; ++ks)
                        pk[ft] = mma32(omc[((size_t)(f0 / 16 + ft) * KSD + ks) * 64 + lane], x[ks], pk[ft]);
                }
            }
#pragma unroll
            for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
                for (int i = 0; i < 4; ++i) pk[ft][i] = exp2f_fast(pk[ft][i]);
#pragma unroll
            for (int kf = 0; kf < KSF; ++kf) ak[tt][kf] = pack8t<T>(pk[2 * kf], pk[2 * kf + 1]);
            // phi(K)^T for the state update: ptw[feature][token]
#pragma unroll
            for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
                for (int i = 0; i < 4; ++i) ptw[(16 * ft + 4 * g + i) * SM::PT_STRIDE + 16 * tt + r] = (T)pk[ft][i];
        }

        // ---- intra-chunk S^T[T_k x T_q], masked T_k <= T_q
        f4 S[2][2];
#pragma unroll
        for (int tk = 0; tk < 2; ++tk)
#pragma unroll
            for (int tq = 0; tq < 2; ++tq) {
                S[tk][tq] = f4splat(0.0f);
                if (tk <= tq) {
#pragma unroll
                    for (int kf = 0; kf < KSF; ++kf) S[tk][tq] = mma32(ak[tk][kf], bq[tq][kf], S[tk][tq]);
                }
            }
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (4 * g + i > r) S[t][t][i] = 0.0f;
        vec8<T> bs[2];
#pragma unroll
        for (int tq = 0; tq < 2; ++tq) bs[tq] = pack8t<T>(S[0][tq], S[1][tq]);

        // ---- partial outputs over this wave's features: out^T = G^T phi(Q)^T + [V|1]^T S^T
        {
            float* pw = part + (size_t)w * 32 * SM::PART_STRIDE;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                vec8<T> ga[KSF];
#pragma unroll
                for (int kf = 0; kf < KSF; ++kf) ga[kf] = pack8t<T>(G[2 * kf][nt], G[2 * kf + 1][nt]);
                const vec8<T> va = nt < NT - 1 ? vt_operand<T, D>(vt_lds, 16 * nt + r, g) : splat8<T>(1.0f);
#pragma unroll
                for (int tq = 0; tq < 2; ++tq) {
                    f4 o = f4splat(0.0f);
#pragma unroll
                    for (int kf = 0; kf < KSF; ++kf) o = mma32(ga[kf], bq[tq][kf], o);
                    o = mma32(va, bs[tq], o);
                    float* row = pw + (16 * tq + r) * SM::PART_STRIDE;
                    if (nt < NT - 1) {
                        *reinterpret_cast<float4*>(row + 16 * nt + 4 * g) = float4{o[0], o[1], o[2], o[3]};
                    } else if (g == 0) {
                        row[D] = o[0];
                    }
                }
            }
            if (g == 0) {
                plam[w * 32 + r] = sq[0] + M;
                plam[w * 32 + 16 + r] = sq[1] + M;
            }
        }
        __syncthreads();
        // combine the waves' partials (rescaled to a common scale) and store
        for (int item = threadIdx.x; item < 32 * (D / 8); item += blockDim.x) {
            const int tl = item / (D / 8), c8 = item % (D / 8);
            const int t = t0 + tl;
            float lmax = kNegInf;
            for (int ww = 0; ww < W; ++ww) lmax = __builtin_fmaxf(lmax, plam[ww * 32 + tl]);
            float num[8] = {0, 0, 0, 0, 0, 0, 0, 0};
            float den = 0.0f;
            for (int ww = 0; ww < W; ++ww) {
                const float lw = plam[ww * 32 + tl];
                const float sc = (lw == kNegInf) ? 0.0f : exp2f_fast(lw - lmax);
                const float* row = part + ((size_t)ww * 32 + tl) * SM::PART_STRIDE;
                const float4 a0 = *reinterpret_cast<const float4*>(row + 8 * c8);
                const float4 a1 = *reinterpret_cast<const float4*>(row + 8 * c8 + 4);
                num[0] += sc * a0.x; num[1] += sc * a0.y; num[2] += sc * a0.z; num[3] += sc * a0.w;
                num[4] += sc * a1.x; num[5] += sc * a1.y; num[6] += sc * a1.z; num[7] += sc * a1.w;
                den += sc * row[D];
            }
            if (t < t_end) {
                const float inv = 1.0f / den;
                f4 o0{num[0] * inv, num[1] * inv, num[2] * inv, num[3] * inv};
                f4 o1{num[4] * inv, num[5] * inv, num[6] * inv, num[7] * inv};
                store4(out + xbase + (size_t)t * D + 8 * c8, o0);
                store4(out + xbase + (size_t)t * D + 8 * c8 + 4, o1);
            }
        }

        // ---- state update G += phi(K)^T [V | 1]
#pragma unroll
        for (int ft = 0; ft < NFT; ++ft) {
            const vec8<T> a = kappa_read<T>(ptw + (16 * ft + r) * SM::PT_STRIDE, g);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const vec8<T> vb = nt < NT - 1 ? vt_operand<T, D>(vt_lds, 16 * nt + r, g) : splat8<T>(1.0f);
                G[ft][nt] = mma32(a, vb, G[ft][nt]);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// features: phi(x) (fp32) for 16 tokens per wave, all m features; optional
// per-row stabiliser (two passes: the maximum, then the features).
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void features_kernel(const T* __restrict__ x, const vec8<T>* __restrict__ ompack,
                                                       long long om_head_vecs, float* __restrict__ phi,
                                                       float* __restrict__ log_scale, int H, int L, int m,
                                                       int stabilize) {
    constexpr int KSD = D < 32 ? 1 : D / 32;
    const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
    const int t0 = (blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)) * 16;
    if (t0 >= L) return;
    const int bh = blockIdx.y, h = bh % H;
    const bool ok = t0 + r < L;
    const long long row = (long long)bh * L + t0 + r;
    const vec8<T>* omh = ompack + (size_t)(om_head_vecs ? h : 0) * (size_t)om_head_vecs;
    vec8<T> xv[KSD];
    float ss = 0.0f;
#pragma unroll
    for (int ks = 0; ks < KSD; ++ks) {
        const bool in = ok && (D >= 32 || g < D / 8);
        xv[ks] = in ? load8(x + (size_t)row * D + 32 * ks + 8 * g) : zero8<T>();
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float t = to_f(xv[ks][j]);
            ss += t * t;
        }
    }
    const float c = -0.5f * kLog2e * col_sum(ss);
    const int nft = m / 16;
    float s = 0.0f;
    if (stabilize) {
        float mx = kNegInf;
        for (int ft = 0; ft < nft; ++ft) {
            f4 p = f4splat(c);
#pragma unroll
            for (int ks = 0; ks < KSD; ++ks) p = mma32(omh[((size_t)ft * KSD + ks) * 64 + lane], xv[ks], p);
#pragma unroll
            for (int i = 0; i < 4; ++i) mx = __builtin_fmaxf(mx, p[i]);
        }
        s = col_max(mx);
        if (ok && g == 0 && log_scale) log_scale[row] = s / kLog2e;
    }
    const float off = c - s - 0.5f * __builtin_log2f((float)m);
    for (int ft = 0; ft < nft; ++ft) {
        f4 p = f4splat(off);
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) p = mma32(omh[((size_t)ft * KSD + ks) * 64 + lane], xv[ks], p);
        f4 e;
#pragma unroll
        for (int i = 0; i < 4; ++i) e[i] = exp2f_fast(p[i]);
        if (ok) store4(phi + (size_t)row * m + 16 * ft + 4 * g, e);
    }
}

// ---------------------------------------------------------------------------
// Host-side launchers (internal interface, see favor_kernels.h).
// ---------------------------------------------------------------------------
static inline void stage_event(const LaunchArgs& a, int i) {
    if (a.events) (void)hipEventRecord(static_cast<hipEvent_t>(a.events[i]), a.stream);
}

template <typename T, int D, int FW, int MAXW>
static hipError_t launch_causal(const LaunchArgs& a, const vec8<T>* ompack, long long om_head_vecs, const T* q,
                                const T* k, const T* v, T* out) {
    const int W = a.m / FW;
    const size_t smem = CausalSmem<T, D, FW>::bytes(W);
    auto kern = causal_chunk_kernel<T, D, FW, MAXW>;
    (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    hipLaunchKernelGGL(kern, dim3(a.nseg, a.B * a.H), dim3(64 * W), smem, a.stream, q, k, v, ompack, om_head_vecs,
                       a.ws_carry, a.ws_cmax, out, a.H, a.L, a.m, a.seg_len, a.nseg);
    stage_event(a, 4);
    return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_all(const LaunchArgs& a) {
    constexpr int KSD = D < 32 ? 1 : D / 32;
    const long long om_head_vecs = a.omega_per_head ? (long long)(a.m / 16) * KSD * 64 : 0;
    const int om_heads = a.omega_per_head ? a.H : 1;
    vec8<T>* ompack = reinterpret_cast<vec8<T>*>(a.ws_ompack);
    hipStream_t st = a.stream;
    stage_event(a, 0);
    {
        const long long total = (long long)om_heads * (a.m / 16) * KSD * 64;
        const int blocks = (int)std::min<long long>((total + 255) / 256, 4096);
        hipLaunchKernelGGL((pack_omega_kernel<T, D>), dim3(blocks), dim3(256), 0, st, a.omega, ompack, om_heads, a.m);
    }
    stage_event(a, 1);
    const int BH = a.B * a.H;
    const T* q = reinterpret_cast<const T*>(a.q);
    const T* k = reinterpret_cast<const T*>(a.k);
    const T* v = reinterpret_cast<const T*>(a.v);
    T* out = reinterpret_cast<T*>(a.out);
    if (a.op == OpKind::Features) {
        const int tiles = (a.L + 15) / 16;
        const int blocks = (tiles + 3) / 4;
        hipLaunchKernelGGL((features_kernel<T, D>), dim3(blocks, BH), dim3(256), 0, st, q, ompack, om_head_vecs,
                           a.phi, a.log_scale, a.H, a.L, a.m, a.stabilize);
        return hipGetLastError();
    }
    const int nfg = (a.m + 255) / 256;
    const int wpg = std::min(a.m, 256) / 32;  // waves per feature group
    hipLaunchKernelGGL((kv_partial_kernel<T, D>), dim3(a.nseg, BH, nfg), dim3(64 * wpg), 0, st, k, v, ompack,
                       om_head_vecs, a.ws_partial, a.ws_pmax, a.H, a.L, a.m, a.seg_len, a.nseg);
    stage_event(a, 2);
    if (a.op == OpKind::Bidir) {
        hipLaunchKernelGGL((merge_scan_kernel<T, D>), dim3(a.m / 32, BH), dim3(256), 0, st, a.ws_partial, a.ws_pmax,
                           a.m, a.nseg, a.nseg, 0, reinterpret_cast<vec8<T>*>(a.ws_kvpack), a.ws_mmax, nullptr,
                           nullptr, 0);
        stage_event(a, 3);
        const int waves = 8;
        const int tok_per_wg = waves * 16 * (D >= 128 ? 2 : 4);
        const int blocks = (a.L + tok_per_wg - 1) / tok_per_wg;
        const size_t om_b = sizeof(vec8<T>) * 64 * (size_t)(a.m / 16) * KSD;
        const size_t kv_b = sizeof(vec8<T>) * 64 * (size_t)(D / 16 + 1) * (a.m / 32);
        const vec8<T>* kvp = reinterpret_cast<const vec8<T>*>(a.ws_kvpack);
        if (om_b + kv_b <= kMaxLds) {
            auto kern = bidir_out_kernel<T, D, true, true>;
            (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)(om_b + kv_b));
            hipLaunchKernelGGL(kern, dim3(blocks, BH), dim3(64 * waves), om_b + kv_b, st, q, ompack, om_head_vecs,
                               kvp, a.ws_mmax, out, a.H, a.L, a.m);
        } else if (kv_b <= kMaxLds) {
            auto kern = bidir_out_kernel<T, D, false, true>;
            (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kv_b);
            hipLaunchKernelGGL(kern, dim3(blocks, BH), dim3(64 * waves), kv_b, st, q, ompack, om_head_vecs, kvp,
                               a.ws_mmax, out, a.H, a.L, a.m);
        } else {
            auto kern = bidir_out_kernel<T, D, false, false>;
            hipLaunchKernelGGL(kern, dim3(blocks, BH), dim3(64 * waves), 0, st, q, ompack, om_head_vecs, kvp,
                               a.ws_mmax, out, a.H, a.L, a.m);
        }
        stage_event(a, 4);
    } else {
        hipLaunchKernelGGL((merge_scan_kernel<T, D>), dim3(a.m / 32, BH), dim3(256), 0, st, a.ws_partial, a.ws_pmax,
                           a.m, a.nseg, a.nseg, 1, nullptr, nullptr, a.ws_carry, a.ws_cmax, a.nseg);
        stage_event(a, 3);
        const CausalCfg cfg = causal_config(D, a.m);
        if (cfg.fw == 32) return launch_causal<T, D, 32, 8>(a, ompack, om_head_vecs, q, k, v, out);
        if constexpr (D <= 64) {
            return launch_causal<T, D, 64, 8>(a, ompack, om_head_vecs, q, k, v, out);
        } else {
            return launch_causal<T, D, 128, 4>(a, ompack, om_head_vecs, q, k, v, out);
        }
    }
    return hipGetLastError();
}

CausalCfg causal_config(int D, int m) {
    // Features per wave: the state slice FW x (D + 16) fp32 must fit the
    // register budget: <= 80 registers per lane at 2 waves per SIMD
    // (MAXW = 8), <= 288 at 1 wave per SIMD (MAXW = 4).
    CausalCfg c{0, 0, 0};
    if (m % 32 != 0) return c;
    if (D <= 64) {
        c.fw = (m % 64 == 0) ? 64 : 32;
        c.maxw = 8;
    } else if (m % 128 == 0) {
        c.fw = 128;
        c.maxw = 4;
    } else {
        c.fw = 32;
        c.maxw = 8;
    }
    c.w = m / c.fw;
    if (c.w > c.maxw) c = CausalCfg{0, 0, 0};
    return c;
}

size_t causal_smem_bytes(int dtype_bytes, int D, int m) {
    const CausalCfg c = causal_config(D, m);
    if (c.w == 0) return ~(size_t)0;
#define FAVOR_SMEM_CASE(TT, DD)                                           \
    switch (c.fw) {                                                        \
        case 32: return CausalSmem<TT, DD, 32>::bytes(c.w);                \
        case 64: return CausalSmem<TT, DD, 64>::bytes(c.w);                \
        default: return CausalSmem<TT, DD, 128>::bytes(c.w);               \
    }
    if (dtype_bytes == 2) {
        switch (D) {
            case 16: FAVOR_SMEM_CASE(bf16, 16)
            case 32: FAVOR_SMEM_CASE(bf16, 32)
            case 64: FAVOR_SMEM_CASE(bf16, 64)
            default: FAVOR_SMEM_CASE(bf16, 128)
        }
    }
    switch (D) {
        case 16: FAVOR_SMEM_CASE(float, 16)
        case 32: FAVOR_SMEM_CASE(float, 32)
        case 64: FAVOR_SMEM_CASE(float, 64)
        default: FAVOR_SMEM_CASE(float, 128)
    }
#undef FAVOR_SMEM_CASE
}

hipError_t launch(const LaunchArgs& a) {
    if (a.dtype_bytes == 2) {
        switch (a.D) {
            case 16: return launch_all<bf16, 16>(a);
            case 32: return launch_all<bf16, 32>(a);
            case 64: return launch_all<bf16, 64>(a);
            case 128: return launch_all<bf16, 128>(a);
        }
    } else {
        switch (a.D) {
            case 16: return launch_all<float, 16>(a);
            case 32: return launch_all<float, 32>(a);
            case 64: return launch_all<float, 64>(a);
            case 128: return launch_all<float, 128>(a);
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace favor
