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
// Kernels (three per attention call):
//   kv_partial      per (head, segment, feature group): sum_s phi(k_s)[v_s | 1]
//                   with a lazily raised key shift per wave
//   merge_scan      per (head, 32-feature block): total over segments
//                   (bidirectional) or exclusive prefix (causal carry-in);
//                   also packs log2(e) omega in operand order
//   bidir_out       phi(q) . [KV | z] for tiles of 32 queries per wave
//   causal_tile     per (head, segment), bf16, d = 64, m <= 256: chunked scan,
//                   64 tokens per step; four query waves (one 16-query tile
//                   each) and four key/state waves (key projection by
//                   feature slice, state by value columns)
//   causal_chunk    per (head, segment), every other shape: chunked scan,
//                   32 tokens per step, state split by features
// and, for bidirectional plans with one segment per head, one kernel per call:
//   bidir_head      per head: the sums by feature-parallel waves, then the
//                   output pass (m <= 256)
//   bidir_small     per head, m = 32: the sums by key-parallel waves, then
//                   the output pass
// and for the features API:
//   pack_omega      omega fp32 -> log2(e) omega in operand order
//   features        phi(x) written to memory
#include "favor_device.h"
#include "favor_kernels.h"

#include <algorithm>
#include <type_traits>

namespace favor {

// d = 16 in bf16: the 32-deep contraction of a bf16 matrix instruction has
// 16 slots of padding.  Instead of zeros they carry the input row again
// (x operand) against the low part of log2(e) omega, bf16(v - bf16(v)) for
// v = log2(e) omega in fp32 (projection operand), so that one instruction
// computes x . (hi + lo): the projection then carries log2(e) omega to
// about 2^-17 instead of bf16's 2^-9, at no extra matrix work.  The rounding
// of that operand is otherwise the largest error term of the bf16 path, and
// at d = 16 it reaches the 2e-2 bar on some heads.  Row norms never include
// the repeated half.  fp32 keeps zero padding (its low part is 0).
template <typename T, int D>
inline constexpr bool kSplitD16 = sizeof(T) == 2 && D == 16;

// ---------------------------------------------------------------------------
// omega packing: A-operand order for the projection D[F x T] = Omega'[F x d] X^T.
// Entry ((ft * KSD + ks) * 64 + lane) holds Omega'[16 ft + r][32 ks + 8 g + j]
// (d = 16 in bf16: the low part of Omega'[16 ft + r][8 g - 16 + j] for g >= 2).
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
            if (c < D) {
                v[j] = (T)(omega[((size_t)h * m + f) * D + c] * kLog2e);
            } else if (kSplitD16<T, D>) {  // the low part (see kSplitD16)
                const float x = omega[((size_t)h * m + f) * D + c - D] * kLog2e;
                v[j] = (T)(x - (float)(T)x);
            } else {
                v[j] = (T)0.0f;
            }
        }
        out[idx] = v;
    }
}

// ---------------------------------------------------------------------------
// Swizzled LDS layouts (bank-conflict free for row reads, 16-lane row-chunk
// reads and transpose reads alike; the row strides are 8 words mod 32).
// 64-column bf16 tile: the 16-byte chunk c of row r sits at chunk c ^ ((r >> 2) & 1).
constexpr int kSwzTileRS = 80;
__device__ __forceinline__ int swz_tile(int row, int col) {
    return row * kSwzTileRS + (((col >> 3) ^ ((row >> 2) & 1)) << 3) + (col & 7);
}
// Row-major bf16 array of row stride RS: the 8-byte chunk c of row r sits at
// chunk c ^ ((r >> 2) & 3).
template <int RS>
__device__ __forceinline__ int swz_rows(int row, int col) {
    return row * RS + (((col >> 2) ^ ((row >> 2) & 3)) << 2) + (col & 3);
}
// Both swizzles only permute chunks inside aligned 16-column groups and
// depend on row bits 2..3, so for row0 and col0 multiples of 16,
// off(row0 + r, col0 + c) = off(r, c) + row0 * RS + col0: a lane offset plus
// a constant (an immediate in the LDS instruction).
//
// kappa_col (rows {4g..4g+3, 16+4g..16+4g+3} of column r) in a swizzled array:
// p = base + lane offset + row0 * RS + col0, with the lane offset from
// kappa_lane_off(); the second read is 16 rows further.
template <typename Off>
__device__ __forceinline__ int kappa_lane_off(int lane, Off off) {
    const int q = lane >> 4, s = lane & 15;
    return off(4 * q + (s >> 2), 4 * (s & 3));
}
template <int RS>
__device__ __forceinline__ bf16x8 kappa_col_at(const bf16* p) {
    const bf16x4 lo = lds_read_tr16(p);
    const bf16x4 hi = lds_read_tr16(p + 16 * RS);
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// The (up to three) tensors a prefetch moves, passed by value: element i is a
// select between registers.  An array of pointers would be indexed at run
// time (the compiler turns a select between two array loads into one load at
// a selected index) and kept in scratch memory.
template <typename P>
struct Ptrs {
    P p0, p1, p2;
    __device__ __forceinline__ P at(int i) const { return i == 2 ? p2 : (i == 1 ? p1 : p0); }
};

// ---------------------------------------------------------------------------
// Tile prefetch by NTHR threads (thread index taken modulo NTHR, so the
// group can be any aligned block of NTHR threads): NTEN tensors, each a
// ROWS-row tile of D columns, split into
// 8-element chunks (chunk c of a tensor = row c / (D/8), columns 8 (c % (D/8))).
// load() issues global loads into registers; store() writes them to LDS
// tiles and, for the tensors in `norm_mask`, the row constants
// -log2(e)|x|^2/2, each summed over the D/8 consecutive lanes that hold one
// row (DPP, no LDS round trip).
// ---------------------------------------------------------------------------
template <typename T, int D, int NTHR, int NTEN, int ROWS = 32>
struct Prefetch {
    static constexpr int CPR = D / 8;
    static constexpr int CH = ROWS * CPR;
    static constexpr int TOT = CH * NTEN;
    static constexpr int PER = (TOT + NTHR - 1) / NTHR;
    vec8<T> v[PER];

    // Branch-free (so the compiler can count the loads in flight): rows are
    // clamped to t_max, a valid row of every tensor; rows at or past t_end
    // are replaced by zeros when stored.
    // chunk index of load i: tensor and position in it (compile-time tensor
    // when every tensor is a whole number of thread blocks)
    __device__ __forceinline__ static void where(int i, int& tn, int& cc) {
        if constexpr (CH % NTHR == 0) {
            tn = (i * NTHR) / CH;
            cc = (i * NTHR) % CH + (int)(threadIdx.x % NTHR);
        } else {
            int c = (int)(threadIdx.x % NTHR) + i * NTHR;
            if (TOT % NTHR != 0) c = min(c, TOT - 1);
            tn = c / CH;
            cc = c % CH;
        }
    }
    __device__ __forceinline__ void load(Ptrs<const T*> src, int t0, int t_max) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            int tn, cc;
            where(i, tn, cc);
            const int t = min(t0 + cc / CPR, t_max);
            v[i] = gload8(src.at(tn) + (size_t)t * D + 8 * (cc % CPR));
        }
    }
    // SWZ: the destination tiles use swz_tile (bf16, D = 64).  Tiles with
    // every row valid (the common case, a wave-uniform test) take a copy of
    // the code without the zeroing selects.
    // NEG_TAIL: rows at or past t_end get the row constant -inf instead of
    // that of a zero row, so a projection initialised with it masks them.
    template <bool SWZ = false, bool NEG_TAIL = false>
    __device__ __forceinline__ void store(Ptrs<T*> dst, float* nrm, int norm_mask, int t0, int t_end) const {
        if (t0 + ROWS <= t_end)
            store_rows<SWZ, false, NEG_TAIL>(dst, nrm, norm_mask, t0, t_end);
        else
            store_rows<SWZ, true, NEG_TAIL>(dst, nrm, norm_mask, t0, t_end);
    }
    template <bool SWZ, bool MASK, bool NEG_TAIL = false>
    __device__ __forceinline__ void store_rows(Ptrs<T*> dst, float* nrm, int norm_mask, int t0, int t_end) const {
        constexpr int RS = LdsTile<T, D>::RS;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int c = (int)(threadIdx.x % NTHR) + i * NTHR;
            if (TOT % NTHR == 0 || c < TOT) {
                int tn, cc;
                where(i, tn, cc);
                const int row = cc / CPR, col = 8 * (cc % CPR);
                vec8<T> x = v[i];
                if (MASK && t0 + row >= t_end) x = zero8<T>();
                // a select between registers (not an indexed array) also
                // keeps the LDS address space visible: no flat stores
                T* d = dst.at(tn);
                int off = row * RS + col;
                if constexpr (SWZ) off = swz_tile(row, col);
                *reinterpret_cast<vec8<T>*>(d + off) = x;
                if ((norm_mask >> tn) & 1) {
                    float ss = sumsq8(x);
                    ss = group_sum<CPR>(ss);
                    if (col == 0)
                        nrm[tn * ROWS + row] = (NEG_TAIL && MASK && t0 + row >= t_end) ? kNegInf : -0.5f * kLog2e * ss;
                }
            }
        }
    }
};

// Operand of 16 rows (row0 + r) x 8 columns (32 ks + 8 g ..) of a staged
// tile: the projection input (A for D[T x F], B for D[F x T]).
template <typename T, int D>
__device__ __forceinline__ vec8<T> row_operand(const T* tile, int row, int ks, int g) {
    constexpr int RS = LdsTile<T, D>::RS;
    if (D < 32 && g >= D / 8) {
        if constexpr (kSplitD16<T, D>) return *reinterpret_cast<const vec8<T>*>(tile + row * RS + 8 * (g - 2));
        return zero8<T>();
    }
    return *reinterpret_cast<const vec8<T>*>(tile + row * RS + 32 * ks + 8 * g);
}

// Projection operand (Omega' rows f0 + 16 ft + r, columns 32 ks + 8 g ..)
// straight from the fp32 projection, scaled by log2(e).
template <typename T, int D>
__device__ __forceinline__ vec8<T> omega_operand(const float* om_head, int f, int ks, int g) {
    vec8<T> v;
    const int c0 = 32 * ks + 8 * g;
    if (c0 >= D && !kSplitD16<T, D>) return zero8<T>();
    const bool lo = c0 >= D;  // the low part (see kSplitD16)
    const int c = lo ? c0 - D : c0;
    const float4 a = *reinterpret_cast<const float4*>(om_head + (size_t)f * D + c);
    const float4 b = *reinterpret_cast<const float4*>(om_head + (size_t)f * D + c + 4);
    const float x[8] = {a.x * kLog2e, a.y * kLog2e, a.z * kLog2e, a.w * kLog2e,
                        b.x * kLog2e, b.y * kLog2e, b.z * kLog2e, b.w * kLog2e};
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = lo ? (T)(x[j] - (float)(T)x[j]) : (T)x[j];
    return v;
}

// ---------------------------------------------------------------------------
// Segment sums (partials, causal carries) of one (head, segment) in the
// matrix-core result layout, so that every lane moves 4 consecutive
// elements (aligned):
//   V part: ((ft * D/16 + nt) * 64 + lane) * 4 + i holds S[16 ft + 4 g + i][16 nt + r]
//   z part: m * D + f holds S[f][D] (the sum of phi)
// m (D + 1) elements in all, stored in the input type: fp32 for fp32 inputs;
// bf16 for bf16 inputs, whose downstream operands (the output contraction's
// [KV | z], the scan's state products) are rounded to bf16 anyway.  The sums
// are accumulated in fp32 and rounded once when stored.
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ size_t seg_v_off(int ft, int nt, int lane) {
    return ((size_t)(ft * (D / 16) + nt) * 64 + lane) * 4;
}

// ---------------------------------------------------------------------------
// kv_partial: one workgroup (8 waves) per (segment, head, group of <= 256
// features).  Wave w owns 32 features.  Steps of 64 tokens are prefetched PD
// ahead into registers and staged into one of three LDS slots (one barrier
// per step).  The loop is software-pipelined: step i's exponentials, step
// i+1's projection and step i's update are independent and interleave.
// Projection D[T x F] = K Omega'^T with the accumulator initialised to
// -log2(e)|k|^2/2 - M: values are relative to the wave's shift M, which is
// set from the first step's maximum and afterwards raised lazily (a
// lane-local test; the wave-wide max only when some value exceeds kTau), with
// exact rescaling of the sums.  phi is the A operand and [V | 1] (kappa
// order, transpose reads) the B operand of the update.
// Output: partial[bh][seg][f][0..D] (column D = sum of phi; input type),
// pmax[bh][seg][f/32].
// ---------------------------------------------------------------------------
// The sums of one (segment, head, feature group), by the eight waves of the
// calling workgroup: the kernel below runs one per workgroup, and the
// one-kernel bidirectional path runs it for a whole head.
template <typename T, int D, int PD, bool RELU>
__device__ __forceinline__ void kv_partial_block(const T* __restrict__ k, const T* __restrict__ v,
                                                 const float* __restrict__ omega, int om_per_head,
                                                 T* __restrict__ partial, float* __restrict__ pmax, int H, int L,
                                                 int m, int seg_len, int nseg, int seg, int bh, int fgroup,
                                                 vec8<T>* __restrict__ om_out = nullptr) {
    using TL = LdsTile<T, D>;
    constexpr int RS = TL::RS;
    constexpr int KSD = D < 32 ? 1 : D / 32;
    constexpr int NT = D / 16 + 1;
    constexpr int FW = 32;
    constexpr int NFT = FW / 16;
    constexpr int ST = 64;         // tokens per step
    constexpr int TILE = ST * RS;  // elements of one staged tensor
    __shared__ __attribute__((aligned(16))) T tiles[3][2][TILE];
    __shared__ float norms[3][ST];

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, r = lane & 15, g = lane >> 4;
    const int h = bh % H;
    const int f0 = fgroup * 256 + w * FW;
    // The last feature group may have fewer than 8 waves' worth of features:
    // the spare waves still load tiles and meet every barrier, but compute and
    // write nothing.
    const bool active = f0 < m;
    const int t_begin = seg * seg_len;
    const int t_end = min(L, t_begin + seg_len);
    const int nsteps = (t_end - t_begin + ST - 1) / ST;
    const size_t xbase = (size_t)bh * L * D;
    const float* omh = omega + (om_per_head ? (size_t)h * m * D : 0);

    vec8<T> om[NFT][KSD];
#pragma unroll
    for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) om[ft][ks] = omega_operand<T, D>(omh, (active ? f0 : 0) + 16 * ft + r, ks, g);
    // the packed projection for the causal scan, when no merge pass follows
    // to pack it (first segment of each projection's first head)
    if (om_out && active && seg == 0 && (om_per_head ? bh < H : bh == 0)) {
        vec8<T>* dst = om_out + (size_t)(om_per_head ? h : 0) * (m / 16) * KSD * 64;
#pragma unroll
        for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
            for (int ks = 0; ks < KSD; ++ks) dst[((size_t)(f0 / 16 + ft) * KSD + ks) * 64 + lane] = om[ft][ks];
    }

    f4 kv[NFT][NT];
#pragma unroll
    for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) kv[ft][nt] = f4splat(0.0f);
    float M = 0.0f;

    const Ptrs<const T*> src{k + xbase, v + xbase, v + xbase};
    // lane part of the transpose-read addresses of the V tiles: each read is
    // then the step's slot base plus this offset plus a constant
    const int voff = kappa_lane_off(lane, [](int row, int col) { return row * RS + col; });
    // PD steps in flight in registers (global latency).  Every unrolled step
    // stores, loads and meets the barrier (loads past the last step re-read
    // it, from cache), so the load count is static.
    Prefetch<T, D, 512, 2, ST> pf[PD];
#pragma unroll
    for (int u = 0; u < PD; ++u) pf[u].load(src, t_begin + ST * min(u, nsteps - 1), L - 1);

    // rows past the segment's end are staged as zeros with the row constant
    // -inf, so their features are 0 without a per-step test
    auto stage = [&](Prefetch<T, D, 512, 2, ST>& pr, int step) {
        const int sl = step % 3;
        const Ptrs<T*> dst{tiles[sl][0], tiles[sl][1], tiles[sl][1]};
        pr.template store<false, true>(dst, norms[sl], 1, t_begin + ST * min(step, nsteps - 1),
                                       step < nsteps ? t_end : -1);
        pr.load(src, t_begin + ST * min(step + PD, nsteps - 1), L - 1);
    };
    // projection of one step (p = exponent - M) and its lane-local maximum;
    // branch-free, so that a whole step is one block for the scheduler
    auto project = [&](int step, f4 (&p)[4][NFT]) -> float {
        const int sl = step % 3;
        const T* kt = tiles[sl][0];
        float lm = kNegInf;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            const f4 nr = *reinterpret_cast<const f4*>(&norms[sl][16 * tt + 4 * g]);
            f4 init;
            if constexpr (RELU) {
#pragma unroll
                for (int i = 0; i < 4; ++i) init[i] = nr[i] == kNegInf ? kNegInf : 0.0f;
            } else {
                init = nr - M;
            }
            vec8<T> x[KSD];
#pragma unroll
            for (int ks = 0; ks < KSD; ++ks) x[ks] = row_operand<T, D>(kt, 16 * tt + r, ks, g);
#pragma unroll
            for (int ft = 0; ft < NFT; ++ft) {
                p[tt][ft] = init;
#pragma unroll
                for (int ks = 0; ks < KSD; ++ks) p[tt][ft] = mma32(x[ks], om[ft][ks], p[tt][ft]);
            }
        }
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
                for (int i = 0; i < 4; ++i) lm = __builtin_fmaxf(lm, p[tt][ft][i]);
        return lm;
    };

    // projections of two consecutive steps, used in turn with the loop
    // unrolled by a multiple of two (no copies); with one step in flight
    // (large d, register-bound) the next step's projection is copied instead
    f4 pj[2][4][NFT];
    constexpr bool PING = PD > 1;
    constexpr int U = !PING ? 1 : (PD % 2 == 0 ? PD : 2 * PD);  // steps per unrolled iteration

    // step 0: stage, project, and take its maximum as the shift
    stage(pf[0], 0);
    __syncthreads();
    if (active && RELU) {
        project(0, pj[0]);  // ReLU features: no shift
    } else if (active) {
        const float tm = wave_max_uniform(project(0, pj[0]));
        M = tm;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int ft = 0; ft < NFT; ++ft) pj[0][tt][ft] -= tm;
    }

    for (int i0 = 0; i0 < nsteps; i0 += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int it = i0 + u;
            stage(pf[(u + 1) % PD], it + 1);
            __syncthreads();
            if (active && it < nsteps) {
                f4(&pc)[4][NFT] = pj[PING ? (u & 1) : 0];
                f4(&pn)[4][NFT] = pj[PING ? ((u + 1) & 1) : 1];
                // this step's features (exponentials of values already relative
                // to M), the next step's projection and this step's update are
                // independent and interleave; the shift test for the next step
                // comes last, so a raise rescales sums that include this step
                vec8<T> a[2][NFT];
#pragma unroll
                for (int ks2 = 0; ks2 < 2; ++ks2)  // tokens 32 ks2 .. 32 ks2 + 31
#pragma unroll
                    for (int ft = 0; ft < NFT; ++ft) {
                        f4 e0, e1;
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            e0[i] = feat<RELU>(pc[2 * ks2][ft][i]);
                            e1[i] = feat<RELU>(pc[2 * ks2 + 1][ft][i]);
                        }
                        a[ks2][ft] = pack8t<T>(e0, e1);
                    }
                // the next step's projection (on the last step the same step
                // again, unused: no branch in the step)
                const bool more = it + 1 < nsteps;
                const float lm = project(more ? it + 1 : it, pn);
                const T* vt = tiles[it % 3][1];
                // the lane offset passes through an empty asm statement, so
                // the compiler cannot hoist (offset + constant) pairs out of
                // the loop into separate registers: every read below is one
                // address per step plus an immediate
                int vo = voff;
                asm volatile("" : "+v"(vo));
                const T* vl = vt + vo;
#pragma unroll
                for (int ks2 = 0; ks2 < 2; ++ks2) {
                    const T* vk = vt + 32 * ks2 * RS;
#pragma unroll
                    for (int nt = 0; nt < NT - 1; ++nt) {
                        vec8<T> vb;
                        if constexpr (sizeof(T) == 2)
                            vb = kappa_col_at<RS>(vl + 32 * ks2 * RS + 16 * nt);
                        else
                            vb = kappa_col<RS>(vk, 16 * nt, lane);
#pragma unroll
                        for (int ft = 0; ft < NFT; ++ft) kv[ft][nt] = mma32(a[ks2][ft], vb, kv[ft][nt]);
                    }
                    const vec8<T> ones = splat8<T>(1.0f);
#pragma unroll
                    for (int ft = 0; ft < NFT; ++ft) kv[ft][NT - 1] = mma32(a[ks2][ft], ones, kv[ft][NT - 1]);
                }
                if (!RELU && more && wave_any(lm > kTau)) {
                    const float tm = wave_max_uniform(lm);  // raise M by tm
                    const float sc = exp2f_fast(-tm);
#pragma unroll
                    for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
                        for (int nt = 0; nt < NT; ++nt) kv[ft][nt] *= sc;
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                        for (int ft = 0; ft < NFT; ++ft) pn[tt][ft] -= tm;
                    M += tm;
                }
                if constexpr (!PING) {
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                        for (int ft = 0; ft < NFT; ++ft) pc[tt][ft] = pn[tt][ft];
                }
            }
        }
    }

    if (!active) return;
    T* pp = partial + ((size_t)bh * nseg + seg) * (size_t)m * (D + 1);
#pragma unroll
    for (int ft = 0; ft < NFT; ++ft) {
        const int fg = f0 / 16 + ft;
#pragma unroll
        for (int nt = 0; nt < NT - 1; ++nt) store4(pp + seg_v_off<D>(fg, nt, lane), kv[ft][nt]);
        if (r == 0) store4(pp + (size_t)m * D + 16 * fg + 4 * g, kv[ft][NT - 1]);
    }
    if (lane == 0) pmax[((size_t)bh * nseg + seg) * (m / 32) + f0 / 32] = M;
}

template <typename T, int D, int PD, bool RELU>
__global__ __launch_bounds__(512) void kv_partial_kernel(const T* __restrict__ k, const T* __restrict__ v,
                                                         const float* __restrict__ omega, int om_per_head,
                                                         T* __restrict__ partial, float* __restrict__ pmax, int H,
                                                         int L, int m, int seg_len, int nseg,
                                                         vec8<T>* __restrict__ om_out) {
    kv_partial_block<T, D, PD, RELU>(k, v, omega, om_per_head, partial, pmax, H, L, m, seg_len, nseg, blockIdx.x,
                                     blockIdx.y, blockIdx.z, om_out);
}

// ---------------------------------------------------------------------------
// merge_scan: one workgroup per (32-feature block, head, half); thread
// (mt, lane) owns one 4-float piece of a result tile: feature tile
// 2 fb + half, and mt < D/16 a value tile or mt = D/16 the z row.
// mode 0 (bidirectional): sum over the segment partials, rescaled to the
//   block's maximum shift; written as the packed A operand of the output
//   contraction (kvpack[bh][fb][mt][lane], kappa order over the block's 32
//   features, this half filling slots 4 half .. 4 half + 3; mt = D/16 is the
//   z row replicated) and mmax[bh][fb].
// mode 1 (causal): carry[bh][s] = sum over segments s' < s, scaled to
//   cmax[bh][s][fb] = max over s' <= s of the partial shifts (every key of
//   segment s has exponents <= cmax + kTau), in the segment-sum layout and
//   type (summed in fp32).
//   A carried-in state (state_in, per head: G[m][D] row-major, z[m], and a
//   natural-log shift s, true values = stored * e^s) enters as a segment
//   before the first, with shift s log2(e) in every block; state_out
//   receives the inclusive total over all segments in the same format, with
//   one shift per head (the largest block shift).
// Both modes also pack log2(e) Omega for the block's 32 features (A-operand
// order of the projection D[F x T]) into ompack, once per projection.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(64 * (D / 16 + 1)) void merge_scan_kernel(
    const T* __restrict__ partial, const float* __restrict__ pmax, const float* __restrict__ omega, int om_per_head,
    int H, int m, int nseg, int mode, vec8<T>* __restrict__ kvpack, float* __restrict__ mmax,
    T* __restrict__ carry, float* __restrict__ cmax, vec8<T>* __restrict__ ompack,
    const float* __restrict__ state_in, float* __restrict__ state_out) {
    constexpr int KSD = D < 32 ? 1 : D / 32;
    constexpr int NTV = D / 16;
    constexpr int NMT = NTV + 1;
    const int fb = blockIdx.x, bh = blockIdx.y, half = blockIdx.z;
    const int h = bh % H, b = bh / H;
    const int nfb = m / 32;
    const int mt = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 4, r = lane & 15;
    const size_t seg_stride = (size_t)m * (D + 1);
    const T* pb = partial + (size_t)bh * nseg * seg_stride;
    const float* pm = pmax + (size_t)bh * nseg * nfb;

    if (b == 0 && (om_per_head || h == 0)) {
        const float* omh = omega + (om_per_head ? (size_t)h * m * D : 0);
        vec8<T>* dst = ompack + (size_t)(om_per_head ? h : 0) * (m / 16) * KSD * 64;
        for (int e = threadIdx.x; e < KSD * 64; e += blockDim.x) {
            const int ln = e % 64, ks = e / 64, ft = 2 * fb + half;
            dst[((size_t)ft * KSD + ks) * 64 + ln] = omega_operand<T, D>(omh, 16 * ft + (ln & 15), ks, ln >> 4);
        }
    }

    // this thread's 4-float piece of a segment sum
    const int ft = 2 * fb + half;
    const size_t o = mt < NTV ? seg_v_off<D>(ft, mt, lane) : (size_t)m * D + 16 * ft + 4 * g;
    constexpr int NB = 8;  // segments loaded per batch

    // the block's segment shifts, gathered once into LDS (one load each, all
    // in flight together, instead of a dependent scalar load per segment)
    __shared__ float pms[kMaxSeg];
    for (int s = threadIdx.x; s < nseg; s += blockDim.x) pms[s] = pm[(size_t)s * nfb + fb];
    __syncthreads();

    if (mode == 0) {
        float Ms = kNegInf;
        for (int s = 0; s < nseg; ++s) Ms = __builtin_fmaxf(Ms, pms[s]);
        f4 acc = f4splat(0.0f);
        for (int s0 = 0; s0 < nseg; s0 += NB) {
            f4 x[NB];
#pragma unroll
            for (int j = 0; j < NB; ++j)  // independent loads in flight
                x[j] = load4f(pb + (size_t)min(s0 + j, nseg - 1) * seg_stride + o);
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const float ms = s0 + j < nseg ? pms[s0 + j] : kNegInf;
                acc += (ms == kNegInf ? 0.0f : exp2f_fast(ms - Ms)) * x[j];
            }
        }
        typedef __attribute__((ext_vector_type(4))) T T4;
        T4 packed;
#pragma unroll
        for (int i = 0; i < 4; ++i) packed[i] = (T)acc[i];
        T4* dst = reinterpret_cast<T4*>(kvpack + (((size_t)bh * nfb + fb) * NMT + mt) * 64 + lane) + half;
        *dst = packed;
        if (threadIdx.x == 0 && half == 0) mmax[(size_t)bh * nfb + fb] = Ms;
    } else {
        T* cb = carry + (size_t)bh * nseg * seg_stride;
        const bool writer = mt < NTV || r == 0;  // the z row: one lane per 4 features
        const size_t st_stride = (size_t)m * (D + 1) + 1;
        // this thread's piece in the row-major state: features 16 ft + 4 g + i,
        // value column 16 mt + r (or z)
        auto st_index = [&](int i) -> size_t {
            const int f = 16 * ft + 4 * g + i;
            return mt < NTV ? (size_t)f * D + 16 * mt + r : (size_t)m * D + f;
        };
        f4 acc = f4splat(0.0f);
        float Mrun = kNegInf;
        float Min = kNegInf;  // carried-in shift, log2 units
        if (state_in) {
            const float* si = state_in + (size_t)bh * st_stride;
            Min = si[(size_t)m * (D + 1)] * kLog2e;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = si[st_index(i)];
            Mrun = Min;
        }
        for (int s0 = 0; s0 < nseg; s0 += NB) {
            f4 x[NB];
#pragma unroll
            for (int j = 0; j < NB; ++j)
                x[j] = load4f(pb + (size_t)min(s0 + j, nseg - 1) * seg_stride + o);
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const int s = s0 + j;
                if (s < nseg) {
                    const float ms = pms[s];
                    if (ms > Mrun) {
                        acc *= (Mrun == kNegInf ? 0.0f : exp2f_fast(Mrun - ms));
                        Mrun = ms;
                    }
                    if (writer) store4(cb + (size_t)s * seg_stride + o, acc);
                    if (ms != kNegInf) acc += exp2f_fast(ms - Mrun) * x[j];
                }
            }
        }
        if (half == 0) {
            // running maxima: thread s takes the maximum over segments <= s
            for (int s = threadIdx.x; s < nseg; s += blockDim.x) {
                float Mr = Min;
                for (int u = 0; u <= s; ++u) Mr = __builtin_fmaxf(Mr, pms[u]);
                cmax[((size_t)bh * nseg + s) * nfb + fb] = Mr;
            }
        }
        if (state_out) {
            // one shift per head: the largest over the carried-in shift and
            // every segment shift of every block
            __shared__ float red[64 * (D / 16 + 1)];
            float mx = Min;
            for (int e = threadIdx.x; e < nseg * nfb; e += blockDim.x) mx = __builtin_fmaxf(mx, pm[e]);
            red[threadIdx.x] = mx;
            __syncthreads();
            float Mall = kNegInf;
            for (int t = 0; t < (int)blockDim.x; ++t) Mall = __builtin_fmaxf(Mall, red[t]);
            const float sc = (Mrun == kNegInf) ? 0.0f : exp2f_fast(Mrun - Mall);
            float* so = state_out + (size_t)bh * st_stride;
            if (writer) {
#pragma unroll
                for (int i = 0; i < 4; ++i) so[st_index(i)] = sc * acc[i];
            }
            if (threadIdx.x == 0 && fb == 0 && half == 0)
                so[(size_t)m * (D + 1)] = (Mall == kNegInf) ? 0.0f : Mall * 0.69314718055994531f;
        }
    }
}

// ---------------------------------------------------------------------------
// bidir_out: workgroup = NW waves x (16 NTT) queries.  The projection operands
// (packed omega') and the output operands ([KV | z]^T) of the head are staged
// once in LDS.  Each wave loops over 32-feature chunks: project its NTT query
// tiles (D[F x T], lanes own token columns), keep a lazily raised per-query
// shift (lane-local test; the cross-lane max only when some lane needs it),
// exponentiate into the B operand and accumulate out^T[dims | z][T].
// ---------------------------------------------------------------------------
// Static LDS of the output pass (the per-block key shifts, m <= 512): the
// launcher leaves room for it beside the dynamically sized operand stages.
constexpr int kBidirOutStaticFloats = 512 / 32;

constexpr int kOutTiles = 2;  // query tiles (16 queries each) per wave

// The query operands of one wave's query tiles (rows tbase + 16 tt + r).
// Rows past the end repeat row L - 1: the products are column-independent
// and those columns are never stored, so the loads need no branch (a branch
// here makes the compiler wait for them before the operand staging).
template <typename T, int D>
__device__ __forceinline__ void load_queries(const T* __restrict__ q, size_t xbase, int L, int tbase,
                                             vec8<T> (&xq)[kOutTiles][D < 32 ? 1 : D / 32]) {
    constexpr int KSD = D < 32 ? 1 : D / 32;
    const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int tt = 0; tt < kOutTiles; ++tt) {
        const int t = min(tbase + 16 * tt + r, L - 1);
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) {
            if (D >= 32)
                xq[tt][ks] = load8(q + xbase + (size_t)t * D + 32 * ks + 8 * g);
            else if (kSplitD16<T, D>)  // d = 16, bf16: lanes g >= 2 repeat the row
                xq[tt][ks] = load8(q + xbase + (size_t)t * D + 8 * (g & 1));
            else  // d = 16, fp32: lanes g >= 2 hold the zero padding of the contraction
                xq[tt][ks] = g < D / 8 ? load8(q + xbase + (size_t)t * D + 8 * g) : zero8<T>();
        }
    }
}

// Their row constants -log2(e) |q|^2 / 2 (0 for ReLU features); computed
// after the operand staging is issued, so its latency overlaps the loads.
template <typename T, int D, bool RELU>
__device__ __forceinline__ void query_consts(const vec8<T> (&xq)[kOutTiles][D < 32 ? 1 : D / 32],
                                             float (&cq)[kOutTiles]) {
    constexpr int KSD = D < 32 ? 1 : D / 32;
    const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
    for (int tt = 0; tt < kOutTiles; ++tt) {
        float ss = 0.0f;
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) ss += sumsq8(xq[tt][ks]);
        if (D < 32 && g >= D / 8) ss = 0.0f;  // padding lanes: zeros or the repeated row
        cq[tt] = RELU ? 0.0f : -0.5f * kLog2e * col_sum(ss);
    }
}

// The output pass over one wave's query tiles, from the packed projection
// operands (om_src), the block-major [KV | z]^T operand (kv_src) and the
// per-block key shifts (offs, relative to the largest): loops over the m/32
// feature blocks and writes the normalised outputs.
template <typename T, int D, bool RELU>
__device__ __forceinline__ void out_tiles(const vec8<T>* om_src, const vec8<T>* kv_src, const float* offs,
                                          const vec8<T> (&xq)[kOutTiles][D < 32 ? 1 : D / 32],
                                          const float (&cq)[kOutTiles], T* __restrict__ out, size_t xbase, int L,
                                          int nfb, int tbase) {
    constexpr int KSD = D < 32 ? 1 : D / 32;
    constexpr int NMT = D / 16 + 1;
    constexpr int NTT = kOutTiles;
    const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
    f4 acc[NMT][NTT];
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) acc[mt][tt] = f4splat(0.0f);
    // per-query shift (log2 units), folded into the projection's
    // initialisation: every projected value is already relative to it
    float sref[NTT];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) sref[tt] = 0.0f;

    // projection of one 32-feature chunk for all query tiles; the next
    // chunk's projection is issued before the current chunk's exponentials
    auto project = [&](int fb, f4 (&pp)[NTT][2]) {
        const float off = offs[fb];
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) pp[tt][hh] = f4splat(cq[tt] + off - sref[tt]);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int ks = 0; ks < KSD; ++ks) {
                const vec8<T> a = om_src[((size_t)(2 * fb + hh) * KSD + ks) * 64 + lane];
#pragma unroll
                for (int tt = 0; tt < NTT; ++tt) pp[tt][hh] = mma32(a, xq[tt][ks], pp[tt][hh]);
            }
    };
    // projections of two consecutive 32-feature blocks, used in turn (the
    // loop body runs twice per iteration with the roles swapped: no copies)
    f4 pa[NTT][2], pb[NTT][2];
    project(0, pa);
    // the first block sets each query's shift to its maximum (ReLU: none)
#pragma unroll
    for (int tt = 0; tt < (RELU ? 0 : NTT); ++tt) {
        float lm = kNegInf;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int i = 0; i < 4; ++i) lm = __builtin_fmaxf(lm, pa[tt][hh][i]);
        sref[tt] = col_max(lm);
        pa[tt][0] -= sref[tt];
        pa[tt][1] -= sref[tt];
    }
    // block fb: its projection is in p; the next block's goes into pn
    auto block = [&](int fb, f4 (&p)[NTT][2], f4 (&pn)[NTT][2]) {
        const bool more = fb + 1 < nfb;
        if (more) project(fb + 1, pn);
        float lm[NTT];
        bool need = false;
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) {
            lm[tt] = kNegInf;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int i = 0; i < 4; ++i) lm[tt] = __builtin_fmaxf(lm[tt], p[tt][hh][i]);
            need |= lm[tt] > kTau;
        }
        if (!RELU && wave_any(need)) {
            // raise the shift of the queries that need it, rescaling their sums
            // and the values already projected with the old shift
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt) {
                const float cm = col_max(lm[tt]);
                const float up = cm > kTau ? cm : 0.0f;
                if (cm > kTau) {
                    const float sc = exp2f_fast(-cm);
#pragma unroll
                    for (int mt = 0; mt < NMT; ++mt) acc[mt][tt] *= sc;
                }
                sref[tt] += up;
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    p[tt][hh] -= up;
                    pn[tt][hh] -= up;
                }
            }
        }
        vec8<T> bq[NTT];
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) {
            f4 e0, e1;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                e0[i] = feat<RELU>(p[tt][0][i]);
                e1[i] = feat<RELU>(p[tt][1][i]);
            }
            bq[tt] = pack8t<T>(e0, e1);
        }
        // the block's [KV | z]^T operands are contiguous (block-major layout):
        // one address per block plus immediate offsets
        const vec8<T>* kb = kv_src + (size_t)fb * NMT * 64 + lane;
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) {
            const vec8<T> a = kb[mt * 64];
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt) acc[mt][tt] = mma32(a, bq[tt], acc[mt][tt]);
        }
    };
    int fb = 0;
    for (; fb + 1 < nfb; fb += 2) {
        block(fb, pa, pb);
        block(fb + 1, pb, pa);
    }
    if (fb < nfb) block(fb, pa, pb);
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) {
        const int t = tbase + 16 * tt + r;
        if (t >= L) continue;
        const float inv = 1.0f / acc[NMT - 1][tt][0];
#pragma unroll
        for (int mt = 0; mt < NMT - 1; ++mt) store4(out + xbase + (size_t)t * D + 16 * mt + 4 * g, acc[mt][tt] * inv);
    }
}


template <typename T, int D, bool OM_LDS, bool KV_LDS, int NW, bool RELU>
__global__ __launch_bounds__(64 * NW) void bidir_out_kernel(const T* __restrict__ q, const vec8<T>* __restrict__ ompack,
                                                        long long om_head_vecs, const vec8<T>* __restrict__ kvpack,
                                                        const float* __restrict__ mmax, T* __restrict__ out, int H,
                                                        int L, int m) {
    constexpr int KSD = D < 32 ? 1 : D / 32;
    constexpr int NMT = D / 16 + 1;
    extern __shared__ __attribute__((aligned(16))) char smem_raw[];
    const int nft = m / 16, nfb = m / 32;
    vec8<T>* kv_stage = reinterpret_cast<vec8<T>*>(smem_raw);
    vec8<T>* om_stage = kv_stage + (KV_LDS ? (size_t)NMT * nfb * 64 : 0);

    const int w = threadIdx.x >> 6;
    const int bh = blockIdx.y, h = bh % H;
    const int tbase = (blockIdx.x * (blockDim.x >> 6) + w) * (16 * kOutTiles);
    const size_t xbase = (size_t)bh * L * D;

    // query operands first, so their latency overlaps the staging below
    vec8<T> xq[kOutTiles][KSD];
    load_queries<T, D>(q, xbase, L, tbase, xq);
    const vec8<T>* omh = ompack + (size_t)(om_head_vecs ? h : 0) * (size_t)om_head_vecs;
    const vec8<T>* kvh = kvpack + (size_t)bh * NMT * nfb * 64;
    if (OM_LDS) copy_to_lds_async<64 * NW>(om_stage, omh, nft * KSD * 64);
    if (KV_LDS) copy_to_lds_async<64 * NW>(kv_stage, kvh, NMT * nfb * 64);
    const vec8<T>* om_src = OM_LDS ? om_stage : omh;
    const vec8<T>* kv_src = KV_LDS ? kv_stage : kvh;
    float Mstar = kNegInf;
    for (int fb = 0; fb < nfb; ++fb) Mstar = __builtin_fmaxf(Mstar, mmax[(size_t)bh * nfb + fb]);
    // per-block key shift relative to the largest one (<= 0; -inf for an
    // empty block), read once per block in the loop
    __shared__ float offs[kBidirOutStaticFloats];
    if ((int)threadIdx.x < nfb) {
        const float mb = mmax[(size_t)bh * nfb + threadIdx.x];
        offs[threadIdx.x] = RELU ? 0.0f : (mb == kNegInf) ? kNegInf : mb - Mstar;
    }
    float cq[kOutTiles];
    query_consts<T, D, RELU>(xq, cq);
    lds_dma_wait();
    __syncthreads();
    if (tbase >= L) return;
    out_tiles<T, D, RELU>(om_src, kv_src, offs, xq, cq, out, xbase, L, nfb, tbase);
}

// ---------------------------------------------------------------------------
// bidir_head: the whole bidirectional operation of one head in one workgroup
// of eight waves, for plans that give each head a single segment (short
// sequences, or enough heads to fill the chip; m <= 256): the head's sums
// over the whole sequence (kv_partial_block), then the output operands built
// straight into LDS (with one segment the merge is a conversion: the packed
// projection from fp32, [KV | z]^T block-major from the sums, the per-block
// shifts), then the output pass, each wave taking query tiles in turn.  One
// launch instead of three; the results equal those of the three kernels on
// the same one-segment plan.
// ---------------------------------------------------------------------------
template <typename T, int D, int PD, bool RELU>
__global__ __launch_bounds__(512) void bidir_head_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                         const T* __restrict__ v, const float* __restrict__ omega,
                                                         int om_per_head, T* __restrict__ partial,
                                                         float* __restrict__ pmax, T* __restrict__ out, int H, int L,
                                                         int m) {
    constexpr int KSD = D < 32 ? 1 : D / 32;
    constexpr int NTV = D / 16;
    constexpr int NMT = NTV + 1;
    typedef __attribute__((ext_vector_type(4))) T T4;
    extern __shared__ __attribute__((aligned(16))) char smem_raw[];
    const int nft = m / 16, nfb = m / 32;
    vec8<T>* kv_stage = reinterpret_cast<vec8<T>*>(smem_raw);
    vec8<T>* om_stage = kv_stage + (size_t)NMT * nfb * 64;
    const int bh = blockIdx.x, h = bh % H;

    kv_partial_block<T, D, PD, RELU>(k, v, omega, om_per_head, partial, pmax, H, L, m, L, 1, 0, bh, 0);
    __syncthreads();  // this workgroup's sums and shifts are written

    // [KV | z]^T operand, block-major (fb, mt, lane), each lane slot holding
    // the two 16-feature halves of block fb (the layout the merge pass writes)
    const T* ps = partial + (size_t)bh * m * (D + 1);
    for (int e = threadIdx.x; e < nfb * NMT * 64 * 2; e += blockDim.x) {
        const int half = e & 1, lane = (e >> 1) & 63, mt = (e >> 7) % NMT, fb = (e >> 7) / NMT;
        const int ft = 2 * fb + half;
        const size_t o = mt < NTV ? seg_v_off<D>(ft, mt, lane) : (size_t)m * D + 16 * ft + 4 * (lane >> 4);
        const f4 x = load4f(ps + o);
        T4 pk;
#pragma unroll
        for (int i = 0; i < 4; ++i) pk[i] = (T)x[i];
        reinterpret_cast<T4*>(kv_stage + ((size_t)fb * NMT + mt) * 64 + lane)[half] = pk;
    }
    // projection operands, packed from fp32 (the order the merge pass packs)
    const float* omh = omega + (om_per_head ? (size_t)h * m * D : 0);
    for (int e = threadIdx.x; e < nft * KSD * 64; e += blockDim.x) {
        const int ln = e & 63, ks = (e >> 6) % KSD, ft = (e >> 6) / KSD;
        om_stage[e] = omega_operand<T, D>(omh, 16 * ft + (ln & 15), ks, ln >> 4);
    }
    // per-block key shifts relative to the largest
    __shared__ float offs[kBidirOutStaticFloats];
    if ((int)threadIdx.x < nfb) {
        const float* pm = pmax + (size_t)bh * nfb;
        float Mstar = kNegInf;
        for (int fb = 0; fb < nfb; ++fb) Mstar = __builtin_fmaxf(Mstar, pm[fb]);
        const float mb = pm[threadIdx.x];
        offs[threadIdx.x] = RELU ? 0.0f : (mb == kNegInf) ? kNegInf : mb - Mstar;
    }
    __syncthreads();

    const size_t xbase = (size_t)bh * L * D;
    const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
    for (int tbase = w * 16 * kOutTiles; tbase < L; tbase += nw * 16 * kOutTiles) {
        vec8<T> xq[kOutTiles][KSD];
        float cq[kOutTiles];
        load_queries<T, D>(q, xbase, L, tbase, xq);
        query_consts<T, D, RELU>(xq, cq);
        out_tiles<T, D, RELU>(om_stage, kv_stage, offs, xq, cq, out, xbase, L, nfb, tbase);
    }
}

// ---------------------------------------------------------------------------
// bidir_small: the whole bidirectional operation of one head in one
// workgroup for 32 features (d <= 64 in bf16, d <= 32 in fp32; the kernel
// takes m = 64 as well, which measured no faster than the feature-split
// path).  With one segment per head
// the feature-parallel sums of bidir_head would keep only m/32 of the eight
// waves busy, so here the waves split the keys instead: wave w takes the
// 32-token chunks w, w + 8, ..., stages each chunk's K and V rows in LDS
// tiles of its own, projects the keys over all m features (D[T x F], the
// projection operands in registers), keeps its own lazily raised shift and
// accumulates phi(K)^T [V | 1] in registers.  The eight partial sums meet in
// LDS rescaled to the largest shift (exact up to rounding), are packed into
// the output operands, and the waves take the head's query tiles through the
// output loop shared with bidir_out.  Phase-one tiles and phase-two operands
// share the LDS.
// ---------------------------------------------------------------------------
template <typename T, int D, int M>
struct SmallSmem {
    static constexpr int RS = LdsTile<T, D>::RS;
    static constexpr int NT = D / 16 + 1, NFT = M / 16, NFB = M / 32, KSD = D < 32 ? 1 : D / 32;
    static constexpr size_t TILES = sizeof(T) * (size_t)8 * 2 * 32 * RS;  // K and V chunk of each wave
    static constexpr size_t NORMS = sizeof(float) * 8 * 32;
    static constexpr size_t SLOT = (size_t)NFT * NT * 64 * 4;  // one wave's sums (floats, D layout)
    static constexpr size_t SUMS = sizeof(float) * 8 * SLOT;
    static constexpr size_t KV = sizeof(vec8<T>) * (size_t)NT * NFB * 64;
    static constexpr size_t OM = sizeof(vec8<T>) * (size_t)NFT * KSD * 64;
    static constexpr size_t P1 = TILES + NORMS, P2 = SUMS + KV + OM;
    static constexpr size_t BYTES = P1 > P2 ? P1 : P2;
};

template <typename T, int D, int M, bool RELU>
__global__ __launch_bounds__(512) void bidir_small_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                          const T* __restrict__ v, const float* __restrict__ omega,
                                                          int om_per_head, T* __restrict__ out, int H, int L) {
    using SM = SmallSmem<T, D, M>;
    constexpr int RS = SM::RS, NT = SM::NT, NFT = SM::NFT, NFB = SM::NFB, KSD = SM::KSD;
    constexpr int CPR = D / 8;      // lanes per staged row, 8 elements each
    constexpr int PIECES = CPR / 2;  // 8-element pieces per lane of a 32-row chunk
    static_assert(M % 32 == 0 && M <= 64 && D >= 16 && D <= (sizeof(T) == 2 ? 64 : 32), "bidir_small shape");
    extern __shared__ __attribute__((aligned(16))) char smem_raw[];
    __shared__ float wave_shift[8];
    __shared__ float offs[NFB];
    const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int bh = blockIdx.x, h = bh % H;
    const size_t xbase = (size_t)bh * L * D;
    const float* omh = omega + (om_per_head ? (size_t)h * M * D : 0);
    T* kt = reinterpret_cast<T*>(smem_raw) + (size_t)w * 2 * 32 * RS;
    T* vt = kt + 32 * RS;
    float* nrm = reinterpret_cast<float*>(smem_raw + SM::TILES) + 32 * w;
    const int nch = (L + 31) / 32;

    // This lane's pieces of a 32-token chunk of K and V (row clamped to the
    // sequence: rows past the end are zeroed when staged).
    vec8<T> ck[PIECES], cv[PIECES];
    auto load_chunk = [&](int c) {
#pragma unroll
        for (int i = 0; i < PIECES; ++i) {
            const int pc = lane + 64 * i, row = pc / CPR, col = 8 * (pc % CPR);
            const size_t go = xbase + (size_t)min(32 * c + row, L - 1) * D + col;
            ck[i] = load8(k + go);
            cv[i] = load8(v + go);
        }
    };
    // Every load a wave needs first goes out at once: its first chunk of keys
    // and values, its first query tile, the projection operands.
    if (w < nch) load_chunk(w);
    vec8<T> xq[kOutTiles][KSD];
    const int tq0 = w * 16 * kOutTiles;
    if (tq0 < L) load_queries<T, D>(q, xbase, L, tq0, xq);
    vec8<T> om[NFT][KSD];  // projection operands of all M features (B of D[T x F])
#pragma unroll
    for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) om[ft][ks] = omega_operand<T, D>(omh, 16 * ft + r, ks, g);

    f4 kv[NFT][NT];
#pragma unroll
    for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) kv[ft][nt] = f4splat(0.0f);
    float Mw = kNegInf;  // this wave's key shift (log2 units); -inf until its first chunk
    const vec8<T> ones = splat8<T>(1.0f);

    for (int c = w; c < nch; c += 8) {
        const int t0 = 32 * c;
        // stage the chunk; rows past the end are zero with the row constant
        // -inf, so their features vanish
#pragma unroll
        for (int i = 0; i < PIECES; ++i) {
            const int pc = lane + 64 * i, row = pc / CPR, col = 8 * (pc % CPR);
            const bool in = t0 + row < L;
            const vec8<T> xk = in ? ck[i] : zero8<T>();
            *reinterpret_cast<vec8<T>*>(kt + row * RS + col) = xk;
            *reinterpret_cast<vec8<T>*>(vt + row * RS + col) = in ? cv[i] : zero8<T>();
            const float ss = group_sum<CPR>(sumsq8(xk));
            if (col == 0) nrm[row] = !in ? kNegInf : RELU ? 0.0f : -0.5f * kLog2e * ss;
        }
        // the next chunk of this wave is loaded while this one is computed
        if (c + 8 < nch) load_chunk(c + 8);
        // the tiles are this wave's own: ordering its LDS accesses suffices
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // projection of the 32 keys over all M features, relative to Mw
        f4 p[2][NFT];
        float lm = kNegInf;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const f4 nr = *reinterpret_cast<const f4*>(nrm + 16 * tt + 4 * g);
            const f4 init = (RELU || Mw == kNegInf) ? nr : nr - Mw;
            vec8<T> x[KSD];
#pragma unroll
            for (int ks = 0; ks < KSD; ++ks) x[ks] = row_operand<T, D>(kt, 16 * tt + r, ks, g);
#pragma unroll
            for (int ft = 0; ft < NFT; ++ft) {
                p[tt][ft] = init;
#pragma unroll
                for (int ks = 0; ks < KSD; ++ks) p[tt][ft] = mma32(x[ks], om[ft][ks], p[tt][ft]);
#pragma unroll
                for (int i = 0; i < 4; ++i) lm = __builtin_fmaxf(lm, p[tt][ft][i]);
            }
        }
        if (RELU) {
            Mw = 0.0f;
        } else if (Mw == kNegInf || wave_any(lm > kTau)) {
            // first chunk of the wave: its maximum becomes the shift (the chunk
            // holds at least one key); later: raise it, rescaling the sums
            const float tm = wave_max_uniform(lm);
            if (Mw != kNegInf) {
                const float sc = exp2f_fast(-tm);
#pragma unroll
                for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) kv[ft][nt] *= sc;
            }
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int ft = 0; ft < NFT; ++ft) p[tt][ft] -= tm;
            Mw = Mw == kNegInf ? tm : Mw + tm;
        }
        // features as the A operand (lane = feature, the 32 keys in kappa
        // order) and the update of the sums
        vec8<T> a[NFT];
#pragma unroll
        for (int ft = 0; ft < NFT; ++ft) {
            f4 e0, e1;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                e0[i] = feat<RELU>(p[0][ft][i]);
                e1[i] = feat<RELU>(p[1][ft][i]);
            }
            a[ft] = pack8t<T>(e0, e1);
        }
#pragma unroll
        for (int nt = 0; nt < NT - 1; ++nt) {
            const vec8<T> vb = kappa_col<RS>(vt, 16 * nt, lane);
#pragma unroll
            for (int ft = 0; ft < NFT; ++ft) kv[ft][nt] = mma32(a[ft], vb, kv[ft][nt]);
        }
#pragma unroll
        for (int ft = 0; ft < NFT; ++ft) kv[ft][NT - 1] = mma32(a[ft], ones, kv[ft][NT - 1]);
        // the next chunk's staging reuses the tiles
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

    // each wave's sums, rescaled to the largest shift, into a slot of its own
    // (the tiles are dead: the space becomes the slots)
    if (lane == 0) wave_shift[w] = Mw;
    __syncthreads();
    float Mall = kNegInf;
#pragma unroll
    for (int i = 0; i < 8; ++i) Mall = __builtin_fmaxf(Mall, wave_shift[i]);
    const float sc = Mw == kNegInf ? 0.0f : exp2f_fast(Mw - Mall);
    float* slots = reinterpret_cast<float*>(smem_raw);
#pragma unroll
    for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
            *reinterpret_cast<f4*>(slots + w * SM::SLOT + ((size_t)(ft * NT + nt) * 64 + lane) * 4) = sc * kv[ft][nt];
    __syncthreads();

    // output operands: [KV | z]^T block-major, the eight slots added in wave
    // order as they are packed, and the packed projection (which is every
    // wave's register operand: wave 0 stores its copy); one shift for all
    // keys, so no block offsets
    typedef __attribute__((ext_vector_type(4))) T T4;
    vec8<T>* kv_stage = reinterpret_cast<vec8<T>*>(smem_raw + SM::SUMS);
    vec8<T>* om_stage = kv_stage + (size_t)NT * NFB * 64;
    for (int e = threadIdx.x; e < NFB * NT * 64 * 2; e += blockDim.x) {
        const int half = e & 1, ln = (e >> 1) & 63, mt = (e >> 7) % NT, fb = (e >> 7) / NT;
        const float* sp = slots + ((size_t)((2 * fb + half) * NT + mt) * 64 + ln) * 4;
        f4 x = *reinterpret_cast<const f4*>(sp);
#pragma unroll
        for (int i = 1; i < 8; ++i) x += *reinterpret_cast<const f4*>(sp + i * SM::SLOT);
        T4 pk;
#pragma unroll
        for (int i = 0; i < 4; ++i) pk[i] = (T)x[i];
        reinterpret_cast<T4*>(kv_stage + ((size_t)fb * NT + mt) * 64 + ln)[half] = pk;
    }
    if (w == 0) {
#pragma unroll
        for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
            for (int ks = 0; ks < KSD; ++ks) om_stage[(ft * KSD + ks) * 64 + lane] = om[ft][ks];
    }
    if ((int)threadIdx.x < NFB) offs[threadIdx.x] = 0.0f;
    __syncthreads();

    // the query tiles, each one's successor loaded while it is computed
    for (int tb = tq0; tb < L; tb += 8 * 16 * kOutTiles) {
        float cq[kOutTiles];
        query_consts<T, D, RELU>(xq, cq);
        const bool more = tb + 8 * 16 * kOutTiles < L;
        vec8<T> xn[kOutTiles][KSD];
        if (more) load_queries<T, D>(q, xbase, L, tb + 8 * 16 * kOutTiles, xn);
        out_tiles<T, D, RELU>(om_stage, kv_stage, offs, xq, cq, out, xbase, L, NFB, tb);
        if (more) {
#pragma unroll
            for (int tt = 0; tt < kOutTiles; ++tt)
#pragma unroll
                for (int ks = 0; ks < KSD; ++ks) xq[tt][ks] = xn[tt][ks];
        }
    }
}

// ---------------------------------------------------------------------------
// causal_chunk: one workgroup (W waves) per (segment, head); wave w owns
// features [FW w, FW w + FW) and keeps its slice of the state
// G = sum phi(k) [v | 1]^T in registers (D layout: rows = features, columns =
// value dims / z).  Chunks of 32 tokens (Q, K, V) are prefetched PD ahead
// into registers and staged in one of two LDS slots, with one barrier per
// chunk.  Per chunk:
//   1. project Q and K (D[F x T]); query shift = per-token max over the wave's
//      features; key shift M = fixed for the segment (no key of the segment
//      exceeds it by more than kTau, from the partial pass);
//   2. intra-chunk S^T[T_k x T_q] = phi(K) phi(Q)^T over the wave's features,
//      masked to T_k <= T_q;
//   3. partial numerator/denominator over this wave's features:
//      out^T = G^T phi(Q)^T + [V | 1]^T S^T, written to LDS with its log-scale;
//   4. G += phi(K)^T [V | 1] (phi(K) written row-major by token, re-read in
//      kappa order with transpose reads);
//   5. the workgroup sums the waves' partials of a chunk (rescaled to a common
//      scale) and writes the outputs -- one chunk later when PARTS = 2.
// The state starts from the exclusive prefix of earlier segments (carry).
// ---------------------------------------------------------------------------
template <typename T, int D, int FW, int W, int PARTS>
struct CausalSmem {
    using TL = LdsTile<T, D>;
    using PTL = LdsTile<T, FW>;
    static constexpr int PART_STRIDE = D + 4;
    static constexpr size_t STAGE = (size_t)3 * TL::ELEMS;  // K, Q, V tiles (elements)
    static constexpr size_t OFF_PT = sizeof(T) * 2 * STAGE;
    static constexpr size_t OFF_PART = OFF_PT + sizeof(T) * (size_t)W * PTL::ELEMS;
    static constexpr size_t OFF_LAM = OFF_PART + sizeof(float) * (size_t)PARTS * W * 32 * PART_STRIDE;
    static constexpr size_t OFF_NRM = OFF_LAM + sizeof(float) * (size_t)PARTS * W * 32;
    static constexpr size_t BYTES = OFF_NRM + sizeof(float) * 2 * 2 * 32;
};

template <typename T, int D, int FW, int W, int PARTS>
__device__ __forceinline__ void causal_reduce(const float* part, const float* plam, T* out, size_t xbase, int t0,
                                              int t_end) {
    using SM = CausalSmem<T, D, FW, W, PARTS>;
    for (int item = threadIdx.x; item < 32 * (D / 8); item += 64 * W) {
        const int tl = item / (D / 8), c8 = item % (D / 8);
        const int t = t0 + tl;
        if (t >= t_end) continue;
        float lmax = kNegInf;
#pragma unroll
        for (int ww = 0; ww < W; ++ww) lmax = __builtin_fmaxf(lmax, plam[ww * 32 + tl]);
        float num[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        float den = 0.0f;
#pragma unroll
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
        const float inv = 1.0f / den;
        store4(out + xbase + (size_t)t * D + 8 * c8, f4{num[0] * inv, num[1] * inv, num[2] * inv, num[3] * inv});
        store4(out + xbase + (size_t)t * D + 8 * c8 + 4, f4{num[4] * inv, num[5] * inv, num[6] * inv, num[7] * inv});
    }
}

template <typename T, int D, int FW, int W, int PARTS, int PD, bool OM_REGS, bool RELU>
__global__ __launch_bounds__(64 * W) void causal_chunk_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                              const T* __restrict__ v, const vec8<T>* __restrict__ ompack,
                                                              long long om_head_vecs, const T* __restrict__ carry,
                                                              const float* __restrict__ cmax, T* __restrict__ out, int H,
                                                              int L, int m, int seg_len, int nseg) {
    using TL = LdsTile<T, D>;
    using PTL = LdsTile<T, FW>;
    using SM = CausalSmem<T, D, FW, W, PARTS>;
    constexpr int RS = TL::RS;
    constexpr int KSD = D < 32 ? 1 : D / 32;
    constexpr int NT = D / 16 + 1;
    constexpr int NFT = FW / 16;
    constexpr int KSF = FW / 32;
    constexpr int D1 = D + 1;
    extern __shared__ __attribute__((aligned(16))) char smem_raw[];
    T* stage = reinterpret_cast<T*>(smem_raw);
    T* pt_all = reinterpret_cast<T*>(smem_raw + SM::OFF_PT);
    float* part_all = reinterpret_cast<float*>(smem_raw + SM::OFF_PART);
    float* plam_all = reinterpret_cast<float*>(smem_raw + SM::OFF_LAM);
    float* nrm_all = reinterpret_cast<float*>(smem_raw + SM::OFF_NRM);

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, r = lane & 15, g = lane >> 4;
    const int seg = blockIdx.x, bh = blockIdx.y, h = bh % H;
    const int f0 = w * FW;
    const int nfb = m / 32;
    const int t_begin = seg * seg_len;
    const int t_end = min(L, t_begin + seg_len);
    const int nchunks = (t_end - t_begin + 31) / 32;
    const size_t xbase = (size_t)bh * L * D;
    const vec8<T>* omh = ompack + (size_t)(om_head_vecs ? h : 0) * (size_t)om_head_vecs;
    T* ptw = pt_all + (size_t)w * PTL::ELEMS;

    // prefetch the first chunks (K, Q, V); loads past the last chunk re-read it
    const Ptrs<const T*> src{k + xbase, q + xbase, v + xbase};
    Prefetch<T, D, 64 * W, 3> pf[PD];
#pragma unroll
    for (int u = 0; u < PD; ++u) pf[u].load(src, t_begin + 32 * min(u, nchunks - 1), L - 1);

    vec8<T> omr[OM_REGS ? NFT : 1][OM_REGS ? KSD : 1];
    if (OM_REGS) {
#pragma unroll
        for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
            for (int ks = 0; ks < KSD; ++ks) omr[ft][ks] = omh[((size_t)(f0 / 16 + ft) * KSD + ks) * 64 + lane];
    }

    // state from the carry-in, rescaled to one fixed key shift per wave
    float M = kNegInf;
    const float* cm = cmax + ((size_t)bh * nseg + seg) * nfb;
#pragma unroll
    for (int b = 0; b < KSF; ++b) M = __builtin_fmaxf(M, cm[f0 / 32 + b]);
    f4 G[NFT][NT];
    if (carry) {
        const T* cb = carry + ((size_t)bh * nseg + seg) * (size_t)m * D1;
#pragma unroll
        for (int ft = 0; ft < NFT; ++ft) {
            const float mb = cm[(f0 + 16 * ft) / 32];
            const float sc = (mb == kNegInf) ? 0.0f : exp2f_fast(mb - M);
            const int fg = f0 / 16 + ft;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const size_t o = nt < NT - 1 ? seg_v_off<D>(fg, nt, lane) : (size_t)m * D + 16 * fg + 4 * g;
                G[ft][nt] = sc * load4f(cb + o);
            }
        }
    } else {  // no carry: the scan starts from a zero state
#pragma unroll
        for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) G[ft][nt] = f4splat(0.0f);
    }

    for (int i0 = 0; i0 < nchunks; i0 += PD) {
#pragma unroll
        for (int u = 0; u < PD; ++u) {
            const int ci = i0 + u;
            const int slot = ci & 1;
            const int t0 = t_begin + 32 * ci;
            T* kt = stage + (size_t)slot * SM::STAGE;
            T* qt = kt + TL::ELEMS;
            T* vt = qt + TL::ELEMS;
            float* nrm = nrm_all + slot * 64;  // [K rows, Q rows]
            {
                const Ptrs<T*> dst{kt, qt, vt};
                pf[u].store(dst, nrm, 3, t_begin + 32 * min(ci, nchunks - 1), ci < nchunks ? t_end : -1);
            }
            pf[u].load(src, t_begin + 32 * min(ci + PD, nchunks - 1), L - 1);
            __syncthreads();
            if (ci < nchunks) {
                if (PARTS == 2 && ci > 0) {
                    const int ps = (ci - 1) & 1;
                    causal_reduce<T, D, FW, W, PARTS>(part_all + (size_t)ps * W * 32 * SM::PART_STRIDE,
                                                      plam_all + ps * W * 32, out, xbase, t0 - 32, t_end);
                }
                const vec8<T>* omc = omh;
                if (!OM_REGS) asm volatile("" : "+s"(omc));
                auto om_op = [&](int ft, int ks) -> vec8<T> {
                    if (OM_REGS) return omr[OM_REGS ? ft : 0][OM_REGS ? ks : 0];
                    return gload_vec(omc + ((size_t)(f0 / 16 + ft) * KSD + ks) * 64 + lane);
                };

                // ---- queries: projection, per-token shift over this wave's features
                vec8<T> bq[2][KSF];
                float sq[2];
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) {
                    vec8<T> x[KSD];
#pragma unroll
                    for (int ks = 0; ks < KSD; ++ks) x[ks] = row_operand<T, D>(qt, 16 * tt + r, ks, g);
                    const float c = RELU ? 0.0f : nrm[32 + 16 * tt + r];
                    f4 pq[NFT];
#pragma unroll
                    for (int ft = 0; ft < NFT; ++ft) {
                        pq[ft] = f4splat(c);
#pragma unroll
                        for (int ks = 0; ks < KSD; ++ks) pq[ft] = mma32(om_op(ft, ks), x[ks], pq[ft]);
                    }
                    float mx = kNegInf;
#pragma unroll
                    for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
                        for (int i = 0; i < 4; ++i) mx = __builtin_fmaxf(mx, pq[ft][i]);
                    mx = RELU ? 0.0f : col_max(mx);
                    sq[tt] = mx;
#pragma unroll
                    for (int kf = 0; kf < KSF; ++kf) {
                        f4 e0, e1;
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            e0[i] = feat<RELU>(pq[2 * kf][i] - mx);
                            e1[i] = feat<RELU>(pq[2 * kf + 1][i] - mx);
                        }
                        bq[tt][kf] = pack8t<T>(e0, e1);
                    }
                }
                // ---- keys: projection and features with the segment's fixed shift M
                vec8<T> ak[2][KSF];
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) {
                    vec8<T> x[KSD];
#pragma unroll
                    for (int ks = 0; ks < KSD; ++ks) x[ks] = row_operand<T, D>(kt, 16 * tt + r, ks, g);
                    const float c = (t0 + 16 * tt + r < t_end) ? (RELU ? 0.0f : nrm[16 * tt + r] - M) : kNegInf;
                    f4 pk[NFT];
#pragma unroll
                    for (int ft = 0; ft < NFT; ++ft) {
                        pk[ft] = f4splat(c);
#pragma unroll
                        for (int ks = 0; ks < KSD; ++ks) pk[ft] = mma32(om_op(ft, ks), x[ks], pk[ft]);
#pragma unroll
                        for (int i = 0; i < 4; ++i) pk[ft][i] = feat<RELU>(pk[ft][i]);
                        // phi(K) row-major by token for the state update
                        lds_store4(ptw + (16 * tt + r) * PTL::RS + 16 * ft + 4 * g, pk[ft]);
                    }
#pragma unroll
                    for (int kf = 0; kf < KSF; ++kf) ak[tt][kf] = pack8t<T>(pk[2 * kf], pk[2 * kf + 1]);
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

                // ---- partial outputs over this wave's features
                const int pslot = PARTS == 2 ? slot : 0;
                float* pw = part_all + ((size_t)pslot * W + w) * 32 * SM::PART_STRIDE;
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    vec8<T> ga[KSF];
#pragma unroll
                    for (int kf = 0; kf < KSF; ++kf) ga[kf] = pack8t<T>(G[2 * kf][nt], G[2 * kf + 1][nt]);
                    const vec8<T> va = nt < NT - 1 ? kappa_col<RS>(vt, 16 * nt, lane) : splat8<T>(1.0f);
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
                    // ---- state update for this column tile: G += phi(K)^T [V | 1]
#pragma unroll
                    for (int ft = 0; ft < NFT; ++ft) G[ft][nt] = mma32(kappa_col<PTL::RS>(ptw, 16 * ft, lane), va, G[ft][nt]);
                }
                if (g == 0) {
                    float* pl = plam_all + ((size_t)pslot * W + w) * 32;
                    pl[r] = sq[0] + M;
                    pl[16 + r] = sq[1] + M;
                }
                if (PARTS == 1) {
                    __syncthreads();
                    causal_reduce<T, D, FW, W, PARTS>(part_all, plam_all, out, xbase, t0, t_end);
                }
            }
        }
    }
    if (PARTS == 2) {
        __syncthreads();
        const int ps = (nchunks - 1) & 1;
        causal_reduce<T, D, FW, W, PARTS>(part_all + (size_t)ps * W * 32 * SM::PART_STRIDE, plam_all + ps * W * 32,
                                          out, xbase, t_begin + 32 * (nchunks - 1), t_end);
    }
}

// ---------------------------------------------------------------------------
// causal_decode: a causal call that carries a state and holds at most one
// 32-token chunk per head (decoding, short streaming pieces), in one launch
// instead of the segment-sum, merge/scan and scan launches and their
// workspace round trips.  One workgroup of W waves per (batch, head); wave w
// owns features [FW w, FW w + FW) as in causal_chunk, whose chunk arithmetic
// it repeats:
//   1. the chunk's keys are projected first; the key shift M is the larger
//      of the incoming state's shift and the largest key exponent (over the
//      waves, through LDS), so every feature and the rescaled state are <= 1;
//   2. the state is read from state_in (per head: G[m][D] row-major, z[m],
//      natural-log shift s; true values = stored e^s) straight into the
//      registers of the segment-sum layout, rescaled to M (zero without one);
//   3. the projection operands come from the fp32 projection (no packed copy
//      is needed by an earlier pass);
//   4. outputs as in causal_chunk; the new state goes to state_out from the
//      registers, with the shift M (ln 2 M in natural-log units).
// ---------------------------------------------------------------------------
template <typename T, int D, int FW, int W>
__global__ __launch_bounds__(64 * W) void causal_decode_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                               const T* __restrict__ v, const float* __restrict__ omega,
                                                               int om_per_head, const float* __restrict__ state_in,
                                                               float* __restrict__ state_out, T* __restrict__ out, int H,
                                                               int L, int m) {
    using TL = LdsTile<T, D>;
    using PTL = LdsTile<T, FW>;
    using SM = CausalSmem<T, D, FW, W, 1>;
    constexpr int RS = TL::RS;
    constexpr int KSD = D < 32 ? 1 : D / 32;
    constexpr int NT = D / 16 + 1;
    constexpr int NFT = FW / 16;
    constexpr int KSF = FW / 32;
    extern __shared__ __attribute__((aligned(16))) char smem_raw[];
    __shared__ float wave_max[W];
    T* kt = reinterpret_cast<T*>(smem_raw);
    T* qt = kt + TL::ELEMS;
    T* vt = qt + TL::ELEMS;
    float* part = reinterpret_cast<float*>(smem_raw + SM::OFF_PART);
    float* plam = reinterpret_cast<float*>(smem_raw + SM::OFF_LAM);
    float* nrm = reinterpret_cast<float*>(smem_raw + SM::OFF_NRM);  // [K rows, Q rows]

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, r = lane & 15, g = lane >> 4;
    const int bh = blockIdx.x, h = bh % H;
    const int f0 = w * FW;
    const size_t xbase = (size_t)bh * L * D;
    const size_t st_stride = (size_t)m * (D + 1) + 1;
    const float* omh = omega + (om_per_head ? (size_t)h * m * D : 0);
    T* ptw = reinterpret_cast<T*>(smem_raw + SM::OFF_PT) + (size_t)w * PTL::ELEMS;

    // the chunk (rows past L zeroed), the carried state (raw; scaled once the
    // shift is known) and this wave's projection operands, all requested
    // before the first barrier.  The state sits in the registers of the
    // segment-sum layout: G[ft][nt][i] holds G[f0 + 16 ft + 4 g + i][16 nt + r]
    // (nt < NT - 1) or z
    const Ptrs<const T*> src{k + xbase, q + xbase, v + xbase};
    Prefetch<T, D, 64 * W, 3> pf;
    pf.load(src, 0, L - 1);
    auto st_index = [&](int ft, int nt, int i) -> size_t {
        const int f = f0 + 16 * ft + 4 * g + i;
        return nt < NT - 1 ? (size_t)f * D + 16 * nt + r : (size_t)m * D + f;
    };
    const float* si = state_in ? state_in + (size_t)bh * st_stride : nullptr;
    f4 G[NFT][NT];
#pragma unroll
    for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) G[ft][nt][i] = si ? si[st_index(ft, nt, i)] : 0.0f;
    const float Ms = si ? si[(size_t)m * (D + 1)] * kLog2e : kNegInf;
    vec8<T> om[NFT][KSD];
#pragma unroll
    for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) om[ft][ks] = omega_operand<T, D>(omh, f0 + 16 * ft + r, ks, g);
    pf.store(Ptrs<T*>{kt, qt, vt}, nrm, 3, 0, L);
    __syncthreads();

    // ---- key projections (log2 units, relative to 0) and the key shift
    f4 pk[2][NFT];
    float lm = kNegInf;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
        vec8<T> x[KSD];
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) x[ks] = row_operand<T, D>(kt, 16 * tt + r, ks, g);
        const float c = 16 * tt + r < L ? nrm[16 * tt + r] : kNegInf;
#pragma unroll
        for (int ft = 0; ft < NFT; ++ft) {
            pk[tt][ft] = f4splat(c);
#pragma unroll
            for (int ks = 0; ks < KSD; ++ks) pk[tt][ft] = mma32(om[ft][ks], x[ks], pk[tt][ft]);  // D[F x T]
#pragma unroll
            for (int i = 0; i < 4; ++i) lm = __builtin_fmaxf(lm, pk[tt][ft][i]);
        }
    }
    lm = wave_max_uniform(lm);
    if (lane == 0) wave_max[w] = lm;
    __syncthreads();
    float M = Ms;
#pragma unroll
    for (int ww = 0; ww < W; ++ww) M = __builtin_fmaxf(M, wave_max[ww]);

    // ---- the carried state rescaled to M
    const float sc = si ? exp2f_fast(Ms - M) : 0.0f;
#pragma unroll
    for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) G[ft][nt] *= sc;

    // ---- key features relative to M: the A operand of the intra-chunk
    // scores and, row-major by token in LDS, of the state update
    vec8<T> ak[2][KSF];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
        for (int ft = 0; ft < NFT; ++ft) {
#pragma unroll
            for (int i = 0; i < 4; ++i) pk[tt][ft][i] = exp2f_fast(pk[tt][ft][i] - M);
            lds_store4(ptw + (16 * tt + r) * PTL::RS + 16 * ft + 4 * g, pk[tt][ft]);
        }
#pragma unroll
        for (int kf = 0; kf < KSF; ++kf) ak[tt][kf] = pack8t<T>(pk[tt][2 * kf], pk[tt][2 * kf + 1]);
    }

    // ---- queries: projection and a per-token shift over this wave's features
    vec8<T> bq[2][KSF];
    float sq[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
        vec8<T> x[KSD];
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) x[ks] = row_operand<T, D>(qt, 16 * tt + r, ks, g);
        const float c = nrm[32 + 16 * tt + r];
        f4 pq[NFT];
#pragma unroll
        for (int ft = 0; ft < NFT; ++ft) {
            pq[ft] = f4splat(c);
#pragma unroll
            for (int ks = 0; ks < KSD; ++ks) pq[ft] = mma32(om[ft][ks], x[ks], pq[ft]);
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

    // ---- partial outputs over this wave's features, and G += phi(K)^T [V | 1]
    float* pw = part + (size_t)w * 32 * SM::PART_STRIDE;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        vec8<T> ga[KSF];
#pragma unroll
        for (int kf = 0; kf < KSF; ++kf) ga[kf] = pack8t<T>(G[2 * kf][nt], G[2 * kf + 1][nt]);
        const vec8<T> va = nt < NT - 1 ? kappa_col<RS>(vt, 16 * nt, lane) : splat8<T>(1.0f);
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
#pragma unroll
        for (int ft = 0; ft < NFT; ++ft) G[ft][nt] = mma32(kappa_col<PTL::RS>(ptw, 16 * ft, lane), va, G[ft][nt]);
    }
    if (g == 0) {
        plam[w * 32 + r] = sq[0] + M;
        plam[w * 32 + 16 + r] = sq[1] + M;
    }
    __syncthreads();
    causal_reduce<T, D, FW, W, 1>(part, plam, out, xbase, 0, L);

    // ---- the new state, relative to M (z: every column of its tile holds it)
    if (state_out) {
        float* so = state_out + (size_t)bh * st_stride;
#pragma unroll
        for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                if (nt < NT - 1 || r == 0) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) so[st_index(ft, nt, i)] = G[ft][nt][i];
                }
        if (threadIdx.x == 0) so[(size_t)m * (D + 1)] = M * 0.69314718055994531f;
    }
}

// ---------------------------------------------------------------------------
// causal_tile: chunked causal scan for bf16, d = 64, m <= 256.  One workgroup
// of eight waves per (segment, head); chunks of 64 tokens.  Waves s and s + 4
// (which share a SIMD) own token tile s (tokens 16s..16s+15 of the chunk) and
// value-column tile s (columns 16s..16s+15):
//   query wave s      projects its 16 queries over all m features (the
//                     per-query shift is a wave-local maximum), publishes
//                     phi(Q) in LDS, then computes the intra-chunk scores
//                     S^T[key][query] (keys <= query) and S [V | 1] for its
//                     queries, and finishes their outputs;
//   key/state wave s  projects all 64 keys over the feature tiles
//                     ft = s (mod 4) (its projection operands stay in
//                     registers), publishes phi(K) in LDS, holds the state
//                     slice G[:, 16s..16s+15] (all m features) and
//                     z for the feature blocks kb = s (mod 4) in fp32
//                     registers, computes the inter-chunk terms phi(Q) G for
//                     all 64 queries (published in LDS) and updates G and z.
// All keys of a segment share one shift (the largest carry-in block shift)
// and each query one shift over all features, so the contraction over
// features is exact up to factors that cancel in the ratio (Simple
// Derivation).  Two barriers per chunk: phi published, then the next chunk's
// tiles and this chunk's inter-chunk terms published; outputs of a chunk are
// written at the start of the next step.
// ---------------------------------------------------------------------------
template <int M>
struct TileSmem {
    static constexpr int D = 64, KSD = 2, NFB = M / 32, NFT = M / 16;
    static constexpr int RS = kSwzTileRS;           // Q/K/V tile row stride (swz_tile)
    static constexpr int PKS = M + 16;               // phi(K) row stride (bf16, swz_rows)
    static constexpr int OS = D + 4;                 // inter-chunk output row stride (fp32)
    static constexpr size_t TILE = (size_t)64 * RS;  // elements of a 64-row tile
    static constexpr size_t OFF_OM = 0;
    static constexpr size_t OFF_TQ = OFF_OM + sizeof(bf16x8) * (size_t)NFT * KSD * 64;
    static constexpr size_t OFF_TK = OFF_TQ + sizeof(bf16) * TILE;
    static constexpr size_t OFF_TV = OFF_TK + sizeof(bf16) * TILE;
    static constexpr size_t OFF_NRM = OFF_TV + sizeof(bf16) * 2 * TILE;
    static constexpr size_t OFF_PQ = OFF_NRM + sizeof(float) * 128;
    static constexpr size_t OFF_PK = OFF_PQ + sizeof(bf16x8) * (size_t)4 * NFB * 64;
    static constexpr size_t OFF_OI = OFF_PK + sizeof(bf16) * (size_t)64 * PKS;
    static constexpr size_t OFF_DP = OFF_OI + sizeof(float) * (size_t)64 * OS;
    static constexpr size_t BYTES = OFF_DP + sizeof(float) * 4 * 64;
};

template <int M, bool RELU>
__global__ __launch_bounds__(512) void causal_tile_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                                                          const bf16* __restrict__ v, const bf16x8* __restrict__ ompack,
                                                          long long om_head_vecs, const bf16* __restrict__ carry,
                                                          const float* __restrict__ cmax, bf16* __restrict__ out, int H,
                                                          int L, int seg_len, int nseg) {
    using SM = TileSmem<M>;
    constexpr int D = SM::D, KSD = SM::KSD, NFB = SM::NFB, NFT = SM::NFT, RS = SM::RS, PKS = SM::PKS, OS = SM::OS;
    constexpr int D1 = D + 1;
    constexpr int ZB = (NFB + 3) / 4;  // z blocks per state wave (kb = s + 4 zb)
    extern __shared__ __attribute__((aligned(16))) char smem_raw[];
    bf16x8* om = reinterpret_cast<bf16x8*>(smem_raw + SM::OFF_OM);
    bf16* tq = reinterpret_cast<bf16*>(smem_raw + SM::OFF_TQ);
    bf16* tk = reinterpret_cast<bf16*>(smem_raw + SM::OFF_TK);
    bf16* tv0 = reinterpret_cast<bf16*>(smem_raw + SM::OFF_TV);
    float* nrm = reinterpret_cast<float*>(smem_raw + SM::OFF_NRM);  // [K rows 0..63 | Q rows 0..63]
    bf16x8* phq = reinterpret_cast<bf16x8*>(smem_raw + SM::OFF_PQ);
    bf16* phk = reinterpret_cast<bf16*>(smem_raw + SM::OFF_PK);
    float* oin = reinterpret_cast<float*>(smem_raw + SM::OFF_OI);
    float* dpart = reinterpret_cast<float*>(smem_raw + SM::OFF_DP);

    const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
    // wave index, wave-uniform for the compiler: branches on it are scalar
    // and skip their matrix instructions
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int s = w & 3;       // token tile and value-column tile of this wave
    // query waves 4..7, key/state waves 0..3: the key/state waves carry the
    // longer path in both phases and, as the older wave of each SIMD, win
    // its instruction arbitration
    const bool qwave = w >= 4;
    const int seg = blockIdx.x, bh = blockIdx.y, h = bh % H;
    const int t_begin = seg * seg_len;
    const int t_end = min(L, t_begin + seg_len);
    const int nch = (t_end - t_begin + 63) / 64;
    const size_t xbase = (size_t)bh * L * D;
    const Ptrs<const bf16*> src{k + xbase, q + xbase, v + xbase};

    // projection operands of this head straight into LDS (complete before
    // the first barrier)
    {
        const bf16x8* omh = ompack + (size_t)(om_head_vecs ? h : 0) * (size_t)om_head_vecs;
        copy_to_lds_async<512>(om, omh, NFT * KSD * 64);
    }

    // Q, K, V tiles are loaded and staged by the query waves alone (the
    // key/state waves carry the longer chain between the two barriers);
    // chunk 0 into registers
    Prefetch<bf16, D, 256, 3, 64> pf;
    if (qwave) pf.load(src, t_begin, L - 1);

    // carry-in (state waves): state slice for columns 16s.. and z for this
    // wave's blocks, rescaled from the per-block shifts to the segment's
    // common key shift
    const float* cm = cmax + ((size_t)bh * nseg + seg) * NFB;
    float Mseg = kNegInf;
#pragma unroll
    for (int b = 0; b < NFB; ++b) Mseg = __builtin_fmaxf(Mseg, cm[b]);
    f4 G[NFT];
    f4 Z[2 * ZB];
    if (!qwave && !carry) {  // no carry: the scan starts from a zero state
#pragma unroll
        for (int ft = 0; ft < NFT; ++ft) G[ft] = f4splat(0.0f);
#pragma unroll
        for (int zb = 0; zb < 2 * ZB; ++zb) Z[zb] = f4splat(0.0f);
    } else if (!qwave) {
        const bf16* cb = carry + ((size_t)bh * nseg + seg) * (size_t)M * D1;
#pragma unroll
        for (int ft = 0; ft < NFT; ++ft) {
            const float mb = cm[ft / 2];
            const float sc = (mb == kNegInf) ? 0.0f : exp2f_fast(mb - Mseg);
            G[ft] = sc * load4f(cb + seg_v_off<D>(ft, s, lane));
        }
#pragma unroll
        for (int zb = 0; zb < ZB; ++zb) {
            const int kb = s + 4 * zb;
            const bool own = kb < NFB;
            const float mb = own ? cm[kb] : kNegInf;
            const float sc = (mb == kNegInf) ? 0.0f : exp2f_fast(mb - Mseg);
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
                Z[2 * zb + hf] = own ? sc * load4f(cb + (size_t)M * D + 32 * kb + 16 * hf + 4 * g)
                                     : f4splat(0.0f);
        }
    }

    auto stage_chunk = [&](int ci) {
        // past the last chunk: rows of the last chunk, zeroed, into the V
        // buffer the last chunk does not use
        const int cc = min(ci, nch - 1);
        const Ptrs<bf16*> dst{tk, tq, tv0 + (size_t)(ci & 1) * SM::TILE};
        pf.template store<true>(dst, nrm, 3, t_begin + 64 * cc, ci < nch ? t_end : -1);
    };
    auto prefetch_chunk = [&](int ci) { pf.load(src, t_begin + 64 * min(ci, nch - 1), L - 1); };

    if (qwave) {
        stage_chunk(0);
        lds_dma_wait();
        prefetch_chunk(1);
    } else {
        lds_dma_wait();
    }
    __syncthreads();

    const bf16x8 ones = splat8<bf16>(1.0f);
    // lane offsets into the swizzled arrays (everything else is a constant)
    const int off_trv = kappa_lane_off(lane, swz_tile);       // V, transpose reads
    const int off_trk = kappa_lane_off(lane, swz_rows<PKS>);  // phi(K), transpose reads
    const int off_row = swz_tile(r, 8 * g);                   // Q/K rows 16 tt + r
    const int off_krow = swz_rows<PKS>(r, 4 * g);             // phi(K) rows 16 kt + r

    // The two roles run separate loops (so each keeps only its own registers
    // live) with the same barriers in the same order.
    if (qwave) {
        f4 oi[5];  // intra-chunk terms of the 16 queries: 4 column tiles, denominator
        // outputs of chunk cc for tokens 16s..16s+15
        auto finalize = [&](int cc) {
            const int row = 16 * s + r;
            const int t = t_begin + 64 * cc + row;
            float den = oi[4][0];
#pragma unroll
            for (int c = 0; c < (NFB < 4 ? NFB : 4); ++c) den += dpart[c * 64 + row];
            const float inv = __builtin_amdgcn_rcpf(den);
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                const f4 o = *reinterpret_cast<const f4*>(oin + row * OS + 16 * ct + 4 * g) + oi[ct];
                if (t < t_end) store4(out + xbase + (size_t)t * D + 16 * ct + 4 * g, o * inv);
            }
        };
        for (int c = 0; c < nch; ++c) {
            const bf16* tv = tv0 + (size_t)(c & 1) * SM::TILE;
            if (c > 0) finalize(c - 1);
            // ---- queries 16s..16s+15: projection, per-query shift, phi(Q)
            bf16x8 bq[NFB];
            {
                const float cq = RELU ? 0.0f : nrm[64 + 16 * s + r];
                bf16x8 xq[KSD];
#pragma unroll
                for (int ks = 0; ks < KSD; ++ks)
                    xq[ks] = *reinterpret_cast<const bf16x8*>(tq + off_row + 16 * s * RS + 32 * ks);
                // projection operands from LDS, read one group of feature
                // tiles ahead of their products.  The per-query shift is the
                // maximum over the first NF0 feature tiles; it is folded into
                // the initialisation of the remaining tiles (no subtraction
                // there), which are only checked against it: a query whose
                // later features exceed it by more than kTau raises its shift
                // (rare), so every value stays <= 2^kTau.
                constexpr int GF = 2, NG = NFT / GF, GO = GF * KSD;
                constexpr int NF0 = NFT < 4 ? NFT : 4;  // tiles that set the shift
                f4 pq[NFT];
                bf16x8 oa[2][GO];
                float mx = kNegInf;
#pragma unroll
                for (int i = 0; i < GO; ++i) oa[0][i] = om[i * 64 + lane];
#pragma unroll
                for (int gi = 0; gi < NG; ++gi) {
                    if (gi + 1 < NG) {
#pragma unroll
                        for (int i = 0; i < GO; ++i) oa[(gi + 1) & 1][i] = om[((gi + 1) * GO + i) * 64 + lane];
                    }
                    if (!RELU && gi * GF == NF0) {  // the first NF0 tiles are done: their maximum
#pragma unroll
                        for (int ft = 0; ft < NF0; ++ft)
#pragma unroll
                            for (int i = 0; i < 4; ++i) mx = __builtin_fmaxf(mx, pq[ft][i]);
                        mx = col_max(mx);
                    }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int f = 0; f < GF; ++f) {
                        const int ft = gi * GF + f;
                        pq[ft] = f4splat((RELU || ft < NF0) ? cq : cq - mx);
#pragma unroll
                        for (int ks = 0; ks < KSD; ++ks) pq[ft] = mma32(oa[gi & 1][f * KSD + ks], xq[ks], pq[ft]);
                    }
                }
                if constexpr (!RELU && NF0 == NFT) {
#pragma unroll
                    for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
                        for (int i = 0; i < 4; ++i) mx = __builtin_fmaxf(mx, pq[ft][i]);
                    mx = col_max(mx);
                }
                if constexpr (!RELU) {
#pragma unroll
                    for (int ft = 0; ft < NF0; ++ft) pq[ft] -= mx;
                }
                if constexpr (!RELU && NF0 < NFT) {
                    float lm = kNegInf;
#pragma unroll
                    for (int ft = NF0; ft < NFT; ++ft)
#pragma unroll
                        for (int i = 0; i < 4; ++i) lm = __builtin_fmaxf(lm, pq[ft][i]);
                    if (wave_any(lm > kTau)) {
                        // raise the shift of the queries that need it
                        const float cm = col_max(lm);
                        const float up = cm > kTau ? cm : 0.0f;
#pragma unroll
                        for (int ft = 0; ft < NFT; ++ft) pq[ft] -= up;
                    }
                }
#pragma unroll
                for (int kb = 0; kb < NFB; ++kb) {
                    f4 e0, e1;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        e0[i] = feat<RELU>(pq[2 * kb][i]);
                        e1[i] = feat<RELU>(pq[2 * kb + 1][i]);
                    }
                    bq[kb] = pack8t<bf16>(e0, e1);
                    phq[(s * NFB + kb) * 64 + lane] = bq[kb];
                }
            }
            __syncthreads();

            // next chunk's tiles (Q, K and this V buffer's partner are free now)
            stage_chunk(c + 1);
            prefetch_chunk(c + 2);

            // ---- intra-chunk terms for queries 16s..16s+15: key tiles 0..s
            // (later ones are all masked), keys after the query zeroed.  One
            // code path per s, so the products of the s + 1 key tiles form
            // independent accumulation chains issued feature block by block.
            auto intra = [&](auto nkt_c) {
                constexpr int NKT = decltype(nkt_c)::value;
                constexpr int NA = NKT <= 2 ? 2 : 1;  // partial sums per key tile
                f4 sa[NKT][NA];
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
                    for (int a = 0; a < NA; ++a) sa[kt][a] = f4splat(0.0f);
                auto read_a = [&](int kb, bf16x8* a) {
#pragma unroll
                    for (int kt = 0; kt < NKT; ++kt) {
                        const bf16* pr = phk + off_krow + 16 * kt * PKS + 32 * kb;
                        const bf16x4 lo = *reinterpret_cast<const bf16x4*>(pr);
                        const bf16x4 hi = *reinterpret_cast<const bf16x4*>(pr + 16);
                        a[kt] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    }
                };
                bf16x8 a[2][NKT];
                read_a(0, a[0]);
#pragma unroll
                for (int kb = 0; kb < NFB; ++kb) {
                    if (kb + 1 < NFB) read_a(kb + 1, a[(kb + 1) & 1]);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int kt = 0; kt < NKT; ++kt) sa[kt][kb % NA] = mma32(a[kb & 1][kt], bq[kb], sa[kt][kb % NA]);
                }
                f4 st[4];
#pragma unroll
                for (int kt = 0; kt < 4; ++kt) st[kt] = f4splat(0.0f);
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt) st[kt] = NA == 2 ? sa[kt][0] + sa[kt][NA - 1] : sa[kt][0];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (4 * g + i > r) st[NKT - 1][i] = 0.0f;
#pragma unroll
                for (int ct = 0; ct < 5; ++ct) oi[ct] = f4splat(0.0f);
#pragma unroll
                for (int j = 0; j < (NKT + 1) / 2; ++j) {
                    const bf16x8 b = pack8t<bf16>(st[2 * j], st[2 * j + 1]);
#pragma unroll
                    for (int ct = 0; ct < 4; ++ct)
                        oi[ct] = mma32(kappa_col_at<RS>(tv + off_trv + 32 * j * RS + 16 * ct), b, oi[ct]);
                    oi[4] = mma32(ones, b, oi[4]);
                }
            };
            switch (s) {
                case 0: intra(IntC<1>{}); break;
                case 1: intra(IntC<2>{}); break;
                case 2: intra(IntC<3>{}); break;
                default: intra(IntC<4>{}); break;
            }
            __syncthreads();
        }
        finalize(nch - 1);
    } else {
        // key/state wave: feature tiles ft = s + 4 f of the key projection,
        // the state slice for value columns 16s.. and z for feature blocks
        // kb = s + 4 zb
        constexpr int KFT = (NFT + 3) / 4;
        for (int c = 0; c < nch; ++c) {
            const int t0 = t_begin + 64 * c;
            const bf16* tv = tv0 + (size_t)(c & 1) * SM::TILE;
            // ---- keys of the chunk, this wave's feature tiles, the segment's shift
            {
                vec8<bf16> omr[KFT][KSD];  // projection operands (from LDS, once per chunk)
#pragma unroll
                for (int f = 0; f < KFT; ++f)
#pragma unroll
                    for (int ks = 0; ks < KSD; ++ks) omr[f][ks] = om[((s + 4 * f) * KSD + ks) * 64 + lane];
                f4 pk[4][KFT];
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    const int row = 16 * tt + r;
                    const float ck = (t0 + row < t_end) ? (RELU ? 0.0f : nrm[row] - Mseg) : kNegInf;
                    bf16x8 xk[KSD];
#pragma unroll
                    for (int ks = 0; ks < KSD; ++ks)
                        xk[ks] = *reinterpret_cast<const bf16x8*>(tk + off_row + 16 * tt * RS + 32 * ks);
#pragma unroll
                    for (int f = 0; f < KFT; ++f) {
                        pk[tt][f] = f4splat(ck);
#pragma unroll
                        for (int ks = 0; ks < KSD; ++ks) pk[tt][f] = mma32(omr[f][ks], xk[ks], pk[tt][f]);
                    }
                }
#pragma unroll
                for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                    for (int f = 0; f < KFT; ++f) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) pk[tt][f][i] = feat<RELU>(pk[tt][f][i]);
                        lds_store4(phk + off_krow + 16 * tt * PKS + 16 * (s + 4 * f), pk[tt][f]);
                    }
            }
            __syncthreads();

            // ---- inter-chunk terms phi(Q) G for all 64 queries and the state
            // update G += phi(K)^T V, z += phi(K)^T 1, interleaved feature
            // block by feature block: block kb's inter-chunk products use G
            // of the previous chunks (packed before its update), then its two
            // feature tiles are updated.  The four query tiles are
            // independent accumulation chains; the denominator terms and z of
            // this wave's blocks (kb = s mod 4) reuse the same operands.
            {
                f4 o[4], dz[4];
#pragma unroll
                for (int qt = 0; qt < 4; ++qt) {
                    o[qt] = f4splat(0.0f);
                    dz[qt] = f4splat(0.0f);
                }
                bf16x8 bv[2];  // V operand of this wave's columns, both token halves
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) bv[jj] = kappa_col_at<RS>(tv + off_trv + 32 * jj * RS + 16 * s);
                // operands of block kb: phi(Q) for the four query tiles, phi(K)^T
                // for its two feature tiles and both token halves (read one
                // block ahead of their products)
                bf16x8 b[2][4], ka[2][4];
                auto read_block = [&](int kb, bf16x8* bb, bf16x8* kk) {
#pragma unroll
                    for (int qt = 0; qt < 4; ++qt) bb[qt] = phq[(qt * NFB + kb) * 64 + lane];
#pragma unroll
                    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                        for (int jj = 0; jj < 2; ++jj)
                            kk[2 * hf + jj] = kappa_col_at<PKS>(phk + off_trk + 32 * jj * PKS + 16 * (2 * kb + hf));
                };
                read_block(0, b[0], ka[0]);
#pragma unroll
                for (int kb = 0; kb < NFB; ++kb) {
                    if (kb + 1 < NFB) read_block(kb + 1, b[(kb + 1) & 1], ka[(kb + 1) & 1]);
                    __builtin_amdgcn_sched_barrier(0);
                    const bf16x8* bb = b[kb & 1];
                    const bf16x8* kk = ka[kb & 1];
                    const bf16x8 ga = pack8t<bf16>(G[2 * kb], G[2 * kb + 1]);
#pragma unroll
                    for (int qt = 0; qt < 4; ++qt) o[qt] = mma32(ga, bb[qt], o[qt]);
#pragma unroll
                    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                        for (int jj = 0; jj < 2; ++jj) G[2 * kb + hf] = mma32(kk[2 * hf + jj], bv[jj], G[2 * kb + hf]);
                    if (kb % 4 == s) {
                        const int zt = 2 * (kb / 4);
                        const bf16x8 za = pack8t<bf16>(Z[zt], Z[zt + 1]);
#pragma unroll
                        for (int qt = 0; qt < 4; ++qt) dz[qt] = mma32(za, bb[qt], dz[qt]);
#pragma unroll
                        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                            for (int jj = 0; jj < 2; ++jj) Z[zt + hf] = mma32(kk[2 * hf + jj], ones, Z[zt + hf]);
                    }
                }
#pragma unroll
                for (int qt = 0; qt < 4; ++qt) {
                    *reinterpret_cast<f4*>(oin + (16 * qt + r) * OS + 16 * s + 4 * g) = o[qt];
                    if (g == 0 && s < NFB) dpart[s * 64 + 16 * qt + r] = dz[qt][0];
                }
            }
            __syncthreads();
        }
    }
}

// ---------------------------------------------------------------------------
// causal_wide: chunked causal scan for bf16, d = 128, m in {256, 512}.  One
// workgroup of eight waves per (segment, head, half of the value columns);
// chunks of 32 tokens.  The fp32 state of a head (m x 129) is too large for
// one wave's registers, and the projection operands (m x 128 bf16) too large
// for LDS next to the feature buffers, so both are split over the waves:
//   wave w projects the chunk's queries and keys over its own m/8 features
//     (operands resident in registers); the per-query shift is the maximum
//     over all m features, reduced across the waves through LDS (queries
//     need no |q|^2 term: it is a per-query factor); keys use the segment's
//     fixed shift;
//   wave w = 4 fh + ct holds the state slice G[features of half fh][value
//     columns 16 nt ..] (nt = 4 half + ct) and z for its projection features;
//   the intra-chunk scores S^T[key][query] are summed over the waves'
//     feature slices through LDS;
//   wave (fh, ct) finishes query tile fh of its columns: its inter-chunk
//     terms over half fh plus its partner's over the other half, S [V | 1],
//     the denominator (z terms of all waves plus the row sums of S).
// Both column halves recompute the projections (the price of keeping the
// state in registers).  Three barriers per chunk: maxima and phi(K) rows
// ready; phi(Q), score and denominator partials published; next tiles
// staged, scores summed and inter-chunk partials exchanged.  Per-query
// values of all waves (maxima, denominator terms) sit side by side, so one
// lane reads them with two 16-byte loads.
// ---------------------------------------------------------------------------
template <int M>
struct WideSmem {
    static constexpr int D = 128, NFB = M / 32;
    static constexpr int RS = LdsTile<bf16, D>::RS;  // Q/K/V tile row stride
    static constexpr int PKS = M + 16;               // phi(K) row stride (bf16)
    static constexpr size_t TILE = (size_t)32 * RS;  // elements of a 32-row tile
    static constexpr size_t OFF_TK = 0;
    static constexpr size_t OFF_TQ = OFF_TK + sizeof(bf16) * TILE;
    static constexpr size_t OFF_TV = OFF_TQ + sizeof(bf16) * TILE;  // two buffers
    static constexpr size_t OFF_NRM = OFF_TV + sizeof(bf16) * 2 * TILE;
    static constexpr size_t OFF_QMAX = OFF_NRM + sizeof(float) * 3 * 32;
    static constexpr size_t OFF_PQ = OFF_QMAX + sizeof(float) * 8 * 32;
    static constexpr size_t OFF_PK = OFF_PQ + sizeof(bf16x8) * (size_t)2 * NFB * 64;
    static constexpr size_t OFF_SP = OFF_PK + sizeof(bf16) * (size_t)32 * PKS;
    static constexpr size_t OFF_ST = OFF_SP + sizeof(f4) * (size_t)8 * 3 * 64;
    static constexpr size_t OFF_DP = OFF_ST + sizeof(f4) * (size_t)3 * 64;
    static constexpr size_t OFF_XO = OFF_DP + sizeof(float) * 8 * 32;
    static constexpr size_t BYTES = OFF_XO + sizeof(f4) * (size_t)4 * 2 * 64;
};

template <int M, bool RELU>
__global__ __launch_bounds__(512) void causal_wide_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                                                          const bf16* __restrict__ v, const bf16x8* __restrict__ ompack,
                                                          long long om_head_vecs, const bf16* __restrict__ carry,
                                                          const float* __restrict__ cmax, bf16* __restrict__ out, int H,
                                                          int L, int seg_len, int nseg) {
    using SM = WideSmem<M>;
    constexpr int D = SM::D, KSD = D / 32, NFB = SM::NFB, RS = SM::RS, PKS = SM::PKS;
    constexpr int D1 = D + 1;
    constexpr int PFT = M / 128;  // projection feature tiles per wave (features 16 PFT w ..)
    constexpr int PFB = PFT / 2;  // projection feature blocks per wave
    constexpr int GFT = M / 32;   // state feature tiles per wave (one half of the features)
    constexpr int GFB = GFT / 2;
    static_assert(PFB >= 1, "m >= 256");
    extern __shared__ __attribute__((aligned(16))) char smem_raw[];
    bf16* tk = reinterpret_cast<bf16*>(smem_raw + SM::OFF_TK);
    bf16* tq = reinterpret_cast<bf16*>(smem_raw + SM::OFF_TQ);
    bf16* tv0 = reinterpret_cast<bf16*>(smem_raw + SM::OFF_TV);
    float* nrm = reinterpret_cast<float*>(smem_raw + SM::OFF_NRM);  // K rows 0..31
    float* qmax = reinterpret_cast<float*>(smem_raw + SM::OFF_QMAX);
    bf16x8* phq = reinterpret_cast<bf16x8*>(smem_raw + SM::OFF_PQ);
    bf16* phk = reinterpret_cast<bf16*>(smem_raw + SM::OFF_PK);
    f4* spart = reinterpret_cast<f4*>(smem_raw + SM::OFF_SP);
    f4* stot = reinterpret_cast<f4*>(smem_raw + SM::OFF_ST);
    float* dpart = reinterpret_cast<float*>(smem_raw + SM::OFF_DP);
    f4* xo = reinterpret_cast<f4*>(smem_raw + SM::OFF_XO);

    const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ct = w & 3, fh = w >> 2;
    const int seg = blockIdx.x, bh = blockIdx.y, h = bh % H;
    const int nt = 4 * (int)blockIdx.z + ct;  // value-column tile of this wave
    const int t_begin = seg * seg_len;
    const int t_end = min(L, t_begin + seg_len);
    const int nch = (t_end - t_begin + 31) / 32;
    if (nch <= 0) return;  // workgroup-uniform
    const size_t xbase = (size_t)bh * L * D;
    const Ptrs<const bf16*> src{k + xbase, q + xbase, v + xbase};

    // chunk 0 into registers first (latency overlaps the loads below)
    Prefetch<bf16, D, 512, 3, 32> pf;
    pf.load(src, t_begin, L - 1);

    bf16x8 om[PFT][KSD];
    {
        const bf16x8* omh = ompack + (size_t)(om_head_vecs ? h : 0) * (size_t)om_head_vecs;
#pragma unroll
        for (int f = 0; f < PFT; ++f)
#pragma unroll
            for (int ks = 0; ks < KSD; ++ks) om[f][ks] = omh[((PFT * w + f) * KSD + ks) * 64 + lane];
    }

    // carry-in rescaled from the per-block shifts to the segment's key shift
    const float* cm = cmax + ((size_t)bh * nseg + seg) * NFB;
    float Mseg = kNegInf;
#pragma unroll
    for (int b = 0; b < NFB; ++b) Mseg = __builtin_fmaxf(Mseg, cm[b]);
    f4 G[GFT];
    f4 Z[PFT];
    if (!carry) {  // no carry: the scan starts from a zero state
#pragma unroll
        for (int i = 0; i < GFT; ++i) G[i] = f4splat(0.0f);
#pragma unroll
        for (int f = 0; f < PFT; ++f) Z[f] = f4splat(0.0f);
    } else {
        const bf16* cb = carry + ((size_t)bh * nseg + seg) * (size_t)M * D1;
#pragma unroll
        for (int i = 0; i < GFT; ++i) {
            const int ft = GFT * fh + i;
            const float mb = cm[ft / 2];
            const float sc = (mb == kNegInf) ? 0.0f : exp2f_fast(mb - Mseg);
            G[i] = sc * load4f(cb + seg_v_off<D>(ft, nt, lane));
        }
#pragma unroll
        for (int f = 0; f < PFT; ++f) {
            const int ft = PFT * w + f;
            const float mb = cm[ft / 2];
            const float sc = (mb == kNegInf) ? 0.0f : exp2f_fast(mb - Mseg);
            Z[f] = sc * load4f(cb + (size_t)M * D + 16 * ft + 4 * g);
        }
    }

    auto stage_chunk = [&](int ci) {
        const int cc = min(ci, nch - 1);
        const Ptrs<bf16*> dst{tk, tq, tv0 + (size_t)(ci & 1) * SM::TILE};
        pf.store(dst, nrm, 1, t_begin + 32 * cc, ci < nch ? t_end : -1);
        pf.load(src, t_begin + 32 * min(ci + 1, nch - 1), L - 1);
    };
    stage_chunk(0);
    __syncthreads();

    const bf16x8 ones = splat8<bf16>(1.0f);
    for (int c = 0; c < nch; ++c) {
        const int t0 = t_begin + 32 * c;
        const bf16* tv = tv0 + (size_t)(c & 1) * SM::TILE;

        // ---- projections over this wave's features (keys first: their
        // exponentials and row stores overlap the query products)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            bf16x8 x[KSD];
#pragma unroll
            for (int ks = 0; ks < KSD; ++ks)
                x[ks] = *reinterpret_cast<const bf16x8*>(tk + (16 * tt + r) * RS + 32 * ks + 8 * g);
            const float ck = (t0 + 16 * tt + r < t_end) ? (RELU ? 0.0f : nrm[16 * tt + r] - Mseg) : kNegInf;
            f4 pk[PFT];
#pragma unroll
            for (int f = 0; f < PFT; ++f) {
                pk[f] = f4splat(ck);
#pragma unroll
                for (int ks = 0; ks < KSD; ++ks) pk[f] = mma32(om[f][ks], x[ks], pk[f]);
#pragma unroll
                for (int i = 0; i < 4; ++i) pk[f][i] = feat<RELU>(pk[f][i]);
                // phi(K) row-major by token (features of tile PFT w + f)
                lds_store4(phk + (16 * tt + r) * PKS + 16 * (PFT * w + f) + 4 * g, pk[f]);
            }
        }
        f4 pq[2][PFT];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            bf16x8 x[KSD];
#pragma unroll
            for (int ks = 0; ks < KSD; ++ks)
                x[ks] = *reinterpret_cast<const bf16x8*>(tq + (16 * tt + r) * RS + 32 * ks + 8 * g);
#pragma unroll
            for (int f = 0; f < PFT; ++f) {
                pq[tt][f] = f4splat(0.0f);
#pragma unroll
                for (int ks = 0; ks < KSD; ++ks) pq[tt][f] = mma32(om[f][ks], x[ks], pq[tt][f]);
            }
        }
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            float mx = kNegInf;
#pragma unroll
            for (int f = 0; f < PFT; ++f)
#pragma unroll
                for (int i = 0; i < 4; ++i) mx = __builtin_fmaxf(mx, pq[tt][f][i]);
            mx = col_max(mx);
            if (g == 0) qmax[(16 * tt + r) * 8 + w] = mx;
        }
        __syncthreads();

        // ---- phi(Q) with the per-query shift, phi(K) rows, score and
        // denominator partials over this wave's features
        bf16x8 bq[2][PFB];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const f4 m0 = *reinterpret_cast<const f4*>(qmax + (16 * tt + r) * 8);
            const f4 m1 = *reinterpret_cast<const f4*>(qmax + (16 * tt + r) * 8 + 4);
            const float mq = RELU ? 0.0f
                                  : __builtin_fmaxf(__builtin_fmaxf(__builtin_fmaxf(m0[0], m0[1]), __builtin_fmaxf(m0[2], m0[3])),
                                                    __builtin_fmaxf(__builtin_fmaxf(m1[0], m1[1]), __builtin_fmaxf(m1[2], m1[3])));
#pragma unroll
            for (int b = 0; b < PFB; ++b) {
                f4 e0, e1;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    e0[i] = feat<RELU>(pq[tt][2 * b][i] - mq);
                    e1[i] = feat<RELU>(pq[tt][2 * b + 1][i] - mq);
                }
                bq[tt][b] = pack8t<bf16>(e0, e1);
                phq[(tt * NFB + PFB * w + b) * 64 + lane] = bq[tt][b];
            }
        }
        {
            f4 sp[3];
#pragma unroll
            for (int i = 0; i < 3; ++i) sp[i] = f4splat(0.0f);
#pragma unroll
            for (int b = 0; b < PFB; ++b) {
                // phi(K) of this wave's block b for keys 16 kt + r (its own
                // rows of the phi(K) array, written before the barrier)
                bf16x8 ak[2];
#pragma unroll
                for (int kt = 0; kt < 2; ++kt) {
                    const bf16* pr = phk + (16 * kt + r) * PKS + 32 * (PFB * w + b) + 4 * g;
                    const bf16x4 lo = *reinterpret_cast<const bf16x4*>(pr);
                    const bf16x4 hi = *reinterpret_cast<const bf16x4*>(pr + 16);
                    ak[kt] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                }
                sp[0] = mma32(ak[0], bq[0][b], sp[0]);  // keys 0..15, queries 0..15
                sp[1] = mma32(ak[0], bq[1][b], sp[1]);  // keys 0..15, queries 16..31
                sp[2] = mma32(ak[1], bq[1][b], sp[2]);  // keys 16..31, queries 16..31
            }
#pragma unroll
            for (int i = 0; i < 3; ++i) spart[(w * 3 + i) * 64 + lane] = sp[i];
            f4 dz[2] = {f4splat(0.0f), f4splat(0.0f)};
#pragma unroll
            for (int b = 0; b < PFB; ++b) {
                const bf16x8 za = pack8t<bf16>(Z[2 * b], Z[2 * b + 1]);
                dz[0] = mma32(za, bq[0][b], dz[0]);
                dz[1] = mma32(za, bq[1][b], dz[1]);
            }
            if (g == 0) {
                dpart[r * 8 + w] = dz[0][0];
                dpart[(16 + r) * 8 + w] = dz[1][0];
            }
        }
        __syncthreads();

        // ---- next chunk's tiles; scores summed over the waves
        stage_chunk(c + 1);
        {
            const float* sps = reinterpret_cast<const float*>(spart);
            float* sts = reinterpret_cast<float*>(stot);
            for (int e = threadIdx.x; e < 3 * 64 * 4; e += 512) {
                float acc = sps[e];
#pragma unroll
                for (int ww = 1; ww < 8; ++ww) acc += sps[ww * 3 * 64 * 4 + e];
                sts[e] = acc;
            }
        }
        // inter-chunk terms of both query tiles over half fh (state before
        // this chunk), then the state update G += phi(K)^T V, z += phi(K)^T 1
        const bf16x8 bv = kappa_col<RS>(tv, 16 * nt, lane);
        f4 o[2] = {f4splat(0.0f), f4splat(0.0f)};
        {
            bf16x8 b[2][2];
            b[0][0] = phq[(0 * NFB + GFB * fh) * 64 + lane];
            b[0][1] = phq[(1 * NFB + GFB * fh) * 64 + lane];
#pragma unroll
            for (int i = 0; i < GFB; ++i) {
                const int kb = GFB * fh + i;
                if (i + 1 < GFB) {
                    b[(i + 1) & 1][0] = phq[(0 * NFB + kb + 1) * 64 + lane];
                    b[(i + 1) & 1][1] = phq[(1 * NFB + kb + 1) * 64 + lane];
                }
                const bf16x8 ga = pack8t<bf16>(G[2 * i], G[2 * i + 1]);
                o[0] = mma32(ga, b[i & 1][0], o[0]);
                o[1] = mma32(ga, b[i & 1][1], o[1]);
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
                    G[2 * i + hf] = mma32(kappa_col<PKS>(phk, 16 * (2 * kb + hf), lane), bv, G[2 * i + hf]);
            }
        }
#pragma unroll
        for (int f = 0; f < PFT; ++f) Z[f] = mma32(kappa_col<PKS>(phk, 16 * (PFT * w + f), lane), ones, Z[f]);
        // the partner wave (other half, same columns) finishes the other query tile
        xo[(ct * 2 + (1 - fh)) * 64 + lane] = fh ? o[0] : o[1];
        __syncthreads();

        // ---- outputs of query tile fh, columns 16 nt ..
        {
            f4 oo = (fh ? o[1] : o[0]) + xo[(ct * 2 + fh) * 64 + lane];
            f4 s0, s1;
            if (fh == 0) {
                s0 = stot[0 * 64 + lane];
                s1 = f4splat(0.0f);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (4 * g + i > r) s0[i] = 0.0f;
            } else {
                s0 = stot[1 * 64 + lane];
                s1 = stot[2 * 64 + lane];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (4 * g + i > r) s1[i] = 0.0f;
            }
            const bf16x8 bs = pack8t<bf16>(s0, s1);
            oo = mma32(bv, bs, oo);
            const f4 di = mma32(ones, bs, f4splat(0.0f));
            const int row = 16 * fh + r;
            const f4 d0 = *reinterpret_cast<const f4*>(dpart + row * 8);
            const f4 d1 = *reinterpret_cast<const f4*>(dpart + row * 8 + 4);
            const float den = di[0] + ((d0[0] + d0[1]) + (d0[2] + d0[3])) + ((d1[0] + d1[1]) + (d1[2] + d1[3]));
            const float inv = __builtin_amdgcn_rcpf(den);
            const int t = t0 + row;
            if (t < t_end) store4(out + xbase + (size_t)t * D + 16 * nt + 4 * g, oo * inv);
        }
    }
}

// ---------------------------------------------------------------------------
// features: phi(x) (fp32) for 16 tokens per wave, all m features; optional
// per-row stabiliser (two passes: the maximum, then the features).
// ---------------------------------------------------------------------------
template <typename T, int D, bool RELU>
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
        const bool pad = D < 32 && g >= D / 8;  // padding lanes of d = 16
        if (kSplitD16<T, D>)  // repeat the row there (see kSplitD16)
            xv[ks] = ok ? load8(x + (size_t)row * D + 8 * (g & 1)) : zero8<T>();
        else
            xv[ks] = ok && !pad ? load8(x + (size_t)row * D + 32 * ks + 8 * g) : zero8<T>();
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float t = to_f(xv[ks][j]);
            ss += pad ? 0.0f : t * t;
        }
    }
    const float c = -0.5f * kLog2e * col_sum(ss);
    const int nft = m / 16;
    float s = 0.0f;
    if (RELU) {
        // no stabiliser for ReLU features: log_scale is 0
        if (stabilize && ok && g == 0 && log_scale) log_scale[row] = 0.0f;
    } else if (stabilize) {
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
    const float off = RELU ? 0.0f : c - s - 0.5f * __builtin_log2f((float)m);
    // ReLU: the packed projection carries log2(e); undo it with m^-1/2
    const float rscale = 1.0f / (kLog2e * __builtin_sqrtf((float)m));
    for (int ft = 0; ft < nft; ++ft) {
        f4 p = f4splat(off);
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) p = mma32(omh[((size_t)ft * KSD + ks) * 64 + lane], xv[ks], p);
        f4 e;
#pragma unroll
        for (int i = 0; i < 4; ++i) e[i] = RELU ? rscale * feat<true>(p[i]) : exp2f_fast(p[i]);
        if (ok) store4(phi + (size_t)row * m + 16 * ft + 4 * g, e);
    }
}

// ---------------------------------------------------------------------------
// Host-side launchers (internal interface, see favor_kernels.h).
// ---------------------------------------------------------------------------
static inline void stage_event(const LaunchArgs& a, int i) {
    if (a.events) (void)hipEventRecord(static_cast<hipEvent_t>(a.events[i]), a.stream);
}

// A carry-free causal call: one segment per head and no carried state.  Its
// merge pass is skipped: the scan starts from a zero state and takes the
// segment-sum pass's key shifts (for one segment the layout of the merged
// shifts, [head][segment][block]), and the segment-sum pass packs the
// projection operands the merge pass would have packed.
static bool causal_carry_free(const LaunchArgs& a) {
    return a.op == OpKind::Causal && a.nseg == 1 && !a.state_in && !a.state_out;
}
template <typename T>
static const T* scan_carry(const LaunchArgs& a) {
    return causal_carry_free(a) ? nullptr : static_cast<const T*>(a.ws_carry);
}
static const float* scan_shifts(const LaunchArgs& a) { return causal_carry_free(a) ? a.ws_pmax : a.ws_cmax; }

template <typename T, int D, int FW, int W, bool RELU>
static hipError_t launch_causal(const LaunchArgs& a, const vec8<T>* ompack, long long om_head_vecs, const T* q,
                                const T* k, const T* v, T* out) {
    constexpr bool OM_REGS = FW * D <= 64 * 64;
    // chunks in flight: as many as fit in a register budget per thread (a
    // 32-token chunk of q, k, v is spread over the workgroup's threads); 48
    // registers, 16 for fp32 with eight waves (two waves per SIMD share its
    // registers, and fp32 operands take twice the registers of bf16 ones)
    constexpr int PER = (32 * (D / 8) * 3 + 64 * W - 1) / (64 * W);
    constexpr int REGS = PER * (int)sizeof(vec8<T>) / 4;
    constexpr int BUDGET = (sizeof(T) == 4 && W >= 8) ? 16 : 48;
    constexpr int PD = REGS >= BUDGET ? 1 : (BUDGET / REGS > 4 ? 4 : BUDGET / REGS);
    constexpr size_t two = CausalSmem<T, D, FW, W, 2>::BYTES;
    const dim3 grid(a.nseg, a.B * a.H), block(64 * W);
    if constexpr (two <= kMaxLds) {
        auto kern = causal_chunk_kernel<T, D, FW, W, 2, PD, OM_REGS, RELU>;
        (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)two);
        hipLaunchKernelGGL(kern, grid, block, two, a.stream, q, k, v, ompack, om_head_vecs,
                           scan_carry<T>(a), scan_shifts(a), out, a.H, a.L, a.m, a.seg_len, a.nseg);
    } else if constexpr (CausalSmem<T, D, FW, W, 1>::BYTES > kMaxLds) {
        return hipErrorInvalidValue;  // rejected by argument validation before any launch
    } else {
        constexpr size_t one = CausalSmem<T, D, FW, W, 1>::BYTES;
        auto kern = causal_chunk_kernel<T, D, FW, W, 1, PD, OM_REGS, RELU>;
        (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)one);
        hipLaunchKernelGGL(kern, grid, block, one, a.stream, q, k, v, ompack, om_head_vecs,
                           scan_carry<T>(a), scan_shifts(a), out, a.H, a.L, a.m, a.seg_len, a.nseg);
    }
    return hipGetLastError();
}

template <typename T, int D, int FW, int W>
static hipError_t launch_causal_decode(const LaunchArgs& a, const T* q, const T* k, const T* v, T* out) {
    constexpr size_t bytes = CausalSmem<T, D, FW, W, 1>::BYTES;
    if constexpr (bytes + sizeof(float) * W > kMaxLds) {
        return hipErrorInvalidValue;  // not a decode shape (causal_decode_shape)
    } else {
        auto kern = causal_decode_kernel<T, D, FW, W>;
        (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
        hipLaunchKernelGGL(kern, dim3(a.B * a.H), dim3(64 * W), bytes, a.stream, q, k, v, a.omega,
                           a.omega_per_head ? 1 : 0, a.state_in, a.state_out, out, a.H, a.L, a.m);
        return hipGetLastError();
    }
}

// The configuration of causal_decode for this shape: the feature-split
// scan's (features per wave, waves), among the pairs instantiated for it.
template <typename T, int D>
static hipError_t dispatch_causal_decode(const LaunchArgs& a, const T* q, const T* k, const T* v, T* out) {
    const CausalCfg cfg = causal_config((int)sizeof(T), D, a.m);
    constexpr bool narrow = (sizeof(T) == 2 && D == 128) || (sizeof(T) == 4 && D == 64);
    if (cfg.fw == 32 && cfg.w == 1) return launch_causal_decode<T, D, 32, 1>(a, q, k, v, out);
    if constexpr (narrow) {
        if (cfg.fw == 32 && cfg.w == 2) return launch_causal_decode<T, D, 32, 2>(a, q, k, v, out);
        if (cfg.fw == 32 && cfg.w == 4) return launch_causal_decode<T, D, 32, 4>(a, q, k, v, out);
        if constexpr (sizeof(T) == 4) {
            if (cfg.fw == 32 && cfg.w == 8) return launch_causal_decode<T, D, 32, 8>(a, q, k, v, out);
        }
    } else {
        if (cfg.fw == 64 && cfg.w == 1) return launch_causal_decode<T, D, 64, 1>(a, q, k, v, out);
        if (cfg.fw == 64 && cfg.w == 2) return launch_causal_decode<T, D, 64, 2>(a, q, k, v, out);
        if (cfg.fw == 64 && cfg.w == 4) return launch_causal_decode<T, D, 64, 4>(a, q, k, v, out);
        if (cfg.fw == 64 && cfg.w == 8) return launch_causal_decode<T, D, 64, 8>(a, q, k, v, out);
    }
    return hipErrorInvalidValue;
}

template <int M, bool RELU>
static hipError_t launch_causal_tile(const LaunchArgs& a, const bf16x8* ompack, long long om_head_vecs, const bf16* q,
                                     const bf16* k, const bf16* v, bf16* out) {
    constexpr size_t bytes = TileSmem<M>::BYTES;
    static_assert(bytes <= kMaxLds, "causal_tile LDS");
    auto kern = causal_tile_kernel<M, RELU>;
    (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    hipLaunchKernelGGL(kern, dim3(a.nseg, a.B * a.H), dim3(512), bytes, a.stream, q, k, v, ompack, om_head_vecs,
                       scan_carry<bf16>(a), scan_shifts(a), out, a.H, a.L, a.seg_len, a.nseg);
    return hipGetLastError();
}

template <int M, bool RELU>
static hipError_t launch_causal_wide(const LaunchArgs& a, const bf16x8* ompack, long long om_head_vecs, const bf16* q,
                                     const bf16* k, const bf16* v, bf16* out) {
    constexpr size_t bytes = WideSmem<M>::BYTES;
    static_assert(bytes <= kMaxLds, "causal_wide LDS");
    auto kern = causal_wide_kernel<M, RELU>;
    (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    hipLaunchKernelGGL(kern, dim3(a.nseg, a.B * a.H, 2), dim3(512), bytes, a.stream, q, k, v, ompack, om_head_vecs,
                       scan_carry<bf16>(a), scan_shifts(a), out, a.H, a.L, a.seg_len, a.nseg);
    return hipGetLastError();
}

template <typename T, int D, int M, bool RELU>
static hipError_t launch_bidir_small(const LaunchArgs& a, const T* q, const T* k, const T* v, T* out, int per_head) {
    constexpr size_t bytes = SmallSmem<T, D, M>::BYTES;
    static_assert(bytes + sizeof(float) * 16 <= kMaxLds, "bidir_small LDS");
    auto kern = bidir_small_kernel<T, D, M, RELU>;
    (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    hipLaunchKernelGGL(kern, dim3(a.B * a.H), dim3(512), bytes, a.stream, q, k, v, a.omega, per_head, out, a.H, a.L);
    return hipGetLastError();
}

template <typename T, int D, bool RELU>
static hipError_t launch_all(const LaunchArgs& a) {
    constexpr int KSD = D < 32 ? 1 : D / 32;
    const long long om_head_vecs = a.omega_per_head ? (long long)(a.m / 16) * KSD * 64 : 0;
    const int om_heads = a.omega_per_head ? a.H : 1;
    vec8<T>* ompack = reinterpret_cast<vec8<T>*>(a.ws_ompack);
    hipStream_t st = a.stream;
    const int BH = a.B * a.H;
    const T* q = reinterpret_cast<const T*>(a.q);
    const T* k = reinterpret_cast<const T*>(a.k);
    const T* v = reinterpret_cast<const T*>(a.v);
    T* out = reinterpret_cast<T*>(a.out);
    if (a.op == OpKind::Features) {
        const long long total = (long long)om_heads * (a.m / 16) * KSD * 64;
        const int pblocks = (int)std::min<long long>((total + 255) / 256, 4096);
        hipLaunchKernelGGL((pack_omega_kernel<T, D>), dim3(pblocks), dim3(256), 0, st, a.omega, ompack, om_heads, a.m);
        const int tiles = (a.L + 15) / 16;
        const int blocks = (tiles + 3) / 4;
        hipLaunchKernelGGL((features_kernel<T, D, RELU>), dim3(blocks, BH), dim3(256), 0, st, q, ompack, om_head_vecs,
                           a.phi, a.log_scale, a.H, a.L, a.m, a.stabilize);
        return hipGetLastError();
    }
    const int per_head = a.omega_per_head ? 1 : 0;
    const int nfg = (a.m + 255) / 256;
    stage_event(a, 0);
    // a carried state over at most one chunk per head: one launch
    if constexpr (!RELU) {
        if (a.op == OpKind::Causal && (a.state_in || a.state_out) && a.L <= kDecodeMaxTokens &&
            causal_decode_shape((int)sizeof(T), D, a.m)) {
            const hipError_t err = dispatch_causal_decode<T, D>(a, q, k, v, out);
            for (int i = 1; i <= 3; ++i) stage_event(a, i);
            return err;
        }
    }
    constexpr int PD_KV = D >= 128 ? 1 : 2;
    // one segment per head and 32 features: the key-split one-kernel path
    // (fp32 with d = 64 would not fit its registers)
    if constexpr (sizeof(T) == 2 ? D <= 64 : D <= 32) {
        if (a.op == OpKind::Bidir && a.nseg == 1 && bidir_small_shape((int)sizeof(T), D, a.m)) {
            const hipError_t err = launch_bidir_small<T, D, 32, RELU>(a, q, k, v, out, per_head);
            for (int i = 1; i <= 3; ++i) stage_event(a, i);
            return err;
        }
    }
    // one segment per head: the one-kernel bidirectional path when its
    // operand stages fit beside the sums' static LDS
    if (a.op == OpKind::Bidir && a.nseg == 1 && bidir_one_kernel((int)sizeof(T), D, a.m)) {
        auto kern = bidir_head_kernel<T, D, PD_KV, RELU>;
        static const size_t static_lds = [kern] {
            hipFuncAttributes at{};
            return hipFuncGetAttributes(&at, (const void*)kern) == hipSuccess ? (size_t)at.sharedSizeBytes
                                                                              : kMaxLds;
        }();
        constexpr int KSD = D < 32 ? 1 : D / 32;
        const size_t dyn = sizeof(vec8<T>) * 64 * ((size_t)(D / 16 + 1) * (a.m / 32) + (size_t)(a.m / 16) * KSD);
        if (static_lds + dyn <= kMaxLds) {
            (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
            hipLaunchKernelGGL(kern, dim3(BH), dim3(512), dyn, st, q, k, v, a.omega, per_head,
                               reinterpret_cast<T*>(a.ws_partial), a.ws_pmax, out, a.H, a.L, a.m);
            for (int i = 1; i <= 3; ++i) stage_event(a, i);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((kv_partial_kernel<T, D, PD_KV, RELU>), dim3(a.nseg, BH, nfg), dim3(512), 0, st, k, v, a.omega, per_head,
                       reinterpret_cast<T*>(a.ws_partial), a.ws_pmax, a.H, a.L, a.m, a.seg_len, a.nseg,
                       causal_carry_free(a) ? ompack : nullptr);
    stage_event(a, 1);
    const int nfb = a.m / 32;
    const int mode = a.op == OpKind::Bidir ? 0 : 1;
    if (!causal_carry_free(a)) {
        hipLaunchKernelGGL((merge_scan_kernel<T, D>), dim3(nfb, BH, 2), dim3(64 * (D / 16 + 1)), 0, st,
                           reinterpret_cast<const T*>(a.ws_partial), a.ws_pmax, a.omega, per_head, a.H, a.m, a.nseg,
                           mode, reinterpret_cast<vec8<T>*>(a.ws_kvpack), a.ws_mmax, static_cast<T*>(a.ws_carry),
                           a.ws_cmax, ompack, mode == 1 ? a.state_in : nullptr, mode == 1 ? a.state_out : nullptr);
    }
    stage_event(a, 2);
    if (a.op == OpKind::Bidir) {
        constexpr int NTT = 2;
        const size_t om_b = sizeof(vec8<T>) * 64 * (size_t)(a.m / 16) * KSD;
        const size_t kv_b = sizeof(vec8<T>) * 64 * (size_t)(D / 16 + 1) * (a.m / 32);
        const vec8<T>* kvp = reinterpret_cast<const vec8<T>*>(a.ws_kvpack);
        auto launch_out = [&](auto nw_c) {
            constexpr int NW = decltype(nw_c)::value;
            const int tok_per_wg = NW * 16 * NTT;
            const int blocks = (a.L + tok_per_wg - 1) / tok_per_wg;
            constexpr size_t lds_free = kMaxLds - sizeof(float) * kBidirOutStaticFloats;
            if (om_b + kv_b <= lds_free) {
                auto kern = bidir_out_kernel<T, D, true, true, NW, RELU>;
                (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)(om_b + kv_b));
                hipLaunchKernelGGL(kern, dim3(blocks, BH), dim3(64 * NW), om_b + kv_b, st, q, ompack, om_head_vecs, kvp,
                                   a.ws_mmax, out, a.H, a.L, a.m);
            } else if (kv_b <= lds_free) {
                auto kern = bidir_out_kernel<T, D, false, true, NW, RELU>;
                (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kv_b);
                hipLaunchKernelGGL(kern, dim3(blocks, BH), dim3(64 * NW), kv_b, st, q, ompack, om_head_vecs, kvp, a.ws_mmax,
                                   out, a.H, a.L, a.m);
            } else {
                auto kern = bidir_out_kernel<T, D, false, false, NW, RELU>;
                hipLaunchKernelGGL(kern, dim3(blocks, BH), dim3(64 * NW), 0, st, q, ompack, om_head_vecs, kvp, a.ws_mmax,
                                   out, a.H, a.L, a.m);
            }
        };
        // waves per workgroup: sixteen where the registers allow (bf16,
        // d <= 64), so each staging of the operands serves 512 queries; twelve
        // (384 queries) when sixteen-wave workgroups would leave compute units
        // idle and twelve-wave ones still fit in one round (1 x 8 x 12288:
        // 256 workgroups instead of 192)
        if constexpr (sizeof(T) == 2 && D <= 64) {
            const long long wg16 = (long long)BH * ((a.L + 511) / 512);
            const long long wg12 = (long long)BH * ((a.L + 383) / 384);
            if (wg16 < kTargetWorkgroups && wg12 <= kTargetWorkgroups)
                launch_out(IntC<12>{});
            else
                launch_out(IntC<16>{});
        } else {
            launch_out(IntC<8>{});
        }
        stage_event(a, 3);
        return hipGetLastError();
    }
    if constexpr (std::is_same<T, bf16>::value && D == 64) {
        // 64-token chunks: the tile scan; 32-token chunks of the same shapes
        // take the feature-split scan below
        if (a.chunk == 64) {
            hipError_t err = a.m == 64    ? launch_causal_tile<64, RELU>(a, ompack, om_head_vecs, q, k, v, out)
                             : a.m == 128 ? launch_causal_tile<128, RELU>(a, ompack, om_head_vecs, q, k, v, out)
                                          : launch_causal_tile<256, RELU>(a, ompack, om_head_vecs, q, k, v, out);
            stage_event(a, 3);
            return err;
        }
    }
    if constexpr (std::is_same<T, bf16>::value && D == 128) {
        if (a.m == 256 || a.m == 512) {
            hipError_t err = a.m == 256 ? launch_causal_wide<256, RELU>(a, ompack, om_head_vecs, q, k, v, out)
                                        : launch_causal_wide<512, RELU>(a, ompack, om_head_vecs, q, k, v, out);
            stage_event(a, 3);
            return err;
        }
    }
    // the feature-split scan; only the (features per wave, waves) pairs that
    // causal_config can return for this element type and d are instantiated
    const CausalCfg cfg = causal_config((int)sizeof(T), D, a.m);
    hipError_t err = hipErrorInvalidValue;
    constexpr bool narrow = (sizeof(T) == 2 && D == 128) || (sizeof(T) == 4 && D == 64);
    if (cfg.fw == 32 && cfg.w == 1) err = launch_causal<T, D, 32, 1, RELU>(a, ompack, om_head_vecs, q, k, v, out);
    if constexpr (narrow) {
        if (cfg.fw == 32 && cfg.w == 2) err = launch_causal<T, D, 32, 2, RELU>(a, ompack, om_head_vecs, q, k, v, out);
        else if (cfg.fw == 32 && cfg.w == 4) err = launch_causal<T, D, 32, 4, RELU>(a, ompack, om_head_vecs, q, k, v, out);
        if constexpr (sizeof(T) == 4) {  // m = 256 (bf16, d = 128, runs the column-half scan)
            if (cfg.fw == 32 && cfg.w == 8) err = launch_causal<T, D, 32, 8, RELU>(a, ompack, om_head_vecs, q, k, v, out);
        }
    } else {
        if (cfg.fw == 64 && cfg.w == 1) err = launch_causal<T, D, 64, 1, RELU>(a, ompack, om_head_vecs, q, k, v, out);
        else if (cfg.fw == 64 && cfg.w == 2) err = launch_causal<T, D, 64, 2, RELU>(a, ompack, om_head_vecs, q, k, v, out);
        else if (cfg.fw == 64 && cfg.w == 4) err = launch_causal<T, D, 64, 4, RELU>(a, ompack, om_head_vecs, q, k, v, out);
        else if (cfg.fw == 64 && cfg.w == 8) err = launch_causal<T, D, 64, 8, RELU>(a, ompack, om_head_vecs, q, k, v, out);
    }
    stage_event(a, 3);
    return err;
}

template <bool RELU>
static hipError_t launch_kind(const LaunchArgs& a) {
    if (a.dtype_bytes == 2) {
        switch (a.D) {
            case 16: return launch_all<bf16, 16, RELU>(a);
            case 32: return launch_all<bf16, 32, RELU>(a);
            case 64: return launch_all<bf16, 64, RELU>(a);
            case 128: return launch_all<bf16, 128, RELU>(a);
        }
    } else {
        switch (a.D) {
            case 16: return launch_all<float, 16, RELU>(a);
            case 32: return launch_all<float, 32, RELU>(a);
            case 64: return launch_all<float, 64, RELU>(a);
        }
    }
    return hipErrorInvalidValue;
}

hipError_t launch(const LaunchArgs& a) { return a.relu ? launch_kind<true>(a) : launch_kind<false>(a); }

}  // namespace favor
