// Internal interface between the C ABI (favor_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace favor {

// LDS available to one workgroup on gfx950.
constexpr size_t kMaxLds = 160 * 1024;
// Workgroups that fill the chip once: one per compute unit of an MI355X.
constexpr int kTargetWorkgroups = 256;
// Most segments per head the launch plan makes (the merge/scan pass keeps
// their shifts in LDS).
constexpr int kMaxSeg = 256;

enum class OpKind { Features, Bidir, Causal };

struct LaunchArgs {
    OpKind op;
    int dtype_bytes;  // 2 = bf16, 4 = fp32
    int B, H, L, D, m;
    bool omega_per_head;
    bool relu;  // generalised ReLU features instead of the positive ones
    const void *q, *k, *v;  // for Features, q is x
    const float* omega;
    void* out;
    float* phi;
    float* log_scale;
    int stabilize;
    int nseg, seg_len;  // segments per head and their length (multiple of 32)
    int chunk;          // causal: tokens per scan step (32 or 64)
    // workspace regions
    void* ws_ompack;
    void* ws_partial;  // segment sums, in the input type
    float* ws_pmax;
    void* ws_kvpack;
    float* ws_mmax;
    void* ws_carry;  // causal carries, in the input type
    float* ws_cmax;
    // causal only: carried-in and carried-out prefix state (nullptr: none);
    // per head m (d + 1) + 1 floats, see favor_causal_state
    const float* state_in;
    float* state_out;
    hipStream_t stream;
    // optional stage events: events[i] before stage i, events[n_stages] after
    // the last one (nullptr: none)
    void* const* events;
};

struct CausalCfg {
    int fw;    // features per wave
    int maxw;  // waves per workgroup the kernel is compiled for
    int w;     // waves per workgroup = m / fw (0: unsupported)
};

hipError_t launch(const LaunchArgs& a);

// Features over the structured Hadamard projection, built with fast
// Walsh-Hadamard transforms from the seed (favor_features_hadamard).
struct HadamardFeaturesArgs {
    int dtype_bytes;
    int B, H, L, D, m;
    bool relu;
    int omega_per_head;  // 1: the blocks of head h; 0: those of head 0 for every head
    unsigned long long seed;
    const void* x;
    float* phi;
    float* log_scale;
    int stabilize;
    hipStream_t stream;
};
hipError_t launch_hadamard_features(const HadamardFeaturesArgs& a);
// Tokens per step of the causal chunked scan for a shape.
int causal_chunk_tokens(int dtype_bytes, int D, int m);
CausalCfg causal_config(int dtype_bytes, int D, int m);
// Shapes with a one-launch path for causal calls that carry a state over at
// most one 32-token chunk per head.
bool causal_decode_shape(int dtype_bytes, int D, int m);
constexpr int kDecodeMaxTokens = 32;
// Shapes whose causal scan is the d = 128 column-half scan (causal_wide).
bool causal_wide_shape(int dtype_bytes, int D, int m);
// LDS bytes the causal kernel needs (SIZE_MAX when the shape is unsupported).
size_t causal_smem_bytes(int dtype_bytes, int D, int m);
// Shapes whose one-segment bidirectional call runs the key-split kernel
// (m = 32: the waves split the keys instead of the features).
bool bidir_small_shape(int dtype_bytes, int D, int m);
// Whether a bidirectional call planned with one segment per head runs as
// one kernel (the key-split kernel, or the feature-split one where its
// operands and staged tiles fit a compute unit's LDS).
bool bidir_one_kernel(int dtype_bytes, int D, int m);

}  // namespace favor
