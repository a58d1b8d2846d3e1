// Host-side planning helpers shared by the C ABI (argument validation,
// workspace sizing) and the kernel launchers: which causal scan a shape runs,
// its chunk length and its LDS footprint.  No device code.
#include "favor_kernels.h"

namespace favor {

int causal_chunk_tokens(int dtype_bytes, int D, int m) {
    return (dtype_bytes == 2 && D == 64 && (m == 64 || m == 128 || m == 256)) ? 64 : 32;
}

bool causal_wide_shape(int dtype_bytes, int D, int m) { return dtype_bytes == 2 && D == 128 && (m == 256 || m == 512); }

CausalCfg causal_config(int dtype_bytes, int D, int m) {
    // The feature-split scan: features per wave (fw) and waves (w = m / fw).
    // A wave keeps its state slice fw x (D + 1) fp32 and its projection
    // operands in registers; where 64 features of that would not fit beside
    // the tiles in flight (bf16 with d = 128, fp32 with d = 64), waves take
    // 32 features each.
    CausalCfg c{0, 0, 0};
    const bool narrow = (dtype_bytes == 2 && D == 128) || (dtype_bytes == 4 && D == 64);
    if (m == 32) {
        c = CausalCfg{32, 1, 1};
    } else if (narrow && (m == 64 || m == 128 || m == 256)) {
        c = CausalCfg{32, m / 32, m / 32};
    } else if (!narrow && (m == 64 || m == 128 || m == 256 || m == 512)) {
        c = CausalCfg{64, m / 64, m / 64};
    }
    return c;
}

size_t causal_smem_bytes(int dtype_bytes, int D, int m) {
    // the d = 128 scan of its own (bf16, m in {256, 512}) fits by construction
    if (causal_wide_shape(dtype_bytes, D, m)) return 0;
    // The feature-split scan with one partial buffer (its smallest form).
    const CausalCfg c = causal_config(dtype_bytes, D, m);
    if (c.w == 0 || (dtype_bytes == 4 && D >= 128)) return ~(size_t)0;
    const size_t eb = (size_t)dtype_bytes;
    const size_t stage = 3 * 32 * (size_t)(D + 16 / dtype_bytes);
    return eb * 2 * stage + eb * (size_t)c.w * 32 * (c.fw + 16 / dtype_bytes) +
           sizeof(float) * (size_t)c.w * 32 * (D + 4) + sizeof(float) * (size_t)c.w * 32 + sizeof(float) * 2 * 2 * 32;
}

bool causal_decode_shape(int dtype_bytes, int D, int m) {
    // the one-launch path for calls that carry a state over at most one
    // 32-token chunk: the feature-split scan's configurations (bf16 with
    // d = 128 and m >= 256 has none: its scan splits the value columns)
    const CausalCfg c = causal_config(dtype_bytes, D, m);
    if (c.w == 0) return false;
    const bool narrow = (dtype_bytes == 2 && D == 128) || (dtype_bytes == 4 && D == 64);
    return !narrow || c.w <= 4 || (dtype_bytes == 4 && c.w == 8);
}

bool bidir_small_shape(int dtype_bytes, int D, int m) {
    // the key-split one-kernel path: every wave sums all 32 features over its
    // own keys (its sums and operands fit the registers for these d)
    return m == 32 && (dtype_bytes == 2 ? D <= 64 : D <= 32);
}

bool bidir_one_kernel(int dtype_bytes, int D, int m) {
    // The one-kernel path holds in LDS the segment-sum pass's staged K/V tiles
    // (three slots of two 64-row tiles, row stride D + 16 / dtype_bytes) and
    // row norms, the per-block key shifts (16 floats), and the two output
    // operands (packed [KV | z]^T: (D/16 + 1) m/32 tiles; packed projection:
    // m/16 max(1, D/32) tiles; 64 lanes x 8 elements each).
    if (bidir_small_shape(dtype_bytes, D, m)) return true;
    if (m > 256 || (dtype_bytes == 4 && D >= 128)) return false;
    const size_t eb = (size_t)dtype_bytes;
    const size_t ksd = D < 32 ? 1 : (size_t)D / 32;
    const size_t lds = eb * 3 * 2 * 64 * (size_t)(D + 16 / dtype_bytes) + sizeof(float) * (3 * 64 + 16) +
                       8 * eb * 64 * ((size_t)(D / 16 + 1) * (m / 32) + (size_t)(m / 16) * ksd);
    return lds <= kMaxLds;
}

}  // namespace favor
