// Host-side planning helpers shared by the C ABI (argument validation,
// workspace sizing) and the kernel launchers: which causal scan a shape runs,
// its chunk length and its LDS footprint.  No device code.
#include "favor_kernels.h"

namespace favor {

int causal_chunk_tokens(int dtype_bytes, int D, int m) {
    return (dtype_bytes == 2 && D == 64 && (m == 64 || m == 128 || m == 256)) ? 64 : 32;
}

CausalCfg causal_config(int D, int m) {
    // Features per wave (fw) and waves (w = m / fw): the wave's state slice
    // fw x (D + 16) fp32 lives in registers.
    CausalCfg c{0, 0, 0};
    if (m == 32) {
        c = CausalCfg{32, 1, 1};
    } else if (m == 64 || m == 128 || m == 256) {
        c = CausalCfg{64, m / 64, m / 64};
    } else if (m == 512) {
        c = D <= 64 ? CausalCfg{64, 8, 8} : CausalCfg{128, 4, 4};
    }
    return c;
}

size_t causal_smem_bytes(int dtype_bytes, int D, int m) {
    // Same layout as CausalSmem with one partial buffer (the smallest form).
    const CausalCfg c = causal_config(D, m);
    if (c.w == 0 || (dtype_bytes == 4 && D >= 128)) return ~(size_t)0;
    const size_t eb = (size_t)dtype_bytes;
    const size_t stage = 3 * 32 * (size_t)(D + 16 / dtype_bytes);
    return eb * 2 * stage + eb * (size_t)c.w * 32 * (c.fw + 16 / dtype_bytes) +
           sizeof(float) * (size_t)c.w * 32 * (D + 4) + sizeof(float) * (size_t)c.w * 32 + sizeof(float) * 2 * 2 * 32;
}

}  // namespace favor
