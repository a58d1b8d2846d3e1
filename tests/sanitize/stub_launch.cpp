// Host-only stand-in for the kernel launcher, for the sanitizer build of the
// C ABI (favor_api.cpp, favor_plan.cpp): instead of launching kernels it
// checks the launch plan and the workspace layout the ABI computed, against
// the bounds the test program (abi_driver.cpp) registered for the call.  Test
// infrastructure only.
#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "../../positive_random_feature_amd/csrc/favor_kernels.h"

// set by the test program before each call that should reach a launch
extern "C" {
const char* g_ws_base = nullptr;
size_t g_ws_bytes = 0;
int g_launches = 0;
}

static void fail(const char* what) {
    std::fprintf(stderr, "stub_launch: %s\n", what);
    std::abort();
}

static void region(const void* p, size_t bytes, const char* name) {
    const char* c = static_cast<const char*>(p);
    if (bytes == 0) return;
    if (c < g_ws_base || c + bytes > g_ws_base + g_ws_bytes) {
        std::fprintf(stderr, "stub_launch: workspace region %s [%p, +%zu) outside [%p, +%zu)\n", name, p, bytes,
                     (const void*)g_ws_base, g_ws_bytes);
        std::abort();
    }
    if (((uintptr_t)c - (uintptr_t)g_ws_base) % 256 != 0) fail("workspace region not 256-byte aligned");
}

namespace favor {

hipError_t launch(const LaunchArgs& a) {
    ++g_launches;
    if (!g_ws_base) fail("launch reached without a registered workspace");
    const size_t BH = (size_t)a.B * a.H;
    const size_t eb = (size_t)a.dtype_bytes;
    const size_t ksd = a.D < 32 ? 1 : (size_t)a.D / 32;
    const size_t om_heads = a.omega_per_head ? (size_t)a.H : 1;
    // packed projection: (m / 16) * ksd * 64 lanes * 8 elements per head
    region(a.ws_ompack, om_heads * (a.m / 16) * ksd * 64 * 8 * eb, "ompack");
    if (a.op == OpKind::Features) return hipSuccess;
    if (a.nseg < 1 || a.seg_len < 32 || a.seg_len % 32 != 0) fail("bad segment plan");
    if ((size_t)a.nseg * a.seg_len < (size_t)a.L) fail("segments do not cover the sequence");
    if ((size_t)(a.nseg - 1) * a.seg_len >= (size_t)a.L) fail("an empty segment");
    if (a.nseg > kMaxSeg) fail("more segments than the merge pass holds");
    const size_t rows = BH * a.nseg * a.m;
    region(a.ws_partial, rows * (a.D + 1) * eb, "partial");  // segment sums in the input type
    region(a.ws_pmax, BH * a.nseg * (a.m / 32) * sizeof(float), "pmax");
    if (a.op == OpKind::Bidir) {
        region(a.ws_kvpack, BH * (a.D / 16 + 1) * (a.m / 32) * 64 * 8 * eb, "kvpack");
        region(a.ws_mmax, BH * (a.m / 32) * sizeof(float), "mmax");
    } else {
        if (a.chunk != 32 && a.chunk != 64) fail("bad chunk");
        region(a.ws_carry, rows * (a.D + 1) * eb, "carry");  // in the input type
        region(a.ws_cmax, BH * a.nseg * (a.m / 32) * sizeof(float), "cmax");
    }
    return hipSuccess;
}

// The transform-features launch takes no workspace; the stub checks the
// arguments the ABI forwards.
hipError_t launch_hadamard_features(const HadamardFeaturesArgs& a) {
    ++g_launches;
    if (!a.x || !a.phi || a.L < 1 || a.m < 1 || (a.stabilize && !a.log_scale)) fail("bad transform-features launch");
    if (a.D != 16 && a.D != 32 && a.D != 64 && a.D != 128) fail("bad d for the transform features");
    return hipSuccess;
}

}  // namespace favor
