// favor_causal_noalloc: causal FAVOR+ for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).  The same kernels and launch plan as favor_causal, with
// the workspace taken from a file-scope device array of fixed size instead of
// a caller-provided buffer.
#include "../../include/favor.h"

#include <hip/hip_runtime.h>

#include <mutex>

// Defined in favor_api.cpp: the workspace size of a causal call with a given
// plan (0 = invalid shape or plan), and the causal call on an explicit
// workspace.
size_t favor_internal_workspace_bytes(int op, const favor_shape* shape, int chunk, int segments);
favor_status favor_internal_causal(const favor_shape* shape, const void* q, const void* k, const void* v,
                                   const float* omega, void* out, int chunk, int segments, void* ws, size_t ws_bytes,
                                   void* stream);

namespace {

static_assert(FAVOR_NOALLOC_SCRATCH_BYTES % 256 == 0, "whole 256-byte blocks");

// One copy per GPU, held until the process ends.  Host code must never pass
// this name to a kernel or copy: on the host it is only a stand-in for the
// symbol; its device address comes from hipGetSymbolAddress below.
static __device__ __align__(256) unsigned char scratch[FAVOR_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 256;
std::mutex g_mutex;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each device, once resolved

// The array's address on the current device, resolved once per device.
favor_status scratch_on_current_device(void** ptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FAVOR_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FAVOR_ERR_HIP;
        g_scratch[dev] = p;
    }
    *ptr = g_scratch[dev];
    return FAVOR_OK;
}

}  // namespace

extern "C" favor_status favor_causal_noalloc(const favor_shape* shape, const void* q, const void* k, const void* v,
                                             const float* omega, void* out, int chunk, void* stream) {
    const size_t need = favor_internal_workspace_bytes(FAVOR_OP_CAUSAL, shape, chunk, 0);
    // an invalid shape or chunk: the ordinary validation reports which
    if (need == 0) return favor_internal_causal(shape, q, k, v, omega, out, chunk, 0, nullptr, 0, stream);
    if (need > FAVOR_NOALLOC_SCRATCH_BYTES) return FAVOR_ERR_WORKSPACE;
    void* ws = nullptr;
    const favor_status st = scratch_on_current_device(&ws);
    if (st != FAVOR_OK) return st;
    // nothing in the workspace needs to start at zero: every kernel writes
    // the regions it reads later in the same call
    return favor_internal_causal(shape, q, k, v, omega, out, chunk, 0, ws, FAVOR_NOALLOC_SCRATCH_BYTES, stream);
}
