// C ABI of the FAVOR+ library: argument validation, work planning, workspace
// layout and dispatch to the gfx950 kernels.  See include/favor.h.
#include "../../include/favor.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "favor_kernels.h"

namespace {

using favor::kTargetWorkgroups;
static_assert(kTargetWorkgroups <= favor::kMaxSeg, "segments per head bounded by the plan");

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Plan {
    int nseg = 1, seg_len = 32;
    size_t ompack = 0, partial = 0, pmax = 0, kvpack = 0, mmax = 0, carry = 0, cmax = 0;
    size_t total = 0;
};

int dtype_bytes(favor_dtype t) { return t == FAVOR_BF16 ? 2 : 4; }

favor_status check_shape(const favor_shape* s, int op) {
    if (!s) return FAVOR_ERR_INVALID_ARG;
    if (s->B < 1 || s->H < 1 || s->L < 0 || s->d < 1 || s->m < 1) return FAVOR_ERR_INVALID_ARG;
    if (s->dtype != FAVOR_F32 && s->dtype != FAVOR_BF16) return FAVOR_ERR_UNSUPPORTED;
    if (s->feature != FAVOR_FEATURE_POSITIVE && s->feature != FAVOR_FEATURE_RELU) return FAVOR_ERR_UNSUPPORTED;
    if (s->d != 16 && s->d != 32 && s->d != 64 && s->d != 128) return FAVOR_ERR_UNSUPPORTED;
    if (s->m % 32 != 0 || s->m > 512) return FAVOR_ERR_UNSUPPORTED;
    if (s->m > 256 && s->m % 64 != 0) return FAVOR_ERR_UNSUPPORTED;
    if (s->dtype == FAVOR_F32 && s->d > 64) return FAVOR_ERR_UNSUPPORTED;
    if (s->omega_head_stride != 0 && s->omega_head_stride != (long long)s->m * s->d) return FAVOR_ERR_INVALID_ARG;
    const long long elems = (long long)s->B * s->H * s->L * s->d;
    if (elems >= (1LL << 31)) return FAVOR_ERR_UNSUPPORTED;
    if (op == FAVOR_OP_CAUSAL && favor::causal_smem_bytes(dtype_bytes(s->dtype), s->d, s->m) > favor::kMaxLds)
        return FAVOR_ERR_UNSUPPORTED;
    return FAVOR_OK;
}

Plan make_plan(int op, const favor_shape& s) {
    Plan p;
    const int BH = s.B * s.H;
    const int D = s.d, m = s.m;
    const int ksd = D < 32 ? 1 : D / 32;
    const size_t vec8 = 8 * (size_t)dtype_bytes(s.dtype);
    const int om_heads = s.omega_head_stride ? s.H : 1;
    const int tiles = (s.L + 31) / 32;
    p.ompack = align256((size_t)om_heads * (m / 16) * ksd * 64 * vec8);
    if (op == FAVOR_OP_FEATURES || s.L == 0) {
        p.total = p.ompack;
        return p;
    }
    const int nfg = (m + 255) / 256;  // feature groups of the partial pass
    // one partial-pass (bidirectional) or chunk-scan (causal) workgroup per
    // compute unit
    // the causal scan for bf16, d = 128 (m = 256, 512) runs two workgroups per
    // (segment, head), one per half of the value columns
    const bool wide = op == FAVOR_OP_CAUSAL && s.dtype == FAVOR_BF16 && D == 128 && (m == 256 || m == 512);
    const int per_seg = op == FAVOR_OP_BIDIR ? BH * nfg : BH * (wide ? 2 : 1);
    int nseg = (kTargetWorkgroups + per_seg - 1) / per_seg;
    if (nseg < 1) nseg = 1;
    if (nseg > tiles) nseg = tiles;
    const int per = (s.L + nseg - 1) / nseg;
    // segments are whole 64-token steps where possible
    const int gran = s.L >= 64 * nseg ? 64 : 32;
    p.seg_len = ((per + gran - 1) / gran) * gran;
    p.nseg = (s.L + p.seg_len - 1) / p.seg_len;
    const size_t rows = (size_t)BH * p.nseg * m;
    p.partial = align256(rows * (D + 1) * sizeof(float));
    p.pmax = align256((size_t)BH * p.nseg * (m / 32) * sizeof(float));
    if (op == FAVOR_OP_BIDIR) {
        p.kvpack = align256((size_t)BH * (D / 16 + 1) * (m / 32) * 64 * vec8);
        p.mmax = align256((size_t)BH * (m / 32) * sizeof(float));
    } else {
        p.carry = align256(rows * (D + 1) * sizeof(float));
        p.cmax = align256((size_t)BH * p.nseg * (m / 32) * sizeof(float));
    }
    p.total = p.ompack + p.partial + p.pmax + p.kvpack + p.mmax + p.carry + p.cmax;
    return p;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

favor_status run(int op, const favor_shape* s, const void* q, const void* k, const void* v, const float* omega,
                 void* out, float* phi, float* log_scale, int stabilize, void* ws, size_t ws_bytes, void* stream,
                 void* const* events = nullptr, const float* state_in = nullptr, float* state_out = nullptr) {
    favor_status st = check_shape(s, op);
    if (st != FAVOR_OK) return st;
    if (s->L == 0) return FAVOR_OK;
    const int eb = dtype_bytes(s->dtype);
    const size_t xbytes = (size_t)s->B * s->H * s->L * s->d * eb;
    if (!omega || !aligned(omega, 4)) return FAVOR_ERR_INVALID_ARG;
    if (op == FAVOR_OP_FEATURES) {
        if (!q || !phi || !aligned(q, 16) || !aligned(phi, 16)) return FAVOR_ERR_INVALID_ARG;
        if (stabilize && (!log_scale || !aligned(log_scale, 4))) return FAVOR_ERR_INVALID_ARG;
        const size_t pbytes = (size_t)s->B * s->H * s->L * s->m * sizeof(float);
        if (overlaps(phi, pbytes, q, xbytes)) return FAVOR_ERR_INVALID_ARG;
        if (stabilize && overlaps(log_scale, (size_t)s->B * s->H * s->L * 4, phi, pbytes)) return FAVOR_ERR_INVALID_ARG;
    } else {
        if (!q || !k || !v || !out) return FAVOR_ERR_INVALID_ARG;
        if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16)) return FAVOR_ERR_INVALID_ARG;
        if (overlaps(out, xbytes, q, xbytes) || overlaps(out, xbytes, k, xbytes) || overlaps(out, xbytes, v, xbytes))
            return FAVOR_ERR_INVALID_ARG;
    }
    const Plan p = make_plan(op, *s);
    if (!ws || !aligned(ws, 256) || ws_bytes < p.total) return FAVOR_ERR_WORKSPACE;
    if (op != FAVOR_OP_FEATURES && overlaps(out, xbytes, ws, p.total)) return FAVOR_ERR_INVALID_ARG;
    if (state_in || state_out) {
        const size_t sbytes = (size_t)s->B * s->H * ((size_t)s->m * (s->d + 1) + 1) * sizeof(float);
        if (!aligned(state_in, 4) || !aligned(state_out, 4)) return FAVOR_ERR_INVALID_ARG;
        if (overlaps(state_in, sbytes, ws, p.total)) return FAVOR_ERR_INVALID_ARG;
        if (state_out) {
            const size_t obytes = (size_t)(s->omega_head_stride ? s->H : 1) * s->m * s->d * sizeof(float);
            if (overlaps(state_out, sbytes, state_in, sbytes) || overlaps(state_out, sbytes, ws, p.total) ||
                overlaps(state_out, sbytes, out, xbytes) || overlaps(state_out, sbytes, q, xbytes) ||
                overlaps(state_out, sbytes, k, xbytes) || overlaps(state_out, sbytes, v, xbytes) ||
                overlaps(state_out, sbytes, omega, obytes))
                return FAVOR_ERR_INVALID_ARG;
        }
    }

    favor::LaunchArgs a{};
    a.op = op == FAVOR_OP_FEATURES ? favor::OpKind::Features
                                   : (op == FAVOR_OP_BIDIR ? favor::OpKind::Bidir : favor::OpKind::Causal);
    a.dtype_bytes = eb;
    a.B = s->B; a.H = s->H; a.L = s->L; a.D = s->d; a.m = s->m;
    a.omega_per_head = s->omega_head_stride != 0;
    a.relu = s->feature == FAVOR_FEATURE_RELU;
    a.q = q; a.k = k; a.v = v; a.omega = omega; a.out = out;
    a.phi = phi; a.log_scale = log_scale; a.stabilize = stabilize ? 1 : 0;
    a.nseg = p.nseg; a.seg_len = p.seg_len;
    char* base = static_cast<char*>(ws);
    size_t off = 0;
    a.ws_ompack = base + off; off += p.ompack;
    a.ws_partial = reinterpret_cast<float*>(base + off); off += p.partial;
    a.ws_pmax = reinterpret_cast<float*>(base + off); off += p.pmax;
    a.ws_kvpack = base + off; off += p.kvpack;
    a.ws_mmax = reinterpret_cast<float*>(base + off); off += p.mmax;
    a.ws_carry = reinterpret_cast<float*>(base + off); off += p.carry;
    a.ws_cmax = reinterpret_cast<float*>(base + off); off += p.cmax;
    a.state_in = state_in;
    a.state_out = state_out;
    a.stream = static_cast<hipStream_t>(stream);
    a.events = events;
    return favor::launch(a) == hipSuccess ? FAVOR_OK : FAVOR_ERR_HIP;
}

}  // namespace

extern "C" {

size_t favor_workspace_bytes(int op, const favor_shape* shape, int chunk) {
    (void)chunk;
    if (op != FAVOR_OP_FEATURES && op != FAVOR_OP_BIDIR && op != FAVOR_OP_CAUSAL) return 0;
    if (check_shape(shape, op) != FAVOR_OK) return 0;
    return make_plan(op, *shape).total;
}

favor_status favor_features(const favor_shape* shape, const void* x, const float* omega, float* phi,
                            float* log_scale, int stabilize, void* ws, size_t ws_bytes, void* stream) {
    return run(FAVOR_OP_FEATURES, shape, x, nullptr, nullptr, omega, nullptr, phi, log_scale, stabilize, ws, ws_bytes,
               stream);
}

favor_status favor_bidir(const favor_shape* shape, const void* q, const void* k, const void* v, const float* omega,
                         void* out, void* ws, size_t ws_bytes, void* stream) {
    return run(FAVOR_OP_BIDIR, shape, q, k, v, omega, out, nullptr, nullptr, 0, ws, ws_bytes, stream);
}

favor_status favor_causal(const favor_shape* shape, const void* q, const void* k, const void* v, const float* omega,
                          void* out, int chunk, void* ws, size_t ws_bytes, void* stream) {
    if (chunk != 0 && shape && chunk != favor::causal_chunk_tokens(dtype_bytes(shape->dtype), shape->d, shape->m))
        return FAVOR_ERR_UNSUPPORTED;
    return run(FAVOR_OP_CAUSAL, shape, q, k, v, omega, out, nullptr, nullptr, 0, ws, ws_bytes, stream);
}

favor_status favor_causal_state(const favor_shape* shape, const void* q, const void* k, const void* v,
                                const float* omega, void* out, int chunk, const float* state_in, float* state_out,
                                void* ws, size_t ws_bytes, void* stream) {
    if (chunk != 0 && shape && chunk != favor::causal_chunk_tokens(dtype_bytes(shape->dtype), shape->d, shape->m))
        return FAVOR_ERR_UNSUPPORTED;
    if (shape && shape->feature != FAVOR_FEATURE_POSITIVE) return FAVOR_ERR_UNSUPPORTED;
    return run(FAVOR_OP_CAUSAL, shape, q, k, v, omega, out, nullptr, nullptr, 0, ws, ws_bytes, stream, nullptr,
               state_in, state_out);
}

favor_status favor_bidir_profiled(const favor_shape* shape, const void* q, const void* k, const void* v,
                                  const float* omega, void* out, void* ws, size_t ws_bytes, void* stream,
                                  void* const* events, int n_events) {
    if (!events || n_events < FAVOR_N_STAGES + 1) return FAVOR_ERR_INVALID_ARG;
    for (int i = 0; i <= FAVOR_N_STAGES; ++i)
        if (!events[i]) return FAVOR_ERR_INVALID_ARG;
    return run(FAVOR_OP_BIDIR, shape, q, k, v, omega, out, nullptr, nullptr, 0, ws, ws_bytes, stream, events);
}

favor_status favor_causal_profiled(const favor_shape* shape, const void* q, const void* k, const void* v,
                                   const float* omega, void* out, int chunk, void* ws, size_t ws_bytes, void* stream,
                                   void* const* events, int n_events) {
    if (!events || n_events < FAVOR_N_STAGES + 1) return FAVOR_ERR_INVALID_ARG;
    for (int i = 0; i <= FAVOR_N_STAGES; ++i)
        if (!events[i]) return FAVOR_ERR_INVALID_ARG;
    if (chunk != 0 && shape && chunk != favor::causal_chunk_tokens(dtype_bytes(shape->dtype), shape->d, shape->m))
        return FAVOR_ERR_UNSUPPORTED;
    return run(FAVOR_OP_CAUSAL, shape, q, k, v, omega, out, nullptr, nullptr, 0, ws, ws_bytes, stream, events);
}

const char* favor_status_string(favor_status status) {
    switch (status) {
        case FAVOR_OK: return "ok";
        case FAVOR_ERR_INVALID_ARG: return "invalid argument";
        case FAVOR_ERR_UNSUPPORTED: return "unsupported shape or dtype";
        case FAVOR_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        case FAVOR_ERR_HIP: return "HIP launch error";
    }
    return "unknown status";
}

}  // extern "C"
