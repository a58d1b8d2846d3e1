// C ABI of the FAVOR+ library: argument validation, work planning, workspace
// layout and dispatch to the gfx950 kernels.  See include/favor.h.
#include "../../include/favor.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "favor_kernels.h"

#include <algorithm>

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
    // B*H*L*d < 2^31, multiplied one factor at a time so that no product can
    // overflow (each factor and each partial product stays below 2^31)
    long long elems = 1;
    for (const int f : {s->B, s->H, s->L, s->d}) {
        elems *= f;
        if (elems >= (1LL << 31)) return FAVOR_ERR_UNSUPPORTED;
    }
    // the kernels index (batch, head) pairs with a grid dimension whose
    // hardware limit is 65535
    if ((long long)s->B * s->H > 65535) return FAVOR_ERR_UNSUPPORTED;
    if (op == FAVOR_OP_CAUSAL && favor::causal_smem_bytes(dtype_bytes(s->dtype), s->d, s->m) > favor::kMaxLds)
        return FAVOR_ERR_UNSUPPORTED;
    return FAVOR_OK;
}

// chunk: effective causal chunk length (ignored otherwise); segments: the
// requested segments per head, 0 = one workgroup per compute unit.
Plan make_plan(int op, const favor_shape& s, int segments = 0) {
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
    int nseg = segments > 0 ? segments : (kTargetWorkgroups + per_seg - 1) / per_seg;
    // bidirectional segments of at least 256 tokens when the partial sums are
    // large (m >= 128): shorter ones cost more in the merge than they add in
    // parallelism
    if (segments <= 0 && op == FAVOR_OP_BIDIR && m >= 128) nseg = std::min(nseg, std::max(1, s.L / 256));
    // causal segments of at least 64 tokens: shorter ones leave the scan's
    // 64-token chunks half empty and measured slower (2x8x512 bf16, d = 64,
    // m = 256: 27.1 us with 16 segments, 21.9 us with 8)
    if (segments <= 0 && op == FAVOR_OP_CAUSAL) nseg = std::min(nseg, std::max(1, s.L / 64));
    // many heads of short bidirectional sequences: one segment per head, so
    // the call runs as one kernel (a workgroup per head does the sums and
    // the output pass) where that kernel fits.  Measured crossover (bf16,
    // d = 64, m = 256): it wins from 128 heads up to 512 tokens and from 64
    // heads up to 384; with fewer heads or longer sequences the segments'
    // parallelism wins
    const int eb = s.dtype == FAVOR_BF16 ? 2 : 4;
    bool short_seq = BH >= 128 ? s.L <= 512 : BH >= 64 && s.L <= 384;
    // with 32 features the key-split kernel keeps all its waves busy: one
    // segment wins up to 512 tokens at any head count, and up to 4096 from
    // 128 heads
    if (favor::bidir_small_shape(eb, D, m)) short_seq = s.L <= 512 || (BH >= 128 && s.L <= 4096);
    if (segments <= 0 && op == FAVOR_OP_BIDIR && short_seq && favor::bidir_one_kernel(eb, D, m)) nseg = 1;
    if (nseg < 1) nseg = 1;
    if (nseg > tiles) nseg = tiles;
    const int per = (s.L + nseg - 1) / nseg;
    // segments are whole 64-token steps where possible
    const int gran = s.L >= 64 * nseg ? 64 : 32;
    p.seg_len = ((per + gran - 1) / gran) * gran;
    p.nseg = (s.L + p.seg_len - 1) / p.seg_len;
    const size_t rows = (size_t)BH * p.nseg * m;
    // segment sums in the input type (bf16 sums feed bf16 operands downstream)
    p.partial = align256(rows * (D + 1) * (size_t)eb);
    p.pmax = align256((size_t)BH * p.nseg * (m / 32) * sizeof(float));
    if (op == FAVOR_OP_BIDIR) {
        p.kvpack = align256((size_t)BH * (D / 16 + 1) * (m / 32) * 64 * vec8);
        p.mmax = align256((size_t)BH * (m / 32) * sizeof(float));
    } else {
        p.carry = align256(rows * (D + 1) * (size_t)eb);  // causal carries, in the input type too
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

// Effective causal chunk length for a requested one (0 = the shape's
// default), or 0 when the shape has no scan with that length.
int resolve_chunk(const favor_shape* s, int chunk) {
    if (!s) return chunk == 0 ? 32 : 0;
    const int native = favor::causal_chunk_tokens(dtype_bytes(s->dtype), s->d, s->m);
    if (chunk == 0 || chunk == native) return native;
    // the shapes with a 64-token tile scan also run the 32-token scan
    if (chunk == 32 && native == 64) return 32;
    return 0;
}

// Plan overrides: segments per head in [0, kMaxSeg] (0 = automatic).
favor_status check_plan(const favor_plan* plan) {
    if (!plan) return FAVOR_OK;
    if (plan->segments < 0 || plan->segments > favor::kMaxSeg) return FAVOR_ERR_INVALID_ARG;
    return FAVOR_OK;
}

struct Call {
    int op = FAVOR_OP_BIDIR;
    const favor_shape* s = nullptr;
    const void *q = nullptr, *k = nullptr, *v = nullptr;
    const float* omega = nullptr;
    void* out = nullptr;
    float* phi = nullptr;
    float* log_scale = nullptr;
    int stabilize = 0;
    int chunk = 0;     // effective causal chunk length
    int segments = 0;  // requested segments per head (0 = automatic)
    void* ws = nullptr;
    size_t ws_bytes = 0;
    void* stream = nullptr;
    void* const* events = nullptr;
    const float* state_in = nullptr;
    float* state_out = nullptr;
};

favor_status run(const Call& c) {
    const favor_shape* s = c.s;
    const int op = c.op;
    favor_status st = check_shape(s, op);
    if (st != FAVOR_OK) return st;
    if (s->L == 0) return FAVOR_OK;
    const int eb = dtype_bytes(s->dtype);
    const size_t xbytes = (size_t)s->B * s->H * s->L * s->d * eb;
    const size_t obytes = (size_t)(s->omega_head_stride ? s->H : 1) * s->m * s->d * sizeof(float);
    if (!c.omega || !aligned(c.omega, 4)) return FAVOR_ERR_INVALID_ARG;
    const size_t pbytes = (size_t)s->B * s->H * s->L * s->m * sizeof(float);
    const size_t lbytes = (size_t)s->B * s->H * s->L * sizeof(float);
    if (op == FAVOR_OP_FEATURES) {
        if (!c.q || !c.phi || !aligned(c.q, 16) || !aligned(c.phi, 16)) return FAVOR_ERR_INVALID_ARG;
        if (c.stabilize && (!c.log_scale || !aligned(c.log_scale, 4))) return FAVOR_ERR_INVALID_ARG;
        if (overlaps(c.phi, pbytes, c.q, xbytes) || overlaps(c.phi, pbytes, c.omega, obytes)) return FAVOR_ERR_INVALID_ARG;
        if (c.stabilize && (overlaps(c.log_scale, lbytes, c.phi, pbytes) || overlaps(c.log_scale, lbytes, c.q, xbytes) ||
                            overlaps(c.log_scale, lbytes, c.omega, obytes)))
            return FAVOR_ERR_INVALID_ARG;
    } else {
        if (!c.q || !c.k || !c.v || !c.out) return FAVOR_ERR_INVALID_ARG;
        if (!aligned(c.q, 16) || !aligned(c.k, 16) || !aligned(c.v, 16) || !aligned(c.out, 16))
            return FAVOR_ERR_INVALID_ARG;
        if (overlaps(c.out, xbytes, c.q, xbytes) || overlaps(c.out, xbytes, c.k, xbytes) ||
            overlaps(c.out, xbytes, c.v, xbytes) || overlaps(c.out, xbytes, c.omega, obytes))
            return FAVOR_ERR_INVALID_ARG;
    }
    const Plan p = make_plan(op, *s, c.segments);
    if (!c.ws || !aligned(c.ws, 256) || c.ws_bytes < p.total) return FAVOR_ERR_WORKSPACE;
    // the kernels write the workspace while other kernels of the call still
    // read the inputs: it must not overlap any of them, nor the outputs
    if (overlaps(c.ws, p.total, c.q, xbytes) || overlaps(c.ws, p.total, c.omega, obytes)) return FAVOR_ERR_INVALID_ARG;
    if (op == FAVOR_OP_FEATURES) {
        if (overlaps(c.ws, p.total, c.phi, pbytes) || (c.stabilize && overlaps(c.ws, p.total, c.log_scale, lbytes)))
            return FAVOR_ERR_INVALID_ARG;
    } else if (overlaps(c.ws, p.total, c.k, xbytes) || overlaps(c.ws, p.total, c.v, xbytes) ||
               overlaps(c.ws, p.total, c.out, xbytes)) {
        return FAVOR_ERR_INVALID_ARG;
    }
    if (c.state_in || c.state_out) {
        const size_t sbytes = (size_t)s->B * s->H * ((size_t)s->m * (s->d + 1) + 1) * sizeof(float);
        if (!aligned(c.state_in, 4) || !aligned(c.state_out, 4)) return FAVOR_ERR_INVALID_ARG;
        if (overlaps(c.state_in, sbytes, c.ws, p.total) || overlaps(c.state_in, sbytes, c.out, xbytes))
            return FAVOR_ERR_INVALID_ARG;
        if (c.state_out) {
            if (overlaps(c.state_out, sbytes, c.state_in, sbytes) || overlaps(c.state_out, sbytes, c.ws, p.total) ||
                overlaps(c.state_out, sbytes, c.out, xbytes) || overlaps(c.state_out, sbytes, c.q, xbytes) ||
                overlaps(c.state_out, sbytes, c.k, xbytes) || overlaps(c.state_out, sbytes, c.v, xbytes) ||
                overlaps(c.state_out, sbytes, c.omega, obytes))
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
    a.q = c.q; a.k = c.k; a.v = c.v; a.omega = c.omega; a.out = c.out;
    a.phi = c.phi; a.log_scale = c.log_scale; a.stabilize = c.stabilize ? 1 : 0;
    a.nseg = p.nseg; a.seg_len = p.seg_len;
    a.chunk = c.chunk;
    char* base = static_cast<char*>(c.ws);
    size_t off = 0;
    a.ws_ompack = base + off; off += p.ompack;
    a.ws_partial = base + off; off += p.partial;
    a.ws_pmax = reinterpret_cast<float*>(base + off); off += p.pmax;
    a.ws_kvpack = base + off; off += p.kvpack;
    a.ws_mmax = reinterpret_cast<float*>(base + off); off += p.mmax;
    a.ws_carry = base + off; off += p.carry;
    a.ws_cmax = reinterpret_cast<float*>(base + off); off += p.cmax;
    a.state_in = c.state_in;
    a.state_out = c.state_out;
    a.stream = static_cast<hipStream_t>(c.stream);
    a.events = c.events;
    return favor::launch(a) == hipSuccess ? FAVOR_OK : FAVOR_ERR_HIP;
}

Call attention(int op, const favor_shape* shape, const void* q, const void* k, const void* v, const float* omega,
               void* out, void* ws, size_t ws_bytes, void* stream) {
    Call c;
    c.op = op; c.s = shape; c.q = q; c.k = k; c.v = v; c.omega = omega; c.out = out;
    c.ws = ws; c.ws_bytes = ws_bytes; c.stream = stream;
    return c;
}

bool events_ok(void* const* events, int n_events) {
    if (!events || n_events < FAVOR_N_STAGES + 1) return false;
    for (int i = 0; i <= FAVOR_N_STAGES; ++i)
        if (!events[i]) return false;
    return true;
}

}  // namespace

// Workspace size of a call (also used by the entry point without a workspace).
size_t favor_internal_workspace_bytes(int op, const favor_shape* shape, int chunk, int segments) {
    if (op != FAVOR_OP_FEATURES && op != FAVOR_OP_BIDIR && op != FAVOR_OP_CAUSAL) return 0;
    if (check_shape(shape, op) != FAVOR_OK) return 0;
    if (op == FAVOR_OP_CAUSAL && resolve_chunk(shape, chunk) == 0) return 0;
    if (segments < 0 || segments > favor::kMaxSeg) return 0;
    return make_plan(op, *shape, segments).total;
}

// Causal attention on a caller-provided workspace with an explicit plan.
favor_status favor_internal_causal(const favor_shape* shape, const void* q, const void* k, const void* v,
                                   const float* omega, void* out, int chunk, int segments, void* ws, size_t ws_bytes,
                                   void* stream) {
    if (segments < 0 || segments > favor::kMaxSeg) return FAVOR_ERR_INVALID_ARG;
    Call c = attention(FAVOR_OP_CAUSAL, shape, q, k, v, omega, out, ws, ws_bytes, stream);
    c.chunk = resolve_chunk(shape, chunk);
    if (shape && c.chunk == 0) return FAVOR_ERR_UNSUPPORTED;
    c.segments = segments;
    return run(c);
}

extern "C" {

size_t favor_workspace_bytes(int op, const favor_shape* shape, int chunk) {
    return favor_internal_workspace_bytes(op, shape, op == FAVOR_OP_CAUSAL ? chunk : 0, 0);
}

size_t favor_workspace_bytes_plan(int op, const favor_shape* shape, const favor_plan* plan) {
    if (check_plan(plan) != FAVOR_OK) return 0;
    return favor_internal_workspace_bytes(op, shape, plan && op == FAVOR_OP_CAUSAL ? plan->chunk : 0,
                                          plan ? plan->segments : 0);
}

favor_status favor_features(const favor_shape* shape, const void* x, const float* omega, float* phi,
                            float* log_scale, int stabilize, void* ws, size_t ws_bytes, void* stream) {
    Call c;
    c.op = FAVOR_OP_FEATURES; c.s = shape; c.q = x; c.omega = omega; c.phi = phi; c.log_scale = log_scale;
    c.stabilize = stabilize; c.ws = ws; c.ws_bytes = ws_bytes; c.stream = stream;
    return run(c);
}

favor_status favor_features_hadamard(const favor_shape* shape, const void* x, unsigned long long seed, float* phi,
                                     float* log_scale, int stabilize, void* stream) {
    const favor_shape* s = shape;
    favor_status st = check_shape(s, FAVOR_OP_FEATURES);
    if (st != FAVOR_OK) return st;
    if (s->L == 0) return FAVOR_OK;
    const size_t xbytes = (size_t)s->B * s->H * s->L * s->d * dtype_bytes(s->dtype);
    const size_t pbytes = (size_t)s->B * s->H * s->L * s->m * sizeof(float);
    const size_t lbytes = (size_t)s->B * s->H * s->L * sizeof(float);
    if (!x || !phi || !aligned(x, 16) || !aligned(phi, 16)) return FAVOR_ERR_INVALID_ARG;
    if (stabilize && (!log_scale || !aligned(log_scale, 4))) return FAVOR_ERR_INVALID_ARG;
    if (overlaps(phi, pbytes, x, xbytes)) return FAVOR_ERR_INVALID_ARG;
    if (stabilize && (overlaps(log_scale, lbytes, phi, pbytes) || overlaps(log_scale, lbytes, x, xbytes)))
        return FAVOR_ERR_INVALID_ARG;
    favor::HadamardFeaturesArgs a{};
    a.dtype_bytes = dtype_bytes(s->dtype);
    a.B = s->B; a.H = s->H; a.L = s->L; a.D = s->d; a.m = s->m;
    a.relu = s->feature == FAVOR_FEATURE_RELU;
    a.omega_per_head = s->omega_head_stride != 0 ? 1 : 0;
    a.seed = seed; a.x = x; a.phi = phi; a.log_scale = stabilize ? log_scale : nullptr;
    a.stabilize = stabilize ? 1 : 0;
    a.stream = static_cast<hipStream_t>(stream);
    return favor::launch_hadamard_features(a) == hipSuccess ? FAVOR_OK : FAVOR_ERR_HIP;
}

favor_status favor_bidir(const favor_shape* shape, const void* q, const void* k, const void* v, const float* omega,
                         void* out, void* ws, size_t ws_bytes, void* stream) {
    return run(attention(FAVOR_OP_BIDIR, shape, q, k, v, omega, out, ws, ws_bytes, stream));
}

favor_status favor_bidir_plan(const favor_shape* shape, const void* q, const void* k, const void* v,
                              const float* omega, void* out, const favor_plan* plan, void* ws, size_t ws_bytes,
                              void* stream) {
    const favor_status ps = check_plan(plan);
    if (ps != FAVOR_OK) return ps;
    Call c = attention(FAVOR_OP_BIDIR, shape, q, k, v, omega, out, ws, ws_bytes, stream);
    c.segments = plan ? plan->segments : 0;
    return run(c);
}

favor_status favor_causal(const favor_shape* shape, const void* q, const void* k, const void* v, const float* omega,
                          void* out, int chunk, void* ws, size_t ws_bytes, void* stream) {
    return favor_internal_causal(shape, q, k, v, omega, out, chunk, 0, ws, ws_bytes, stream);
}

favor_status favor_causal_plan(const favor_shape* shape, const void* q, const void* k, const void* v,
                               const float* omega, void* out, const favor_plan* plan, void* ws, size_t ws_bytes,
                               void* stream) {
    const favor_status ps = check_plan(plan);
    if (ps != FAVOR_OK) return ps;
    return favor_internal_causal(shape, q, k, v, omega, out, plan ? plan->chunk : 0, plan ? plan->segments : 0, ws,
                                 ws_bytes, stream);
}

favor_status favor_causal_state(const favor_shape* shape, const void* q, const void* k, const void* v,
                                const float* omega, void* out, int chunk, const float* state_in, float* state_out,
                                void* ws, size_t ws_bytes, void* stream) {
    Call c = attention(FAVOR_OP_CAUSAL, shape, q, k, v, omega, out, ws, ws_bytes, stream);
    c.chunk = resolve_chunk(shape, chunk);
    if (shape && c.chunk == 0) return FAVOR_ERR_UNSUPPORTED;
    if (shape && shape->feature != FAVOR_FEATURE_POSITIVE) return FAVOR_ERR_UNSUPPORTED;
    c.state_in = state_in;
    c.state_out = state_out;
    return run(c);
}

favor_status favor_bidir_profiled(const favor_shape* shape, const void* q, const void* k, const void* v,
                                  const float* omega, void* out, void* ws, size_t ws_bytes, void* stream,
                                  void* const* events, int n_events) {
    if (!events_ok(events, n_events)) return FAVOR_ERR_INVALID_ARG;
    Call c = attention(FAVOR_OP_BIDIR, shape, q, k, v, omega, out, ws, ws_bytes, stream);
    c.events = events;
    return run(c);
}

favor_status favor_causal_profiled(const favor_shape* shape, const void* q, const void* k, const void* v,
                                   const float* omega, void* out, int chunk, void* ws, size_t ws_bytes, void* stream,
                                   void* const* events, int n_events) {
    if (!events_ok(events, n_events)) return FAVOR_ERR_INVALID_ARG;
    Call c = attention(FAVOR_OP_CAUSAL, shape, q, k, v, omega, out, ws, ws_bytes, stream);
    c.chunk = resolve_chunk(shape, chunk);
    if (shape && c.chunk == 0) return FAVOR_ERR_UNSUPPORTED;
    c.events = events;
    return run(c);
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
