/*
 * favor.h — C ABI of the MI355X (gfx950) FAVOR+ attention library.
 *
 * FAVOR+ ("Fast Attention Via positive Orthogonal Random features") replaces
 * the softmax kernel exp(q.k) by an inner product of positive random features
 *     phi(x)_i = m^-1/2 exp(omega_i . x - |x|^2 / 2),   i = 1..m,
 * over a projection Omega in R^{m x d} with orthogonal Gaussian rows, and
 * evaluates attention by associativity, never forming the L x L matrix.
 * Pages: "Performer — 랜덤 특징으로 어텐션을 다시 생각하기" (digest of
 * *Rethinking Attention with Performers*, irregular6612.github.io), sections
 * "Methods (FAVOR+)", core components and key formulas; Su Jianlin, "From
 * Performer to Linear Attention", Simple Derivation; paperlayer.ai summary of
 * arXiv:2009.14794v4, sections 2, A.2 and B.3.
 *
 * Conventions for every entry point below:
 *   - Tensor arguments are DEVICE pointers owned by the caller, contiguous,
 *     row-major.  q, k, v, out (and x) are [B, H, L, d]; omega is fp32 and is
 *     either [m, d] (omega_head_stride = 0: one projection for all heads) or
 *     [H, m, d] (omega_head_stride = m*d: one per head); every batch element
 *     uses the same projection, and queries and keys of a head share it.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream);
 *     nothing synchronises, nothing allocates device memory, no global
 *     mutable state is kept: calls are re-entrant and thread-safe.
 *   - The return value reports argument validation (done before any HIP call)
 *     and launch errors.  Device faults surface at the caller's next
 *     synchronisation.  No C++ exception crosses this interface.
 *   - Accumulation is fp32.  bf16 inputs give bf16 outputs.  There is no
 *     temperature: the library computes exp(q.k) exactly as defined; callers
 *     wanting softmax(q.k / sqrt(d)) pre-scale q and k by d^-1/4.
 *   - Feature map: shape->feature selects the positive random features of
 *     the softmax kernel (FAVOR+) or the generalised ReLU features
 *     (Performer-ReLU; "Performer" digest and paperlayer.ai summary, section
 *     2, name it without printing the map: phi_i = m^-1/2 max(omega_i . x, 0)
 *     is the reading taken).  ReLU features need no stabiliser.  A query or
 *     key prefix whose ReLU features are all zero has a zero normaliser: its
 *     output is not finite, as in the exact formula.
 *   - Supported: d in {16, 32, 64, 128}; fp32 only with d <= 64;
 *     bidirectional and features: m a multiple of 32 up to 256, or a
 *     multiple of 64 up to 512; causal: m in {32, 64, 128, 256, 512}, except
 *     fp32 with d = 64 and m = 512 (its scan's tiles exceed the LDS);
 *     B, H >= 1; B*H <= 65535 (one grid row per batch and head); L >= 0
 *     (L = 0 is a no-op); B*H*L*d < 2^31.
 */
#ifndef FAVOR_H_
#define FAVOR_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FAVOR_F32 = 0, FAVOR_BF16 = 1 } favor_dtype;

typedef enum {
    FAVOR_OK = 0,
    FAVOR_ERR_INVALID_ARG = 1, /* null pointer, bad dimension, out aliasing an input  */
    FAVOR_ERR_UNSUPPORTED = 2, /* d, m or dtype outside the supported set             */
    FAVOR_ERR_WORKSPACE = 3,   /* workspace pointer null or smaller than required     */
    FAVOR_ERR_HIP = 4          /* a HIP launch failed (hipGetLastError after launch)   */
} favor_status;

typedef enum {
    FAVOR_FEATURE_POSITIVE = 0, /* phi_i = m^-1/2 exp(omega_i . x - |x|^2/2): softmax kernel      */
    FAVOR_FEATURE_RELU = 1      /* phi_i = m^-1/2 max(omega_i . x, 0): generalised ReLU kernel */
} favor_feature;

typedef struct {
    int B, H, L, d, m;           /* q, k, v, out: [B, H, L, d]; m random features        */
    favor_dtype dtype;           /* element type of q, k, v, out, x                      */
    long long omega_head_stride; /* 0: omega is [m, d]; m*d: omega is [H, m, d]          */
    int feature;                 /* a favor_feature value; 0, the zero default: positive */
} favor_shape;

/* Operation codes for favor_workspace_bytes. */
#define FAVOR_OP_FEATURES 0
#define FAVOR_OP_BIDIR 1
#define FAVOR_OP_CAUSAL 2

/*
 * Bytes of device workspace the given operation needs for this shape.
 * `chunk` is the causal chunk length (0 = default) and is ignored otherwise.
 * Returns 0 for an invalid or unsupported shape (the operation itself reports
 * which).  The size depends only on the shape, never on the device.
 */
size_t favor_workspace_bytes(int op, const favor_shape *shape, int chunk);

/*
 * Positive random features of x ([B, H, L, d]) into phi ([B, H, L, m], fp32):
 *     phi_i = m^-1/2 exp(omega_i . x - |x|^2/2 - s)
 * ("Performer" digest, core components: the positive random feature map).
 * stabilize = 0: s = 0 and log_scale may be NULL.
 * stabilize = 1: s = max_i(omega_i . x - |x|^2/2) per row, written to
 *                log_scale ([B, H, L] fp32, natural-log units), so that the
 *                unstabilised features are phi * exp(log_scale).
 * ReLU features (shape->feature = FAVOR_FEATURE_RELU):
 *     phi_i = m^-1/2 max(omega_i . x, 0); with stabilize, log_scale is 0.
 * The projection uses omega rounded to the input dtype (bf16 inputs: bf16
 * omega * log2(e), fp32 accumulation).  ws/ws_bytes: device workspace of at
 * least favor_workspace_bytes(FAVOR_OP_FEATURES, shape, 0) bytes, 256-byte
 * aligned.  phi must not overlap x or omega; log_scale must not overlap
 * phi, x or omega; ws must not overlap x, omega, phi or log_scale
 * (FAVOR_ERR_INVALID_ARG).
 */
favor_status favor_features(const favor_shape *shape, const void *x, const float *omega, float *phi,
                            float *log_scale, int stabilize, void *ws, size_t ws_bytes, void *stream);

/*
 * favor_features over the structured Hadamard projection that
 * favor_hadamard_omega(seed, n, m, d) would generate (n = H when
 * shape->omega_head_stride != 0, one set of blocks per head; else the blocks
 * of head 0 for every head), without materialising it: the blocks
 * sqrt(d) H S1 H S2 H S3 are applied to x as three fast Walsh-Hadamard
 * transforms with sign flips, d log2 d additions each instead of a dense
 * d x d product (paperlayer.ai summary, B.3: structured projections build
 * the features in O(L m log d)).  The signs are drawn from the seed inside
 * the call; no workspace, and the projection is exact in fp32 (no rounding
 * of omega to the input dtype).  Same shapes, outputs, stabiliser and
 * overlap rules as favor_features (x, phi, log_scale).
 */
favor_status favor_features_hadamard(const favor_shape *shape, const void *x, unsigned long long seed, float *phi,
                                     float *log_scale, int stabilize, void *stream);

/*
 * Bidirectional FAVOR+ ("Performer" digest, key formulas and method
 * flowchart):
 *     out_t = phi(q_t)^T (sum_s phi(k_s) v_s^T) / phi(q_t)^T (sum_s phi(k_s)).
 * ws/ws_bytes: device workspace of at least
 * favor_workspace_bytes(FAVOR_OP_BIDIR, shape, 0) bytes, 256-byte aligned;
 * its contents need not be initialised and are garbage afterwards.
 * out must not overlap q, k, v, omega or ws, and ws must not overlap q, k,
 * v or omega (FAVOR_ERR_INVALID_ARG): the kernels write the workspace while
 * later kernels of the same call still read the inputs.
 */
favor_status favor_bidir(const favor_shape *shape, const void *q, const void *k, const void *v,
                         const float *omega, void *out, void *ws, size_t ws_bytes, void *stream);

/*
 * Causal (unidirectional) FAVOR+ by prefix sums ("Performer" digest, Methods:
 * G_t = sum_{s<=t} phi(k_s) v_s^T; paperlayer.ai summary, A.2 unidirectional
 * attention):
 *     out_t = phi(q_t)^T G_t / phi(q_t)^T (sum_{s<=t} phi(k_s)),
 * with an inclusive mask (position t attends to keys 0..t).
 * chunk: tokens per step of the chunked scan (any length gives the same
 * result up to rounding).  Accepted: 0 (the shape's default), 32, and 64
 * where the shape has a 64-token scan: bf16 with d = 64 and m in
 * {64, 128, 256} default to 64 (tile scan) and also accept 32
 * (feature-split scan); every other shape accepts 32, its default.  Other
 * values: FAVOR_ERR_UNSUPPORTED.
 * Workspace as for favor_bidir with FAVOR_OP_CAUSAL.
 */
favor_status favor_causal(const favor_shape *shape, const void *q, const void *k, const void *v,
                          const float *omega, void *out, int chunk, void *ws, size_t ws_bytes,
                          void *stream);

/*
 * Launch-plan overrides, for tuning and for testing that the result does not
 * depend on how the sequence is split ("paperlayer.ai" summary, A.2: the
 * prefix sums run in O(log L) parallel time, so any split of the scan into
 * segments gives the same result up to rounding).
 *   chunk:    causal chunk length as for favor_causal (0 = default);
 *             ignored by bidirectional attention.
 *   segments: token segments per head, 0 = automatic (sized so that one
 *             pass fills 256 compute units, with segments of at least 256
 *             tokens for bidirectional m >= 128 and 64 tokens for causal;
 *             one per head for many heads of short bidirectional sequences
 *             (from 128 heads up to 512 tokens, from 64 up to 384) and,
 *             with m = 32, up to 512 tokens, or 4096 from 128 heads: the
 *             whole call then runs as one kernel), else 1..256.  A bidirectional plan with
 *             one segment runs as one kernel wherever that kernel's operands
 *             fit on a compute unit.  Segments are whole 32- or 64-token
 *             steps, so fewer may be used than requested (at most
 *             ceil(L / 32)).  Negative or > 256: FAVOR_ERR_INVALID_ARG.
 * A NULL plan means both defaults.  The workspace size depends on the plan:
 * favor_workspace_bytes_plan returns it (0 for an invalid shape or plan).
 * The other arguments are those of favor_bidir / favor_causal.
 */
typedef struct {
    int chunk;
    int segments;
} favor_plan;

size_t favor_workspace_bytes_plan(int op, const favor_shape *shape, const favor_plan *plan);
favor_status favor_bidir_plan(const favor_shape *shape, const void *q, const void *k, const void *v,
                              const float *omega, void *out, const favor_plan *plan, void *ws, size_t ws_bytes,
                              void *stream);
favor_status favor_causal_plan(const favor_shape *shape, const void *q, const void *k, const void *v,
                               const float *omega, void *out, const favor_plan *plan, void *ws, size_t ws_bytes,
                               void *stream);

/*
 * Causal FAVOR+ continuing from a carried prefix state, and the state after
 * the last position: for streaming and autoregressive use, where a sequence
 * arrives in pieces ("Performer" digest, Methods: G_t is a running sum over
 * s <= t; Su Jianlin, Simple Derivation: the recurrent form).  A sequence
 * split into pieces, each call taking the previous call's state_out as its
 * state_in, gives the outputs of one call over the whole sequence (up to
 * rounding).
 * State format, per head (b, h) at offset (b H + h) (m (d + 1) + 1) floats,
 * fp32, device memory, caller-owned:
 *     S[m][d] row-major, then z[m], then one shift s (natural-log units),
 * meaning G = S e^s and zsum = z e^s with
 *     G = sum over the keys so far of e(k) v^T,  zsum = sum of e(k),
 *     e(k)_i = exp(omega_i . k - |k|^2/2)   (the feature map without m^-1/2).
 * state_in: NULL = no keys seen yet.  A state with S = z = 0 should be passed
 * as NULL: its shift still takes part in the key stabiliser.
 * state_out: NULL = not written; otherwise it receives the state including
 * this call's keys, with one shift per head.
 * Calls of at most 32 tokens per head (decoding) run as one kernel that
 * reads state_in and writes state_out itself, for every shape with a
 * feature-split scan (all but bf16 with d = 128 and m >= 256); the
 * workspace is still required and validated.  state_out must not overlap
 * state_in, q, k, v, out, omega or ws, and state_in must not overlap out or
 * ws (FAVOR_ERR_INVALID_ARG).  Both must be
 * 4-byte aligned.  L = 0 writes nothing.  Positive features only
 * (FAVOR_FEATURE_RELU: FAVOR_ERR_UNSUPPORTED).  Other arguments as for
 * favor_causal.
 */
favor_status favor_causal_state(const favor_shape *shape, const void *q, const void *k, const void *v,
                                const float *omega, void *out, int chunk, const float *state_in,
                                float *state_out, void *ws, size_t ws_bytes, void *stream);

/*
 * Causal FAVOR+ that allocates nothing, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, kernels and results as
 * favor_causal, without ws/ws_bytes: the workspace is a static device array
 * of FAVOR_NOALLOC_SCRATCH_BYTES (96 MiB) inside the library, one per GPU,
 * held from the first call on that GPU until the process ends.
 *   - A shape whose workspace (favor_workspace_bytes(FAVOR_OP_CAUSAL, shape,
 *     chunk)) exceeds FAVOR_NOALLOC_SCRATCH_BYTES returns
 *     FAVOR_ERR_WORKSPACE before any launch; invalid arguments are reported
 *     as by favor_causal.
 *   - The array belongs to the current device (hipGetDevice); `stream` must
 *     belong to it too.  The first call on a device resolves the array's
 *     address (hipGetSymbolAddress); make that call outside graph capture.
 *   - Every call on one GPU shares its array: calls that overlap in time on
 *     one GPU (different streams, or different host threads without
 *     ordering) race and give wrong results.  Calls ordered on one stream
 *     are safe; nothing in the array needs clearing between calls.
 *   - No hipMalloc, hipFree or other allocation happens in the call.
 */
#define FAVOR_NOALLOC_SCRATCH_BYTES ((size_t)96 << 20)
favor_status favor_causal_noalloc(const favor_shape *shape, const void *q, const void *k, const void *v,
                                  const float *omega, void *out, int chunk, void *stream);

/*
 * Stage-timed variants.  Identical results to favor_bidir / favor_causal;
 * additionally, events[i] (caller-created hipEvent_t handles) is recorded on
 * `stream` before stage i and events[FAVOR_N_STAGES] after the last stage.
 * Stages: 0 segment partials of phi(K)^T [V | 1], 1 merge over segments
 * (bidir) / exclusive scan (causal), both also packing the projection,
 * 2 output pass (bidir) / chunked scan (causal).  n_events must be
 * >= FAVOR_N_STAGES + 1, else FAVOR_ERR_INVALID_ARG.  For callers measuring
 * each kernel.
 */
#define FAVOR_N_STAGES 3
favor_status favor_bidir_profiled(const favor_shape *shape, const void *q, const void *k, const void *v,
                                  const float *omega, void *out, void *ws, size_t ws_bytes, void *stream,
                                  void *const *events, int n_events);
favor_status favor_causal_profiled(const favor_shape *shape, const void *q, const void *k, const void *v,
                                   const float *omega, void *out, int chunk, void *ws, size_t ws_bytes,
                                   void *stream, void *const *events, int n_events);

/*
 * Seeded orthogonal random projection, written to HOST memory
 * omega_host[n_heads, m, d] (fp32), computed on the CPU.  For each head,
 * ceil(m/d) independent blocks: a d x d Gaussian whose rows are
 * orthonormalised by Gram-Schmidt in row order, each row then scaled to the
 * length of an independent N(0, I_d) vector, so rows are marginally
 * N(0, I_d) ("Performer" digest, core components: Gram-Schmidt on the rows,
 * block-wise when m > d; paperlayer.ai summary, A.2: marginals preserved).
 * Gaussians come from Philox4x64-10 (Salmon et al., SC'11) with key
 * (seed, 0): block b of head h reads counter (j, b, h, 0) for the matrix and
 * (j, b, h, 1) for the lengths, four normals per counter via Box-Muller on
 * 53-bit uniforms u = ((w >> 11) + 1) 2^-53.
 * Returns FAVOR_ERR_INVALID_ARG for a null pointer or non-positive size.
 */
favor_status favor_orf_omega(unsigned long long seed, int n_heads, int m, int d, float *omega_host);

/*
 * Structured (Hadamard) orthogonal projection generated on the DEVICE:
 * omega[n_heads, m, d] (fp32, device memory, 16-byte aligned), enqueued on
 * `stream`.  Hadamard ORFs need only O(m) random numbers and carry a small
 * bias that vanishes as d grows (paperlayer.ai summary, A.2 ORF bullet and
 * B.3 trade-offs; the pages print no construction).  Each d x d block is
 * sqrt(d) H S1 H S2 H S3, H the normalised Sylvester-Hadamard matrix
 * (H[i][j] = (-1)^popcount(i & j) / sqrt(d)) and S_t diagonal +-1; rows are
 * orthogonal with norm sqrt(d); ceil(m/d) independent blocks per head, the
 * last cut to the rows needed.  Diagonal t of block b of head h takes its
 * signs from Philox4x64-10 with key (seed, 0) and counter (0, b, h, 2 + t):
 * entry j is -1 when bit j % 64 of output word j / 64 is set.  Values are
 * exact in fp32.  The result is an ordinary projection for the attention
 * entry points.  d in {16, 32, 64, 128} (else FAVOR_ERR_UNSUPPORTED); null or
 * misaligned omega, n_heads < 1 or m < 1: FAVOR_ERR_INVALID_ARG.
 */
favor_status favor_hadamard_omega(unsigned long long seed, int n_heads, int m, int d, float *omega,
                                  void *stream);

/*
 * Structured (Givens) orthogonal projection generated on the DEVICE:
 * omega[n_heads, m, d] (fp32, device memory, 16-byte aligned), enqueued on
 * `stream`.  Givens ORFs keep O(m log d) random numbers and carry a small
 * bias that vanishes as d grows (paperlayer.ai summary, A.2 ORF bullet and
 * B.3 trade-offs; the pages print no construction).  Each d x d block is the
 * product G_{K-1} ... G_1 G_0 of K plane rotations applied to the identity
 * (K = rotations, or d * ceil(log2 d) when rotations = 0); G_k acts on rows
 * (i_k, j_k) as [[cos t_k, -sin t_k], [sin t_k, cos t_k]].  Row r of a block
 * is then scaled to the chi(d) length favor_orf_omega gives row r of the same
 * block.  Rotation k of block b of head h: Philox4x64-10 with key (seed, 0)
 * and counter (k, b, h, 5), output words w0..w2:
 * i = floor(d (w0 >> 32) / 2^32), j' = floor((d - 1) (w1 >> 32) / 2^32),
 * j = j' + (j' >= i), t = 2 pi ((w2 >> 11) + 1) 2^-53.  Computed in fp64 and
 * rounded to fp32 once.  ceil(m/d) blocks per head, the last cut to the rows
 * needed.  2 <= d <= 128, n_heads <= 65535 and n_heads * m * d < 2^31 (else
 * FAVOR_ERR_UNSUPPORTED); null or misaligned omega, n_heads < 1, m < 1 or
 * rotations outside [0, 2^24]: FAVOR_ERR_INVALID_ARG.
 */
favor_status favor_givens_omega(unsigned long long seed, int n_heads, int m, int d, int rotations, float *omega,
                                void *stream);

/* Static, human-readable name of a status code. */
const char *favor_status_string(favor_status status);

#ifdef __cplusplus
}
#endif

#endif /* FAVOR_H_ */
