"""Pins for the CPU oracle: checks against what the pages and the mathematics
fix, independent of the oracle's own formulas.

Pages: [P1] "Performer — 랜덤 특징으로 어텐션을 다시 생각하기" (digest of
*Rethinking Attention with Performers*); [P2] Su Jianlin, "From Performer to
Linear Attention"; [P3] paperlayer.ai summary of arXiv:2009.14794v4.

Every statistical test uses fixed seeds, so it is deterministic; the margins
were set from the sampling error, not from the result.
"""

import math

import numpy as np
import pytest
import torch

import oracle.native as native
import oracle.reference as ref


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------------------
# Features: deterministic identities and hand-worked values
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("impl", ["numpy", "c"])
@pytest.mark.parametrize("m,d", [(1, 3), (7, 5), (32, 16), (40, 16)])
def test_feature_identity_opposite_vectors(impl, m, d):
    """phi(x).phi(-x) = exp(-|x|^2) for ANY omega: every term of the PRF
    estimator equals exp(-|x|^2)/m ([P1] key formulas; the |x+y| -> 0 limit of
    Lemma 2 in [P1] Theoretical bounds).  Catches a dropped or mis-signed
    |x|^2/2 term and a wrong 1/sqrt(m) factor."""
    rng = _rng(m * 100 + d)
    omega = rng.standard_normal((m, d)) * rng.uniform(0.2, 3.0, size=(m, 1))
    x = rng.standard_normal((9, d)) * 0.7
    f = ref.features if impl == "numpy" else native.features
    got = np.sum(f(x, omega) * f(-x, omega), axis=-1)
    want = np.exp(-np.sum(x * x, axis=-1))
    np.testing.assert_allclose(got, want, rtol=1e-13)


@pytest.mark.parametrize("impl", ["numpy", "c"])
def test_feature_hand_values(impl):
    """Hand-worked feature values.  omega rows (1,0,0) and (0,2,0), x=(1,0,0):
    omega_1.x = 1, omega_2.x = 0, |x|^2/2 = 1/2, m = 2, so
    phi = (e^{1/2}, e^{-1/2}) / sqrt(2).  A transposed omega gives different
    numbers (and a shape error for m != d)."""
    omega = np.array([[1.0, 0.0, 0.0], [0.0, 2.0, 0.0]])
    x = np.array([[1.0, 0.0, 0.0]])
    f = ref.features if impl == "numpy" else native.features
    got = f(x, omega)[0]
    want = np.array([math.exp(0.5), math.exp(-0.5)]) / math.sqrt(2.0)
    np.testing.assert_allclose(got, want, rtol=1e-14)
    # x = (0, 1, 1): omega_1.x = 0, omega_2.x = 2, |x|^2/2 = 1
    got2 = f(np.array([[0.0, 1.0, 1.0]]), omega)[0]
    np.testing.assert_allclose(got2, np.array([math.exp(-1.0), math.exp(1.0)]) / math.sqrt(2.0), rtol=1e-14)


def test_stabilized_features_scale():
    """The stabilised features differ from the plain ones by the reported
    per-row factor exp(s), and their largest entry is m^-1/2."""
    rng = _rng(5)
    omega = rng.standard_normal((24, 8))
    x = rng.standard_normal((11, 8)) * 2.0
    phi = ref.features(x, omega)
    phs, s = ref.features_stabilized(x, omega)
    np.testing.assert_allclose(phs * np.exp(s)[:, None], phi, rtol=1e-12)
    np.testing.assert_allclose(phs.max(axis=1), 1.0 / math.sqrt(24), rtol=1e-14)


# ---------------------------------------------------------------------------
# Estimator statistics: Theorem 1, Lemma 2, Theorem 2
# ---------------------------------------------------------------------------

def _pair(seed, d, sq):
    """x, y with |x+y|^2 = sq (kept <= 1 so the estimator's 4th moment is tame)."""
    rng = _rng(seed)
    x = rng.standard_normal(d)
    y = rng.standard_normal(d)
    f = math.sqrt(sq) / np.linalg.norm(x + y)
    return x * f, y * f


def _iid_errors(x, y, m, R, seed, chunk=20000):
    rng = _rng(seed)
    d = x.shape[0]
    out = []
    for c in range(0, R, chunk):
        n = min(chunk, R - c)
        om = rng.standard_normal((n, m, d))
        out.append(ref.sm_hat(x, y, om) - math.exp(float(x @ y)))
    return np.concatenate(out)


@pytest.mark.parametrize("sq,m", [(0.5, 1), (0.5, 8), (1.0, 8)])
def test_unbiased_and_lemma2_mse(sq, m):
    """i.i.d. PRF estimator: mean equals exp(x.y) (Theorem 1, [P1]
    Theoretical bounds) and the mean squared error equals the closed form
    (1/m) exp(|x+y|^2) SM^2 (1 - exp(-|x+y|^2)) (Lemma 2, [P1] Theoretical
    bounds and key formulas), each within 5 standard errors."""
    d = 16
    x, y = _pair(11 + m, d, sq)
    R = 100000
    e = _iid_errors(x, y, m, R, seed=1000 + m)
    se_mean = e.std() / math.sqrt(R)
    assert abs(e.mean()) < 5 * se_mean
    sq_err = e * e
    se_mse = sq_err.std() / math.sqrt(R)
    assert abs(sq_err.mean() - ref.lemma2_mse(x, y, m)) < 5 * se_mse


def test_lemma2_limit_zero():
    """Lemma 2 gives MSE 0 when x + y = 0; the estimator is then exact for
    every draw (see also the deterministic identity test)."""
    x = np.array([0.3, -0.2, 0.5, 0.1])
    assert ref.lemma2_mse(x, -x, 8) == 0.0
    om = _rng(3).standard_normal((50, 8, 4))
    np.testing.assert_allclose(ref.sm_hat(x, -x, om), math.exp(-float(x @ x)), rtol=1e-13)


@pytest.mark.parametrize("m", [16, 32])
def test_orf_variance_below_iid(m):
    """Orthogonal features: still unbiased, and their MSE is strictly below
    the i.i.d. one (Theorem 2: [P1] Theoretical bounds; [P3] section 3 and
    F.4.1).  d = 16: m = 16 is one full block, m = 32 two independent blocks."""
    d = 16
    x, y = _pair(77, d, 1.0)
    R = 40000
    rng = _rng(2024 + m)
    nb = (m + d - 1) // d
    om_orf = ref.orf_from_gaussians(rng.standard_normal((R, nb, d, d)), rng.standard_normal((R, nb, d, d)), m)
    e_orf = ref.sm_hat(x, y, om_orf) - math.exp(float(x @ y))
    e_iid = _iid_errors(x, y, m, R, seed=4048 + m)
    assert abs(e_orf.mean()) < 5 * e_orf.std() / math.sqrt(R)
    diff = e_orf ** 2 - e_iid ** 2
    assert diff.mean() < -3 * diff.std() / math.sqrt(R)


# ---------------------------------------------------------------------------
# Orthogonal projections and the counter-based generator
# ---------------------------------------------------------------------------

def test_philox_matches_numpy_library():
    """The oracle's Philox4x64-10 equals numpy's ``Philox`` bit generator (the
    same published generator; numpy advances the counter by one before each
    block, so counter c here is numpy's c - 1)."""
    for key in [(0, 0), (5, 7), (2 ** 64 - 1, 123456789)]:
        for ctr0 in [0, 1, 77, 2 ** 40]:
            bg = np.random.Philox(counter=ctr0, key=np.array(key, dtype=np.uint64))
            want = bg.random_raw(8)
            got = ref.philox4x64_10(np.array([[ctr0 + 1, 0, 0, 0], [ctr0 + 2, 0, 0, 0]], dtype=np.uint64), key)
            assert np.array_equal(got.reshape(-1), want)
    # higher counter words: numpy's 256-bit counter [c0, c1, c2, c3]
    bg = np.random.Philox(counter=[5, 9, 3, 1], key=[42, 0])
    want = bg.random_raw(4)
    got = ref.philox4x64_10(np.array([6, 9, 3, 1], dtype=np.uint64), (42, 0))
    assert np.array_equal(got, want)


def test_philox_normals_distribution():
    """Box-Muller normals from the generator are N(0, 1) (Kolmogorov-Smirnov
    against scipy's normal CDF, plus the first four moments)."""
    from scipy import stats
    z = ref.philox_normals(7, (3, 1, 0), 200001)
    assert z.shape == (200001,)
    assert stats.kstest(z, "norm").pvalue > 1e-3
    n = z.size
    assert abs(z.mean()) < 5 / math.sqrt(n)
    assert abs(z.var() - 1.0) < 5 * math.sqrt(2.0 / n)
    assert abs(np.mean(z ** 4) - 3.0) < 5 * math.sqrt(96.0 / n)


@pytest.mark.parametrize("m,d", [(16, 16), (40, 16), (256, 64), (10, 4)])
def test_orf_structure(m, d):
    """Rows inside each d x d block are mutually orthogonal; blocks are
    independent, so rows of different blocks are not ([P1] core components:
    Gram-Schmidt on the rows; block-wise when m > d).  Deterministic per seed."""
    om = ref.orf_omega(3, 2, m, d).astype(np.float64)
    assert om.shape == (2, m, d)
    assert np.array_equal(om, ref.orf_omega(3, 2, m, d).astype(np.float64))
    assert not np.array_equal(om[0], om[1])
    for h in range(2):
        for b0 in range(0, m, d):
            blk = om[h, b0:b0 + d]
            unit = blk / np.linalg.norm(blk, axis=1, keepdims=True)
            gram = unit @ unit.T
            off = gram - np.diag(np.diag(gram))
            assert np.abs(off).max() < 2e-6
    if m > d:
        unit = om[0] / np.linalg.norm(om[0], axis=1, keepdims=True)
        assert np.abs(unit[0] @ unit[d:].T).max() > 1e-3


def test_orf_marginals():
    """Each row is marginally N(0, I_d) ([P3] A.2: orthogonal features keep the
    marginals): squared row lengths are chi-square(d) (mean d, variance 2d) and
    entries have mean 0 and variance 1, over many seeds."""
    d, m = 8, 16
    rows = np.concatenate([ref.orf_omega(s, 1, m, d)[0] for s in range(600)]).astype(np.float64)
    n = rows.shape[0]
    sq = np.sum(rows ** 2, axis=1)
    assert abs(sq.mean() - d) < 5 * math.sqrt(2 * d / n)
    assert abs(sq.var() - 2 * d) < 0.15 * 2 * d
    ent = rows.reshape(-1)
    assert abs(ent.mean()) < 5 / math.sqrt(ent.size)
    assert abs(ent.var() - 1.0) < 0.05


def test_gram_schmidt_against_qr():
    """Row-wise Gram-Schmidt equals the (sign-fixed) Q factor of the QR
    decomposition of the transposed block (numpy's LAPACK routine)."""
    g = _rng(9).standard_normal((6, 6))
    u = ref.gram_schmidt_rows(g)
    q, r = np.linalg.qr(g.T)
    q = q * np.sign(np.diag(r))[None, :]
    np.testing.assert_allclose(u, q.T, atol=1e-12)


# ---------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------

def _qkv(seed, L, d, scale=0.5):
    rng = _rng(seed)
    return (rng.standard_normal((L, d)) * scale, rng.standard_normal((L, d)) * scale, rng.standard_normal((L, d)))


@pytest.mark.parametrize("L,d,m", [(1, 2, 1), (2, 4, 3), (3, 2, 8), (17, 4, 8), (64, 16, 32)])
def test_causal_equals_masked_brute_force(L, d, m):
    """Prefix-sum recurrence = explicit lower-triangular L x L evaluation with
    the same features ([P1] Methods and core components; [P3] section 2 and
    A.2); the bidirectional form = the unmasked L x L evaluation
    (associativity, [P1] atomic insights).  Both oracles."""
    q, k, v = _qkv(L * 1000 + d * 10 + m, L, d)
    om = _rng(m).standard_normal((m, d))
    bf_c = ref.brute_force(q, k, v, om, causal_mask=True)
    bf_b = ref.brute_force(q, k, v, om, causal_mask=False)
    Q, K, V = (a[None, None] for a in (q, k, v))
    np.testing.assert_allclose(ref.causal(Q, K, V, om)[0, 0], bf_c, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(native.causal(Q, K, V, om)[0, 0], bf_c, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ref.bidir(Q, K, V, om)[0, 0], bf_b, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(native.bidir(Q, K, V, om)[0, 0], bf_b, rtol=1e-12, atol=1e-12)


def test_attention_special_cases():
    """Exact special cases: the first causal row attends to one key only, so
    it is v_0; the last causal row is the last bidirectional row; constant V
    rows give out = V; jointly permuting (K, V) leaves the bidirectional output
    unchanged; permuting Q permutes the output rows."""
    L, d, m = 23, 8, 16
    q, k, v = _qkv(4, L, d)
    om = ref.orf_omega(1, 1, m, d)[0]
    Q, K, V = (a[None, None] for a in (q, k, v))
    c = ref.causal(Q, K, V, om)[0, 0]
    b = ref.bidir(Q, K, V, om)[0, 0]
    np.testing.assert_allclose(c[0], v[0], rtol=1e-13)
    np.testing.assert_allclose(c[-1], b[-1], rtol=1e-12)
    const = np.tile(np.arange(d, dtype=np.float64), (L, 1))
    np.testing.assert_allclose(ref.bidir(Q, K, const[None, None], om)[0, 0], const, rtol=1e-12)
    np.testing.assert_allclose(ref.causal(Q, K, const[None, None], om)[0, 0], const, rtol=1e-12)
    p = _rng(8).permutation(L)
    np.testing.assert_allclose(ref.bidir(Q, K[:, :, p], V[:, :, p], om)[0, 0], b, rtol=1e-12)
    np.testing.assert_allclose(ref.bidir(Q[:, :, p], K, V, om)[0, 0], b[p], rtol=1e-12)


def test_scale_invariance():
    """A per-row factor on query features and one common factor on all key
    features leave the normalised output unchanged ([P2] Simple Derivation);
    this is what licenses the GPU's stabilisers."""
    L, d, m = 31, 8, 24
    q, k, v = _qkv(12, L, d, scale=1.5)
    om = _rng(2).standard_normal((m, d))
    pq, _ = ref.features_stabilized(q, om)
    pk = ref.features(k, om) * math.exp(-7.5)
    a = np.tril(pq @ pk.T)
    out = (a @ v) / a.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(out, ref.brute_force(q, k, v, om, causal_mask=True), rtol=1e-12)


@pytest.mark.parametrize("causal_mask", [False, True])
def test_softmax_attention_matches_torch(causal_mask):
    """The exact-softmax target equals torch's scaled_dot_product_attention
    (fp64, CPU) with scale 1 (the kernel is exp(q.k), [P1] Methods)."""
    q, k, v = _qkv(21, 40, 8, scale=0.8)
    t = [torch.from_numpy(a)[None, None] for a in (q, k, v)]
    want = torch.nn.functional.scaled_dot_product_attention(*t, is_causal=causal_mask, scale=1.0)[0, 0].numpy()
    np.testing.assert_allclose(ref.softmax_attention(q, k, v, causal_mask), want, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("causal_mask", [False, True])
def test_monte_carlo_convergence_to_softmax(causal_mask):
    """FAVOR+ with orthogonal features converges to exact softmax attention as
    m grows (Theorem 1 and uniform convergence, [P1] Theoretical bounds; the
    L = 4096, d = 16 approximation study of [P3] section 3, here at L = 256).

    Lemma 2 puts the per-entry variance at exp(|q+k|^2)/m, so the Monte-Carlo
    rate m^-1/2 shows once m >> exp(|q+k|^2): with entries of q, k at 0.25
    (|q+k|^2 about 2) the median error over seeds must fall at a log-log slope
    near -1/2.  At the workloads' d^-1/4 scale (|q+k|^2 about 8) the error must
    still fall from m = 256 to m = 16384."""
    L, d = 256, 16
    ms = [64, 256, 1024, 4096, 16384]

    def medians(sigma, seeds):
        rng = _rng(0)
        q = rng.standard_normal((L, d)) * sigma
        k = rng.standard_normal((L, d)) * sigma
        v = rng.standard_normal((L, d))
        exact = ref.softmax_attention(q, k, v, causal_mask)
        med = []
        for m in ms:
            errs = []
            for s in range(seeds):
                g = _rng(100 * m + s).standard_normal((2, (m + d - 1) // d, d, d))
                approx = ref.brute_force(q, k, v, ref.orf_from_gaussians(g[0], g[1], m), causal_mask)
                errs.append(np.linalg.norm(approx - exact) / np.linalg.norm(exact))
            med.append(float(np.median(errs)))
        return med

    med = medians(0.25, 8)
    assert all(med[i + 1] < med[i] for i in range(len(ms) - 1))
    slope = (math.log(med[-1]) - math.log(med[1])) / (math.log(ms[-1]) - math.log(ms[1]))
    assert -0.65 < slope < -0.35
    assert med[-1] < 0.05
    med_w = medians(d ** -0.25, 4)
    assert med_w[-1] < 0.75 * med_w[1]


def test_rows_helpers_match_full():
    """Single-row evaluations used for long sequences equal the full oracle."""
    L, d, m = 50, 8, 16
    q, k, v = _qkv(3, L, d)
    om = ref.orf_omega(0, 1, m, d)[0]
    Q, K, V = (a[None, None] for a in (q, k, v))
    rows = np.array([0, 1, 17, 49])
    np.testing.assert_allclose(ref.causal_rows(q, k, v, om, rows), ref.causal(Q, K, V, om)[0, 0, rows], rtol=1e-12)
    np.testing.assert_allclose(ref.bidir_rows(q, k, v, om, rows), ref.bidir(Q, K, V, om)[0, 0, rows], rtol=1e-12)


def test_c_and_numpy_oracles_agree_multihead():
    """The plain-C and numpy oracles agree on multi-batch, multi-head inputs
    with per-head and shared omega."""
    rng = _rng(31)
    B, H, L, d, m = 2, 3, 45, 16, 40
    q, k, v = (rng.standard_normal((B, H, L, d)) * s for s in (0.5, 0.5, 1.0))
    for om in (ref.orf_omega(2, H, m, d), ref.orf_omega(2, 1, m, d)[0]):
        np.testing.assert_allclose(native.bidir(q, k, v, om), ref.bidir(q, k, v, om), rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(native.causal(q, k, v, om), ref.causal(q, k, v, om), rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------------------
# causal FAVOR+ with a carried prefix state
# ---------------------------------------------------------------------------

def _rand_qkv(rng, B, H, L, d, scale=0.5):
    q = rng.standard_normal((B, H, L, d)) * scale
    k = rng.standard_normal((B, H, L, d)) * scale
    v = rng.standard_normal((B, H, L, d))
    return q, k, v


@pytest.mark.parametrize("split", [1, 17, 40])
def test_causal_state_split_continues_the_recurrence(split):
    """Two pieces with the state handed over give the single-pass causal
    output (itself pinned to the masked L x L brute force)."""
    rng = np.random.default_rng(11)
    q, k, v = _rand_qkv(rng, 1, 2, 41, 8)
    om = ref.orf_omega(3, 2, 16, 8)
    want = ref.causal(q, k, v, om)
    out1, st = ref.causal_with_state(q[:, :, :split], k[:, :, :split], v[:, :, :split], om)
    out2, st2 = ref.causal_with_state(q[:, :, split:], k[:, :, split:], v[:, :, split:], om, st)
    got = np.concatenate([out1, out2], axis=2)
    assert np.max(np.abs(got - want)) <= 1e-12 * np.max(np.abs(want))
    _, st_full = ref.causal_with_state(q, k, v, om)
    for a, b in zip(st2, st_full):
        assert np.allclose(a, b, rtol=1e-12, atol=0)


def test_causal_state_empty_and_zero_match_causal():
    rng = np.random.default_rng(12)
    q, k, v = _rand_qkv(rng, 2, 1, 9, 4)
    om = ref.orf_omega(5, 1, 8, 4)[0]
    want = ref.causal(q, k, v, om)
    out_none, _ = ref.causal_with_state(q, k, v, om)
    out_zero, _ = ref.causal_with_state(q, k, v, om, (np.zeros((2, 1, 8, 4)), np.zeros((2, 1, 8))))
    assert np.max(np.abs(out_none - want)) <= 1e-12 * np.max(np.abs(want))
    assert np.max(np.abs(out_zero - want)) <= 1e-12 * np.max(np.abs(want))


def test_causal_state_final_state_gives_bidirectional():
    """The state after the last position, normalised for any query, is the
    bidirectional output for that query (all keys seen)."""
    rng = np.random.default_rng(13)
    q, k, v = _rand_qkv(rng, 1, 3, 23, 8)
    om = ref.orf_omega(7, 3, 24, 8)
    _, (G, z) = ref.causal_with_state(q, k, v, om)
    want = ref.bidir(q, k, v, om)
    for h in range(3):
        e_q = np.exp(q[0, h] @ om[h].T.astype(np.float64) - 0.5 * np.sum(q[0, h] ** 2, axis=-1, keepdims=True))
        got = (e_q @ G[0, h]) / (e_q @ z[0, h])[:, None]
        assert np.max(np.abs(got - want[0, h])) <= 1e-12 * np.max(np.abs(want[0, h]))


@pytest.mark.parametrize("m,d", [(4, 4), (24, 8), (7, 3)])
def test_causal_state_scale_convention(m, d):
    """The state carries the feature map without its m^-1/2 factor: after one
    key k, z = e(k), and e(-k) . z = m exp(-|k|^2) for any projection (the
    Lemma 2 limit |x + y| -> 0, [P1] Theoretical bounds)."""
    rng = np.random.default_rng(m * 100 + d)
    k = rng.standard_normal((1, 1, 1, d)) * 0.7
    v = rng.standard_normal((1, 1, 1, d))
    om = rng.standard_normal((m, d))
    _, (_, z) = ref.causal_with_state(k, k, v, om)
    phi_neg = ref.features(-k[0, 0, 0], om)  # m^-1/2 exp(-omega.k - |k|^2/2)
    lhs = float(phi_neg @ z[0, 0]) / math.sqrt(m)
    assert lhs == pytest.approx(math.exp(-float(np.sum(k ** 2))), rel=1e-12)


# ---------------------------------------------------------------------------
# generalised (ReLU) features
# ---------------------------------------------------------------------------

def test_relu_features_hand_values():
    om = np.array([[1.0, 0.0], [0.0, 1.0], [-1.0, 0.0], [1.0, 1.0]])
    x = np.array([2.0, -1.0])
    want = np.array([2.0, 0.0, 0.0, 1.0]) / 2.0  # max(omega x, 0) / sqrt(4)
    np.testing.assert_allclose(ref.features_relu(x, om), want, rtol=0, atol=1e-15)


@pytest.mark.parametrize("theta", [0.3, 1.2, 2.0, 2.9])
def test_relu_features_arc_cosine_kernel(theta):
    """With i.i.d. N(0, I) rows, E[phi(x) . phi(y)] for phi = m^-1/2 ReLU(omega . x)
    is the first-order arc-cosine kernel |x||y| (sin t + (pi - t) cos t) / (2 pi),
    t the angle between x and y (Cho and Saul, NIPS 2009): a closed form
    independent of the oracle's code."""
    d, m, R = 6, 16, 40000
    rng = np.random.default_rng(int(theta * 100))
    e1 = np.zeros(d); e1[0] = 1.0
    e2 = np.zeros(d); e2[1] = 1.0
    x = 1.3 * e1
    y = 0.8 * (np.cos(theta) * e1 + np.sin(theta) * e2)
    om = rng.standard_normal((R, m, d))
    est = np.sum(ref.features_relu(x, om) * ref.features_relu(y, om), axis=-1)
    want = np.linalg.norm(x) * np.linalg.norm(y) * (np.sin(theta) + (np.pi - theta) * np.cos(theta)) / (2 * np.pi)
    se = est.std(ddof=1) / math.sqrt(R)
    assert abs(est.mean() - want) <= 5 * se


@pytest.mark.filterwarnings("ignore:invalid value encountered in divide:RuntimeWarning")
@pytest.mark.parametrize("L,d,m", [(1, 2, 3), (17, 4, 8), (40, 8, 32)])
def test_relu_causal_and_bidir_equal_brute_force(L, d, m):
    """Recurrence and the explicit L x L form agree (associativity).  With few
    features a query can have none positive: both forms then give 0/0 (NaN)
    for that row, which the comparison treats as equal."""
    rng = np.random.default_rng(L + 10 * d + 100 * m)
    q, k, v = (rng.standard_normal((L, d)) for _ in range(3))
    om = rng.standard_normal((m, d))
    Q, K, V = (a[None, None] for a in (q, k, v))
    np.testing.assert_allclose(ref.causal(Q, K, V, om, kind="relu")[0, 0],
                               ref.brute_force(q, k, v, om, causal_mask=True, kind="relu"), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ref.bidir(Q, K, V, om, kind="relu")[0, 0],
                               ref.brute_force(q, k, v, om, causal_mask=False, kind="relu"), rtol=1e-12, atol=1e-12)
    rows = np.arange(L)
    np.testing.assert_allclose(ref.causal_rows(q, k, v, om, rows, kind="relu"),
                               ref.causal(Q, K, V, om, kind="relu")[0, 0], rtol=1e-12, atol=1e-12)


def test_relu_attention_positive_homogeneity():
    """ReLU features are positively homogeneous, so scaling queries (per row)
    or all keys by positive factors leaves the outputs unchanged; the
    softmax-kernel features are not (a check that no |x|^2 or exponential
    term is present)."""
    rng = np.random.default_rng(21)
    q, k, v = (rng.standard_normal((1, 1, 30, 4)) for _ in range(3))
    om = rng.standard_normal((16, 4))
    lam = rng.uniform(0.2, 5.0, size=(1, 1, 30, 1))
    for fn in (ref.bidir, ref.causal):
        base = fn(q, k, v, om, kind="relu")
        np.testing.assert_allclose(fn(q * lam, k * 3.0, v, om, kind="relu"), base, rtol=1e-12, atol=1e-12)
        assert not np.allclose(fn(q * lam, k * 3.0, v, om), fn(q, k, v, om), rtol=1e-6)


# ---------------------------------------------------------------------------
# structured (Hadamard) orthogonal projections
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("d", [1, 2, 16, 128])
def test_sylvester_hadamard_matches_library(d):
    import scipy.linalg
    np.testing.assert_array_equal(ref.sylvester_hadamard(d) * np.sqrt(d), scipy.linalg.hadamard(d))


def test_hadamard_block_structure_from_signs():
    """All-plus signs give sqrt(d) H^3 = sqrt(d) H (H is symmetric and
    orthogonal, so H^2 = I): a missing or extra Hadamard factor fails.  One
    flipped sign flips the matching column."""
    d = 16
    h = ref.sylvester_hadamard(d)
    ones = np.ones((3, d))
    np.testing.assert_allclose(ref.hadamard_block_from_signs(ones), np.sqrt(d) * h, atol=1e-12)
    s = ones.copy()
    s[2, 5] = -1.0
    want = np.sqrt(d) * h
    want[:, 5] *= -1.0
    np.testing.assert_allclose(ref.hadamard_block_from_signs(s), want, atol=1e-12)


@pytest.mark.parametrize("m,d", [(16, 16), (40, 16), (512, 128), (96, 32)])
def test_hadamard_omega_orthogonal_rows(m, d):
    om = ref.hadamard_omega(3, 2, m, d).astype(np.float64)
    for h in range(2):
        for b in range((m + d - 1) // d):
            blk = om[h, b * d: min(m, (b + 1) * d)]
            g = blk @ blk.T
            np.testing.assert_allclose(g, d * np.eye(len(blk)), atol=1e-4 * d)


def test_hadamard_signs_balanced_and_seeded():
    """Signs are fair coins across blocks and heads (binomial bounds), and
    different seeds give different projections."""
    s = np.stack([ref.hadamard_signs(7, b, h, 128) for b in range(8) for h in range(8)])
    n = s.size
    frac = (s > 0).mean()
    assert abs(frac - 0.5) <= 5 * 0.5 / np.sqrt(n)
    assert not np.array_equal(ref.hadamard_omega(1, 1, 32, 16), ref.hadamard_omega(2, 1, 32, 16))


# ---------------------------------------------------------------------------
# structured (Givens) orthogonal projections
# ---------------------------------------------------------------------------

def test_givens_block_special_cases():
    """No rotation gives the identity; in the plane (d = 2) any product of
    rotations is a rotation [[c, -s], [s, c]] with c^2 + s^2 = 1 and
    determinant +1 (a reflection or a transposed entry fails)."""
    i, j, t = ref.givens_rotations(4, 0, 0, 8, 0)
    np.testing.assert_array_equal(ref.givens_block(i, j, t, 8), np.eye(8))
    for count in (1, 2, 7):
        q = ref.givens_block(*ref.givens_rotations(5, 1, 2, 2, count), 2)
        assert q[0, 0] == pytest.approx(q[1, 1], abs=1e-15)
        assert q[0, 1] == pytest.approx(-q[1, 0], abs=1e-15)
        assert np.linalg.det(q) == pytest.approx(1.0, abs=1e-14)


@pytest.mark.parametrize("d", [5, 16, 64])
def test_givens_block_is_rotation(d):
    """Any count of plane rotations gives an orthogonal matrix of
    determinant +1 (d need not be a power of two)."""
    q = ref.givens_block(*ref.givens_rotations(9, 0, 1, d, ref.givens_default_rotations(d)), d)
    np.testing.assert_allclose(q @ q.T, np.eye(d), atol=1e-13)
    assert np.linalg.det(q) == pytest.approx(1.0, abs=1e-10)


def test_givens_draws_uniform():
    """Coordinate pairs are uniform over the 12 ordered pairs of d = 4 with
    i != j (chi-square at 11 degrees of freedom, p > 1e-4) and angles are
    uniform on (0, 2 pi] (Kolmogorov-Smirnov, p > 1e-4)."""
    from scipy import stats
    i, j, t = ref.givens_rotations(1, 0, 0, 4, 24000)
    assert np.all(i != j) and i.min() >= 0 and j.max() <= 3
    counts = np.bincount(i * 4 + j, minlength=16)[[a * 4 + b for a in range(4) for b in range(4) if a != b]]
    assert stats.chisquare(counts).pvalue > 1e-4
    assert np.all((t > 0) & (t <= 2 * np.pi))
    assert stats.kstest(t / (2 * np.pi), "uniform").pvalue > 1e-4


def test_givens_mixing_toward_uniform_rotation():
    """A row of a uniformly random rotation has E[u_c^2] = 1/d in every
    coordinate.  Over 300 seeds at d = 16 the default 64 rotations bring
    every coordinate's mean within 5 standard errors of 1/d, while 2 or 16
    rotations leave the row near its starting axis (the statistic has the
    power to tell), and the starting coordinate's excess shrinks as the
    count grows."""
    d = 16

    def stats_for(count):
        c = np.array([ref.givens_block(*ref.givens_rotations(s, 0, 0, d, count), d)[0] ** 2 for s in range(300)])
        z = (c.mean(0) - 1.0 / d) / (c.std(0, ddof=1) / np.sqrt(len(c)))
        return float(np.abs(z).max()), float(c.mean(0)[0] - 1.0 / d)

    z2, e2 = stats_for(2)
    z16, e16 = stats_for(16)
    z64, e64 = stats_for(ref.givens_default_rotations(d))
    assert ref.givens_default_rotations(d) == 64
    assert z64 <= 5.0
    assert z2 > 20.0 and z16 > 8.0
    assert e2 > e16 > e64 > -0.01


def test_givens_omega_rows_orthogonal_with_chi_lengths():
    """Rows of a block are orthogonal, and row i of block b has the length
    the Gram-Schmidt construction gives the same row (both take chi(d)
    lengths from Philox stream (b, h, 1)); the last block is cut to m."""
    seed, H, m, d = 3, 2, 40, 16
    om = ref.givens_omega(seed, H, m, d).astype(np.float64)
    orf = ref.orf_omega(seed, H, m, d).astype(np.float64)
    np.testing.assert_allclose(np.linalg.norm(om, axis=-1), np.linalg.norm(orf, axis=-1), rtol=1e-6)
    for h in range(H):
        for b in range((m + d - 1) // d):
            blk = om[h, b * d: min(m, (b + 1) * d)]
            g = blk @ blk.T
            off = g - np.diag(np.diag(g))
            assert np.abs(off).max() <= 1e-5 * np.diag(g).max()
    assert not np.array_equal(ref.givens_omega(1, 1, 32, 16), ref.givens_omega(2, 1, 32, 16))


def test_givens_features_nearly_unbiased():
    """Theorem 1 with a Givens projection: over 3000 seeds (m = d = 16,
    small |x|, |y|) the mean estimate is within 5 standard errors of
    exp(x.y); the pages state a small bias that vanishes as d grows, and
    here it is below the Monte-Carlo resolution."""
    rng = _rng(77)
    d = 16
    x = rng.normal(size=d) * 0.25
    y = rng.normal(size=d) * 0.25
    sm = np.exp(x @ y)
    e = np.array([ref.sm_hat(x, y, ref.givens_omega(s, 1, d, d)[0].astype(np.float64)) for s in range(3000)])
    se = e.std(ddof=1) / np.sqrt(len(e))
    assert abs(e.mean() - sm) <= 5 * se


# ---------------------------------------------------------------------------
# trigonometric features (the estimator the approximation study compares with)
# ---------------------------------------------------------------------------

def test_trig_features_self_identity():
    """phi_trig(x) . phi_trig(x) = exp(|x|^2) for ANY projection (sin^2 + cos^2
    = 1): pins the exp(|x|^2 / 2) scale and the m^-1/2 factor."""
    rng = _rng(31)
    for m, d in ((1, 3), (7, 16), (64, 16)):
        om = rng.standard_normal((m, d)) * 3.0
        x = rng.standard_normal(d) * 0.7
        phi = ref.features_trig(x, om)
        assert phi.shape == (2 * m,)
        np.testing.assert_allclose(phi @ phi, np.exp(x @ x), rtol=1e-13)
        np.testing.assert_allclose(ref.sm_hat_trig(x, x, om), np.exp(x @ x), rtol=1e-13)
        y = rng.standard_normal(d) * 0.7
        np.testing.assert_allclose(ref.features_trig(x, om) @ ref.features_trig(y, om), ref.sm_hat_trig(x, y, om),
                                   rtol=1e-12)


@pytest.mark.parametrize("z2", [0.3, 1.0, 2.5])
def test_trig_estimator_unbiased_with_closed_form_mse(z2):
    """E[phi_trig(x).phi_trig(y)] = exp(x.y) over i.i.d. Gaussian rows (within
    5 standard errors), and its empirical MSE matches
    exp(|x|^2+|y|^2)(1-exp(-|x-y|^2))^2/(2m) within 5 standard errors.  A
    sign slip (x + y in the cosine) or a lost scale fails one of them."""
    rng = _rng(int(z2 * 100))
    d, m, R = 16, 8, 200_000
    x = rng.standard_normal(d)
    x *= 0.5 / np.linalg.norm(x)
    u = rng.standard_normal(d)
    u *= math.sqrt(z2) / np.linalg.norm(u)
    y = x - u  # |x - y|^2 = z2
    est = np.empty(R)
    for c in range(0, R, 20000):
        om = rng.standard_normal((20000, m, d))
        est[c:c + 20000] = ref.sm_hat_trig(x, y, om)
    target = math.exp(float(x @ y))
    mse_cf = ref.trig_mse(x, y, m)
    assert abs(est.mean() - target) <= 5 * math.sqrt(mse_cf / R)
    sq = (est - target) ** 2
    assert abs(sq.mean() - mse_cf) <= 5 * sq.std() / math.sqrt(R)


def test_trig_attention_is_brute_force_of_its_features():
    """Attention through trigonometric features by associativity equals the
    explicit L x L form with the same features (normalisers can change sign,
    so only the algebra is pinned here)."""
    q, k, v = _qkv(41, 30, 4, scale=0.3)
    om = _rng(42).standard_normal((12, 4))
    want = ref.brute_force(q, k, v, om, causal_mask=False, kind="trig")
    got = ref.bidir(q[None, None], k[None, None], v[None, None], om, kind="trig")[0, 0]
    np.testing.assert_allclose(got, want, rtol=1e-9)


def test_iid_omega_is_standard_normal():
    om = ref.iid_omega(3, 4096, 16).astype(np.float64)
    assert om.shape == (4096, 16)
    assert abs(om.mean()) < 5 / math.sqrt(om.size)
    assert abs(om.var() - 1.0) < 5 * math.sqrt(2.0 / om.size)
    assert not np.array_equal(ref.iid_omega(3, 8, 16), ref.iid_omega(4, 8, 16))
