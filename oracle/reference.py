"""Plain fp64 CPU oracle for FAVOR+ attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import or run anything under ``oracle/``.
The GPU library never calls it and shares no code with it.

Pages this follows (cited by title and section):

* [P1] "Performer — 랜덤 특징으로 어텐션을 다시 생각하기" (digest of
  *Rethinking Attention with Performers*, irregular6612.github.io):
  sections "Methods (FAVOR+)", "Theoretical bounds", "핵심 구성요소" (core
  components), "핵심 수식" (key formulas), "원자적 인사이트" (atomic
  insights).
* [P2] Su Jianlin, "The Road to Transformer Upgrade 3: From Performer to
  Linear Attention" (kexue.fm): sections "Simple Derivation" and
  "Concentrating Attention".
* [P3] paperlayer.ai summary of *Rethinking Attention with Performers*
  (arXiv:2009.14794v4): sections "2 FAVOR+ mechanism & positive orthogonal
  random features", "A.2 Training hyperparameters" (unidirectional
  attention, ORF bullets), "B.3 Time and space complexity".

What the oracle computes is the FAVOR+ algorithm itself for a given
projection Omega (an unbiased randomised estimate of softmax attention), not
softmax attention; exact softmax attention is a separate function used only
by the Monte-Carlo checks.

Readings where the pages leave a step open:

* The 1/sqrt(m) factor belongs to the feature map ([P1] core components;
  [P2] Simple Derivation); it cancels in normalised attention.
* The causal mask is inclusive: the prefix state at position t sums keys
  s <= t ([P1] Methods, G_t).
* No epsilon is added to the normaliser; positive features keep it > 0.
* No stabiliser: fp64 ``exp`` has the range for every workload used here.
* Omega is [m, d] shared by all heads or [H, m, d] per head, identical for
  every batch element; queries and keys of a head use the same Omega
  ([P1] method-framework flowchart, "shared omega").
* Orthogonal blocks: each block is a fresh d x d Gaussian whose rows are
  orthogonalised by Gram-Schmidt in row order; each unit row is then given
  the length of an independent N(0, I_d) vector (chi(d)), so every row is
  marginally N(0, I_d); ceil(m/d) independent blocks are stacked and the last
  is cut to the rows needed ([P1] core components and atomic insights:
  block-wise orthogonalisation when r > d; [P3] A.2: marginals preserved).
* Structured orthogonal blocks: the pages name Hadamard and Givens ORFs as
  cheaper variants with a small bias that vanishes as d grows ([P3] A.2 ORF
  bullet, B.3) and print neither construction.  Hadamard: sqrt(d) H S1 H S2
  H S3 (hadamard_omega).  Givens: a product of d ceil(log2 d) random plane
  rotations of the identity, rows scaled to chi(d) lengths (givens_omega).
* Generalised (ReLU) features: the pages name Performer-ReLU as FAVOR+ with
  another kernel function ([P1] Digest; [P3] section 2) without printing its
  map; the reading taken is phi(x)_i = m^-1/2 max(omega_i . x, 0), the same
  projection with no |x|^2 term and no exponential.
* Random numbers: the counter-based generator Philox4x64-10 (Salmon, Moraes,
  Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC'11) turned
  into uniforms with 53-bit mantissas and into normals with the Box-Muller
  transform.

Parity unpinned: none of the functions here; each one is checked in
``tests/test_oracle_*.py`` against identities, closed forms, brute force or
library routines.
"""

from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# Counter-based random numbers (Philox4x64-10, published definition)
# ---------------------------------------------------------------------------

_PHILOX_M0 = 0xD2E7470EE14C6C93
_PHILOX_M1 = 0xCA5A826395121157
_PHILOX_W0 = 0x9E3779B97F4A7C15
_PHILOX_W1 = 0xBB67AE8584CAA73B
_MASK32 = np.uint64(0xFFFFFFFF)


def _mulhilo64(a: int, b: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Full 64x64 -> 128-bit product of a constant ``a`` and uint64 array ``b``."""
    b = b.astype(np.uint64)
    a_lo = np.uint64(a & 0xFFFFFFFF)
    a_hi = np.uint64(a >> 32)
    b_lo = b & _MASK32
    b_hi = b >> np.uint64(32)
    ll = a_lo * b_lo
    lh = a_lo * b_hi
    hl = a_hi * b_lo
    hh = a_hi * b_hi
    mid = (ll >> np.uint64(32)) + (lh & _MASK32) + (hl & _MASK32)
    lo = (ll & _MASK32) | ((mid & _MASK32) << np.uint64(32))
    hi = hh + (lh >> np.uint64(32)) + (hl >> np.uint64(32)) + (mid >> np.uint64(32))
    return hi, lo


def philox4x64_10(counter: np.ndarray, key: tuple[int, int]) -> np.ndarray:
    """Philox4x64 with 10 rounds.

    ``counter`` is a uint64 array of shape [..., 4] (word 0 first); returns
    the four output words with the same shape.
    """
    c = np.array(counter, dtype=np.uint64, copy=True)
    c0, c1, c2, c3 = (c[..., i].copy() for i in range(4))
    k0, k1 = int(key[0]) & 0xFFFFFFFFFFFFFFFF, int(key[1]) & 0xFFFFFFFFFFFFFFFF
    for rnd in range(10):
        if rnd > 0:
            k0 = (k0 + _PHILOX_W0) & 0xFFFFFFFFFFFFFFFF
            k1 = (k1 + _PHILOX_W1) & 0xFFFFFFFFFFFFFFFF
        hi0, lo0 = _mulhilo64(_PHILOX_M0, c0)
        hi1, lo1 = _mulhilo64(_PHILOX_M1, c2)
        c0, c1, c2, c3 = hi1 ^ c1 ^ np.uint64(k0), lo1, hi0 ^ c3 ^ np.uint64(k1), lo0
    return np.stack([c0, c1, c2, c3], axis=-1)


def philox_normals(seed: int, stream: tuple[int, int, int], n: int) -> np.ndarray:
    """``n`` standard normals from the Philox stream (counter words 1..3 fixed).

    Call j uses counter (j, stream[0], stream[1], stream[2]) and key
    (seed, 0); its four 64-bit words w0..w3 give uniforms
    u = ((w >> 11) + 1) * 2**-53 in (0, 1]; the pairs (u0, u1) and (u2, u3)
    give two normals each by Box-Muller: sqrt(-2 ln u_a) * (cos, sin)(2 pi u_b).
    Normal number e of the stream is output e % 4 of call e // 4.
    """
    calls = (n + 3) // 4
    ctr = np.zeros((calls, 4), dtype=np.uint64)
    ctr[:, 0] = np.arange(calls, dtype=np.uint64)
    ctr[:, 1] = np.uint64(stream[0])
    ctr[:, 2] = np.uint64(stream[1])
    ctr[:, 3] = np.uint64(stream[2])
    w = philox4x64_10(ctr, (seed, 0))
    u = ((w >> np.uint64(11)).astype(np.float64) + 1.0) * 2.0 ** -53
    r01 = np.sqrt(-2.0 * np.log(u[:, 0]))
    r23 = np.sqrt(-2.0 * np.log(u[:, 2]))
    t01 = 2.0 * np.pi * u[:, 1]
    t23 = 2.0 * np.pi * u[:, 3]
    z = np.stack([r01 * np.cos(t01), r01 * np.sin(t01), r23 * np.cos(t23), r23 * np.sin(t23)], axis=-1)
    return z.reshape(-1)[:n]


# ---------------------------------------------------------------------------
# Random projections ([P1] core components; [P3] section 2 and A.2)
# ---------------------------------------------------------------------------

def gram_schmidt_rows(g: np.ndarray) -> np.ndarray:
    """Orthonormalise the rows of ``g`` ([..., r, d], r <= d) in row order.

    Modified Gram-Schmidt: each row has the components along every earlier
    (already orthonormal) row removed one at a time, then is normalised.
    """
    u = np.array(g, dtype=np.float64, copy=True)
    r = u.shape[-2]
    for i in range(r):
        for j in range(i):
            proj = np.sum(u[..., i, :] * u[..., j, :], axis=-1, keepdims=True)
            u[..., i, :] = u[..., i, :] - proj * u[..., j, :]
        u[..., i, :] = u[..., i, :] / np.sqrt(np.sum(u[..., i, :] ** 2, axis=-1, keepdims=True))
    return u


def orf_from_gaussians(blocks: np.ndarray, lengths: np.ndarray, m: int) -> np.ndarray:
    """Orthogonal random features from raw Gaussian draws.

    ``blocks`` is [..., nb, d, d] (nb = ceil(m/d) Gaussian blocks), ``lengths``
    is [..., nb, d, d] (row i of block b gets the length of the Gaussian
    vector lengths[..., b, i, :]).  Each block's rows are orthonormalised in
    order and rescaled to those lengths; blocks are stacked and the first
    ``m`` rows kept.  Returns [..., m, d].
    """
    u = gram_schmidt_rows(blocks)
    norms = np.sqrt(np.sum(np.asarray(lengths, dtype=np.float64) ** 2, axis=-1, keepdims=True))
    w = u * norms
    d = w.shape[-1]
    w = w.reshape(*w.shape[:-3], -1, d)
    return w[..., :m, :]


def orf_omega(seed: int, n_heads: int, m: int, d: int) -> np.ndarray:
    """Seeded orthogonal projection, [n_heads, m, d] float32.

    Head h, block b: the d x d Gaussian is the first d*d normals of Philox
    stream (b, h, 0) read row-major; the chi(d) length of row i is the norm
    of normals i*d .. i*d+d-1 of stream (b, h, 1).
    """
    nb = (m + d - 1) // d
    out = np.empty((n_heads, m, d), dtype=np.float32)
    for h in range(n_heads):
        blocks = np.stack([philox_normals(seed, (b, h, 0), d * d).reshape(d, d) for b in range(nb)])
        lengths = np.stack([philox_normals(seed, (b, h, 1), d * d).reshape(d, d) for b in range(nb)])
        out[h] = orf_from_gaussians(blocks, lengths, m).astype(np.float32)
    return out


# ---------------------------------------------------------------------------
# Positive random features ([P1] core components and key formulas;
# [P2] Simple Derivation)
# ---------------------------------------------------------------------------

def sylvester_hadamard_int(d: int) -> np.ndarray:
    """Unnormalised Walsh-Hadamard matrix of order d (a power of two),
    Sylvester order: entries (-1)^popcount(i & j), as float64 integers."""
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    assert h.shape[0] == d, "d must be a power of two"
    return h


def sylvester_hadamard(d: int) -> np.ndarray:
    """Normalised Walsh-Hadamard matrix H = (unnormalised) / sqrt(d)."""
    return sylvester_hadamard_int(d) / np.sqrt(d)


def hadamard_block_from_signs(signs: np.ndarray) -> np.ndarray:
    """One structured orthogonal block sqrt(d) H S1 H S2 H S3 for sign rows
    ``signs`` ([3, d] of +-1), S_t = diag(signs[t]).  Computed exactly as
    (1/d) Hu S1 Hu S2 Hu S3 with the integer matrix Hu = sqrt(d) H: every
    product is an integer below 2^53 and d is a power of two."""
    d = signs.shape[1]
    hu = sylvester_hadamard_int(d)
    w = np.eye(d)
    for t in range(3):
        w = w @ hu @ np.diag(signs[t].astype(np.float64))
    return w / d


def hadamard_signs(seed: int, block: int, head: int, d: int) -> np.ndarray:
    """The +-1 diagonals of one block: diagonal t reads Philox4x64-10 with key
    (seed, 0) and counter (0, block, head, 2 + t); entry j is -1 when bit
    j % 64 of output word j // 64 is set (d <= 256)."""
    assert d <= 256
    ctr = np.array([[0, block, head, 2 + t] for t in range(3)], dtype=np.uint64)
    w = philox4x64_10(ctr, (seed, 0))
    j = np.arange(d)
    bits = (w[:, j // 64] >> (j % 64).astype(np.uint64)) & np.uint64(1)
    return np.where(bits == 1, -1.0, 1.0)


def hadamard_omega(seed: int, n_heads: int, m: int, d: int) -> np.ndarray:
    """Structured (Hadamard) orthogonal projection, [n_heads, m, d] float32.

    The pages name Hadamard ORFs as a cheaper ORF variant with a small bias
    that vanishes as d grows ([P3] A.2 ORF bullet and B.3 space/time
    trade-offs) without printing a construction; the reading taken is the
    structured block sqrt(d) H S1 H S2 H S3 (rows orthogonal, each of norm
    sqrt(d)), ceil(m/d) independent blocks per head, the last cut to the rows
    needed.
    """
    out = np.empty((n_heads, m, d), dtype=np.float32)
    nb = (m + d - 1) // d
    for h in range(n_heads):
        for b in range(nb):
            blk = hadamard_block_from_signs(hadamard_signs(seed, b, h, d))
            rows = min(d, m - b * d)
            out[h, b * d: b * d + rows] = blk[:rows].astype(np.float32)
    return out


def givens_default_rotations(d: int) -> int:
    """Default number of rotations per block: d * ceil(log2 d), the order of
    steps after which a walk of random plane rotations on d coordinates is
    close to a uniformly random rotation."""
    return d * max(1, int(np.ceil(np.log2(d))))


def givens_rotations(seed: int, block: int, head: int, d: int, count: int):
    """Plane rotations of one block, in the order they are applied.

    Rotation k reads Philox4x64-10 with key (seed, 0) and counter
    (k, block, head, 5); of its output words w0, w1, w2:
      i  = floor(d * (w0 >> 32) / 2^32),
      j' = floor((d - 1) * (w1 >> 32) / 2^32), j = j' + (j' >= i)  (so j != i,
           uniform over the other d - 1 coordinates),
      theta = 2 pi u, u = ((w2 >> 11) + 1) 2^-53.
    Returns (i, j, theta) arrays of length ``count``.
    """
    if count == 0:
        return np.zeros(0, np.int64), np.zeros(0, np.int64), np.zeros(0)
    ctr = np.zeros((count, 4), dtype=np.uint64)
    ctr[:, 0] = np.arange(count, dtype=np.uint64)
    ctr[:, 1] = np.uint64(block)
    ctr[:, 2] = np.uint64(head)
    ctr[:, 3] = np.uint64(5)
    w = philox4x64_10(ctr, (seed, 0))
    hi0 = (w[:, 0] >> np.uint64(32)).astype(object)
    hi1 = (w[:, 1] >> np.uint64(32)).astype(object)
    i = np.array([(d * int(a)) >> 32 for a in hi0], dtype=np.int64)
    jp = np.array([((d - 1) * int(a)) >> 32 for a in hi1], dtype=np.int64)
    j = jp + (jp >= i)
    theta = 2.0 * np.pi * (((w[:, 2] >> np.uint64(11)).astype(np.float64) + 1.0) * 2.0 ** -53)
    return i, j, theta


def givens_block(i: np.ndarray, j: np.ndarray, theta: np.ndarray, d: int) -> np.ndarray:
    """Product of plane rotations G_{K-1} ... G_1 G_0 (G_0 applied first) as
    a d x d matrix.  G_k is the identity except in rows/columns (i_k, j_k):
    [[cos, -sin], [sin, cos]], so left-multiplying mixes rows i_k and j_k."""
    qm = np.eye(d)
    for a, b, t in zip(i, j, theta):
        c, s = np.cos(t), np.sin(t)
        ra, rb = qm[a].copy(), qm[b].copy()
        qm[a] = c * ra - s * rb
        qm[b] = s * ra + c * rb
    return qm


def givens_omega(seed: int, n_heads: int, m: int, d: int, rotations: int = 0) -> np.ndarray:
    """Structured (Givens) orthogonal projection, [n_heads, m, d] float32.

    The pages name Givens ORFs beside Hadamard ones: orthogonal random
    features that keep O(log d) random numbers per row (O(m log d) in all),
    with a small bias that vanishes as d grows ([P3] A.2 ORF bullet, B.3
    space/time trade-offs), without printing a construction.  The reading
    taken: each d x d block is a product of ``rotations`` random plane
    rotations (d ceil(log2 d) when 0) applied to the identity
    (givens_rotations for the draws, givens_block for the order), and row i
    of the block is scaled to the length of an independent N(0, I_d) vector
    (the same chi(d) lengths as orf_omega: normals i*d .. i*d+d-1 of Philox
    stream (block, head, 1)).  ceil(m/d) independent blocks per head, the
    last cut to the rows needed.
    """
    if rotations < 0:
        raise ValueError("rotations must be >= 0")
    count = givens_default_rotations(d) if rotations == 0 else int(rotations)
    nb = (m + d - 1) // d
    out = np.empty((n_heads, m, d), dtype=np.float32)
    for h in range(n_heads):
        for b in range(nb):
            qm = givens_block(*givens_rotations(seed, b, h, d, count), d)
            lens = np.sqrt(np.sum(philox_normals(seed, (b, h, 1), d * d).reshape(d, d) ** 2, axis=1))
            rows = min(d, m - b * d)
            out[h, b * d: b * d + rows] = (qm * lens[:, None])[:rows].astype(np.float32)
    return out


def features(x: np.ndarray, omega: np.ndarray) -> np.ndarray:
    """phi(x)_i = m**-1/2 * exp(omega_i . x - |x|^2 / 2).

    ``x`` is [..., d], ``omega`` is [m, d] (or broadcastable [..., m, d]);
    returns [..., m] in float64.
    """
    x = np.asarray(x, dtype=np.float64)
    omega = np.asarray(omega, dtype=np.float64)
    m = omega.shape[-2]
    proj = np.einsum("...d,...md->...m", x, omega) if omega.ndim > 2 else x @ omega.T
    half_sq_norm = 0.5 * np.sum(x * x, axis=-1, keepdims=True)
    return np.exp(proj - half_sq_norm) / np.sqrt(m)


def features_relu(x: np.ndarray, omega: np.ndarray) -> np.ndarray:
    """Generalised (ReLU) random features phi(x)_i = m**-1/2 * max(omega_i . x, 0)
    (FAVOR+ with the ReLU kernel function; [P1] Digest, [P3] section 2).

    ``x`` is [..., d], ``omega`` [m, d]; returns [..., m] in float64.
    """
    x = np.asarray(x, dtype=np.float64)
    omega = np.asarray(omega, dtype=np.float64)
    m = omega.shape[-2]
    proj = np.einsum("...d,...md->...m", x, omega) if omega.ndim > 2 else x @ omega.T
    return np.maximum(proj, 0.0) / np.sqrt(m)


def features_trig(x: np.ndarray, omega: np.ndarray) -> np.ndarray:
    """Trigonometric random features of the softmax kernel, the estimator the
    pages compare positive features against ([P1] Digest: the cos/sin
    features of Rahimi and Recht; [P3] section 3, empirical approximation):

        phi(x) = m**-1/2 * exp(|x|^2 / 2) * [sin(omega_i . x), cos(omega_i . x)]_i

    so phi(x) . phi(y) = exp((|x|^2 + |y|^2)/2) * (1/m) sum_i cos(omega_i . (x - y)),
    whose expectation over omega ~ N(0, I_d) is exp(x . y) (the Gaussian
    characteristic function gives E cos(omega . z) = exp(-|z|^2 / 2)).
    ``x`` is [..., d], ``omega`` [m, d]; returns [..., 2m] in float64 (sines
    first).  Its values can be negative, so normalisers built from it can
    change sign.
    """
    x = np.asarray(x, dtype=np.float64)
    omega = np.asarray(omega, dtype=np.float64)
    m = omega.shape[-2]
    proj = x @ omega.T
    scale = np.exp(0.5 * np.sum(x * x, axis=-1, keepdims=True)) / np.sqrt(m)
    return scale * np.concatenate([np.sin(proj), np.cos(proj)], axis=-1)


def sm_hat_trig(x: np.ndarray, y: np.ndarray, omega: np.ndarray) -> np.ndarray:
    """Trigonometric estimate of exp(x . y): phi_trig(x) . phi_trig(y), for
    ``omega`` [m, d] or many independent draws [R, m, d] (returns [R])."""
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    omega = np.asarray(omega, dtype=np.float64)
    m = omega.shape[-2]
    z = x - y
    return np.exp(0.5 * (np.dot(x, x) + np.dot(y, y))) * np.sum(np.cos(omega @ z), axis=-1) / m


def trig_mse(x: np.ndarray, y: np.ndarray, m: int) -> float:
    """MSE of the trigonometric estimator with m i.i.d. Gaussian rows:
    exp(|x|^2 + |y|^2) * (1 - exp(-|x - y|^2))^2 / (2m), from
    Var cos(omega . z) = E cos^2 - (E cos)^2 = (1 + e^{-2|z|^2})/2 - e^{-|z|^2}.
    (The pages state only that this error explodes where the softmax kernel
    is small, [P1] Theoretical bounds; the closed form is the mathematics of
    the estimator.)"""
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    z2 = float(np.sum((x - y) ** 2))
    return float(np.exp(np.dot(x, x) + np.dot(y, y)) * (1.0 - np.exp(-z2)) ** 2 / (2.0 * m))


def iid_omega(seed: int, m: int, d: int) -> np.ndarray:
    """m i.i.d. N(0, I_d) projection rows (float32, numpy PCG64 seeded
    [seed, 7]): the unstructured projection the orthogonal one is compared
    with ([P1] Theoretical bounds, Theorem 2)."""
    rng = np.random.default_rng([seed, 7])
    return rng.standard_normal((m, d)).astype(np.float32)


def feature_map(kind: str):
    """The feature map of a kind: "positive" (softmax kernel, the default),
    "relu", or "trig" (trigonometric features, 2m columns)."""
    if kind == "positive":
        return features
    if kind == "relu":
        return features_relu
    if kind == "trig":
        return features_trig
    raise ValueError(f"unknown feature kind {kind!r}")


def features_stabilized(x: np.ndarray, omega: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Features with the per-row maximum exponent taken out.

    Returns (phi_s, s) with s = max_i(omega_i . x - |x|^2/2) and
    phi_s = m**-1/2 exp(omega_i . x - |x|^2/2 - s), so phi = phi_s * exp(s).
    A per-row factor on a query's features leaves the normalised attention
    unchanged ([P2] Simple Derivation).
    """
    x = np.asarray(x, dtype=np.float64)
    omega = np.asarray(omega, dtype=np.float64)
    m = omega.shape[-2]
    proj = x @ omega.T
    expo = proj - 0.5 * np.sum(x * x, axis=-1, keepdims=True)
    s = np.max(expo, axis=-1)
    return np.exp(expo - s[..., None]) / np.sqrt(m), s


def sm_hat(x: np.ndarray, y: np.ndarray, omega: np.ndarray) -> np.ndarray:
    """PRF estimate of the softmax kernel exp(x . y): phi(x) . phi(y).

    ([P1] key formulas, estimator SM-hat_m^PRF.)  ``omega`` may carry leading
    batch dimensions [R, m, d] for many independent draws; returns [R].
    """
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    omega = np.asarray(omega, dtype=np.float64)
    m = omega.shape[-2]
    px = omega @ x - 0.5 * np.dot(x, x)
    py = omega @ y - 0.5 * np.dot(y, y)
    return np.sum(np.exp(px + py), axis=-1) / m


def lemma2_mse(x: np.ndarray, y: np.ndarray, m: int) -> float:
    """Closed-form MSE of the i.i.d. PRF estimator ([P1] Theoretical bounds, Lemma 2).

    MSE = (1/m) * exp(|x+y|^2) * SM(x,y)^2 * (1 - exp(-|x+y|^2)).
    """
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    s = float(np.sum((x + y) ** 2))
    sm = float(np.exp(np.dot(x, y)))
    return (1.0 / m) * np.exp(s) * sm * sm * (1.0 - np.exp(-s))


# ---------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------

def _head_omega(omega: np.ndarray, h: int) -> np.ndarray:
    omega = np.asarray(omega, dtype=np.float64)
    if omega.ndim == 2:
        return omega
    if omega.shape[0] == 1:
        return omega[0]
    return omega[h]


def bidir(q: np.ndarray, k: np.ndarray, v: np.ndarray, omega: np.ndarray, kind: str = "positive") -> np.ndarray:
    """Bidirectional FAVOR+ ([P1] key formulas and method flowchart).

    For each head: KV = phi(K)^T V (m x d), z = phi(K)^T 1_L (m),
    out_t = phi(q_t)^T KV / phi(q_t)^T z.  Inputs [B, H, L, d]; output float64.
    ``kind`` selects the feature map (``feature_map``).
    """
    features = feature_map(kind)
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, L, d = q.shape
    out = np.empty((B, H, L, v.shape[-1]), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            om = _head_omega(omega, h)
            phi_q = features(q[b, h], om)
            phi_k = features(k[b, h], om)
            kv = phi_k.T @ v[b, h]
            z = phi_k.sum(axis=0)
            out[b, h] = (phi_q @ kv) / (phi_q @ z)[:, None]
    return out


def causal(q: np.ndarray, k: np.ndarray, v: np.ndarray, omega: np.ndarray, kind: str = "positive") -> np.ndarray:
    """Unidirectional FAVOR+ by the prefix-sum recurrence ([P1] Methods, core
    components: G_t = sum_{s<=t} phi(k_s) v_s^T; [P3] A.2 unidirectional
    attention).

    Walks t = 0 .. L-1 in order: G += phi(k_t) v_t^T, z += phi(k_t),
    out_t = phi(q_t)^T G / phi(q_t)^T z.  Inputs [B, H, L, d]; float64 out.
    ``kind`` selects the feature map (``feature_map``).
    """
    features = feature_map(kind)
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, L, d = q.shape
    dv = v.shape[-1]
    out = np.empty((B, H, L, dv), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            om = _head_omega(omega, h)
            m = om.shape[0]
            phi_q = features(q[b, h], om)
            phi_k = features(k[b, h], om)
            G = np.zeros((m, dv))
            z = np.zeros(m)
            for t in range(L):
                G += np.outer(phi_k[t], v[b, h, t])
                z += phi_k[t]
                out[b, h, t] = (phi_q[t] @ G) / (phi_q[t] @ z)
    return out


def causal_with_state(q: np.ndarray, k: np.ndarray, v: np.ndarray, omega: np.ndarray, state=None):
    """Causal FAVOR+ continuing from a carried prefix state, and the state
    after the last position ([P1] Methods: G_t is a running sum over s <= t, so
    a sequence split into pieces can hand G and z from one piece to the next;
    [P2] Simple Derivation: the recurrent form of causal linear attention).

    The state of a head is (G, z) with G = sum over the keys seen so far of
    e(k_s) v_s^T ([m, d]) and z = sum e(k_s) ([m]), where
    e(k)_i = exp(omega_i . k - |k|^2/2) is the feature map without its m^-1/2
    factor.  ``state`` is None (nothing seen yet) or a pair of arrays
    ([B, H, m, d], [B, H, m]).  Walks t = 0 .. L-1 in order: G += e(k_t) v_t^T,
    z += e(k_t), out_t = e(q_t)^T G / e(q_t)^T z.  Returns (out [B, H, L, d],
    (G, z)) in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, L, d = q.shape
    dv = v.shape[-1]
    out = np.empty((B, H, L, dv), dtype=np.float64)
    m = np.asarray(omega).shape[-2]
    G_all = np.zeros((B, H, m, dv))
    z_all = np.zeros((B, H, m))
    for b in range(B):
        for h in range(H):
            om = _head_omega(omega, h)
            e_q = features(q[b, h], om) * np.sqrt(m)
            e_k = features(k[b, h], om) * np.sqrt(m)
            if state is None:
                G = np.zeros((m, dv))
                z = np.zeros(m)
            else:
                G = np.array(state[0][b, h], dtype=np.float64)
                z = np.array(state[1][b, h], dtype=np.float64)
            for t in range(L):
                G += np.outer(e_k[t], v[b, h, t])
                z += e_k[t]
                out[b, h, t] = (e_q[t] @ G) / (e_q[t] @ z)
            G_all[b, h] = G
            z_all[b, h] = z
    return out, (G_all, z_all)


def causal_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, omega: np.ndarray, rows: np.ndarray,
                kind: str = "positive") -> np.ndarray:
    """Causal FAVOR+ output at selected positions of one head.

    ``q, k, v`` are [L, d] for one head, ``omega`` [m, d]; for each t in
    ``rows`` returns sum_{s<=t} (phi(q_t).phi(k_s)) v_s / sum_{s<=t}
    phi(q_t).phi(k_s), the same quantity as ``causal`` written as a sum over
    keys (associativity, [P1] atomic insights), so that single rows of very
    long sequences can be checked without the whole prefix scan.
    """
    features = feature_map(kind)
    om = np.asarray(omega, dtype=np.float64)
    phi_k = features(np.asarray(k, dtype=np.float64), om)
    v = np.asarray(v, dtype=np.float64)
    res = np.empty((len(rows), v.shape[-1]))
    for i, t in enumerate(rows):
        pq = features(np.asarray(q[t], dtype=np.float64), om)
        w = phi_k[: t + 1] @ pq
        res[i] = (w @ v[: t + 1]) / w.sum()
    return res


def bidir_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, omega: np.ndarray, rows: np.ndarray,
               kind: str = "positive") -> np.ndarray:
    """Bidirectional FAVOR+ output at selected positions of one head."""
    features = feature_map(kind)
    om = np.asarray(omega, dtype=np.float64)
    phi_k = features(np.asarray(k, dtype=np.float64), om)
    v = np.asarray(v, dtype=np.float64)
    kv = phi_k.T @ v
    z = phi_k.sum(axis=0)
    pq = features(np.asarray(q, dtype=np.float64)[np.asarray(rows)], om)
    return (pq @ kv) / (pq @ z)[:, None]


def brute_force(q: np.ndarray, k: np.ndarray, v: np.ndarray, omega: np.ndarray, causal_mask: bool,
                kind: str = "positive") -> np.ndarray:
    """FAVOR+ through the explicit L x L matrix A-hat = phi(Q) phi(K)^T.

    out = diag(A-hat 1)^-1 A-hat V, with A-hat zeroed above the diagonal for
    the causal variant ([P3] section 2: the unidirectional form uses the
    lower-triangular part).  One head: q, k, v are [L, d].  Tiny inputs only.
    """
    features = feature_map(kind)
    om = np.asarray(omega, dtype=np.float64)
    a_hat = features(q, om) @ features(k, om).T
    if causal_mask:
        a_hat = np.tril(a_hat)
    return (a_hat @ np.asarray(v, dtype=np.float64)) / a_hat.sum(axis=1, keepdims=True)


def softmax_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, causal_mask: bool) -> np.ndarray:
    """Exact softmax attention with the kernel exp(q . k) and no temperature.

    A(i,j) = exp(q_i.k_j) / sum_j exp(q_i.k_j) over all j, or over j <= i for
    the causal variant ([P1] Methods; [P2] Concentrating Attention).  One
    head: q, k, v are [L, d].  Used only as the Monte-Carlo target.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    s = q @ k.T
    if causal_mask:
        s = np.where(np.tril(np.ones_like(s, dtype=bool)), s, -np.inf)
    s = s - s.max(axis=1, keepdims=True)
    a = np.exp(s)
    a = a / a.sum(axis=1, keepdims=True)
    return a @ np.asarray(v, dtype=np.float64)
