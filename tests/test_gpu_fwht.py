"""GPU parity of favor_features_hadamard: features over the structured
Hadamard projection built with fast Walsh-Hadamard transforms, against the
oracle's features over the materialised projection (oracle.hadamard_omega),
for both dtypes, per-head and shared projections, ragged lengths, the
stabiliser and ReLU features; and agreement with the dense entry point fed
the device-generated projection."""

import numpy as np
import pytest
import torch

import oracle.reference as ref
import positive_random_feature_amd as favor
from positive_random_feature_amd.workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
# The transform path projects in fp32 with exact +-1 entries (no rounding of
# the projection to the input dtype), so both dtypes meet the fp32 bar.
TOL = 1e-5


def _x(dtype, B, H, L, d, seed=3):
    w = WORKLOADS["bidir_bf16_4k" if dtype == "bf16" else "bidir_f32_tiny"].replace(d=d)
    inp = make_inputs(w, B=B, H=H, L=L, seed=seed)
    if dtype == "bf16":
        x = torch.from_numpy(inp.q_bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    else:
        x = torch.from_numpy(inp.q).to(DEV)
    return x, inp.q.astype(np.float64)


def _rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


@pytest.mark.parametrize("dtype,d,m,per_head", [("bf16", 64, 256, True), ("bf16", 128, 512, True),
                                                ("bf16", 16, 32, False), ("f32", 64, 96, True),
                                                ("f32", 32, 64, False), ("bf16", 32, 160, True)])
def test_fwht_features_match_oracle(dtype, d, m, per_head):
    B, H, L, seed = 2, 3, 333, 17
    x, xs = _x(dtype, B, H, L, d)
    om = ref.hadamard_omega(seed, H if per_head else 1, m, d).astype(np.float64)
    want = np.stack([np.stack([ref.features(xs[b, h], om[h if per_head else 0]) for h in range(H)]) for b in range(B)])
    phi, _ = favor.features_hadamard(x, seed, m, per_head=per_head)
    got = phi.cpu().numpy().astype(np.float64)
    err = _rel(got, want)
    print(f"[fwht] {dtype} d={d} m={m} per_head={per_head}: rel L2 {err:.3e}", flush=True)
    assert err <= TOL
    # stabilised: phi_s exp(s) = phi and s is the oracle's row maximum
    phs, ls = favor.features_hadamard(x, seed, m, per_head=per_head, stabilize=True)
    phs = phs.cpu().numpy().astype(np.float64)
    ls = ls.cpu().numpy().astype(np.float64)
    assert phs.max() <= 1.0 / np.sqrt(m) * (1 + 1e-5)
    assert _rel(phs * np.exp(ls)[..., None], want) <= TOL
    s_want = np.stack([np.stack([ref.features_stabilized(xs[b, h], om[h if per_head else 0])[1] for h in range(H)])
                       for b in range(B)])
    assert np.abs(ls - s_want).max() <= 1e-4 * (1 + np.abs(s_want).max())


@pytest.mark.parametrize("dtype,d,m", [("bf16", 64, 256), ("f32", 16, 64)])
def test_fwht_relu_features_match_oracle(dtype, d, m):
    B, H, L, seed = 1, 2, 129, 5
    x, xs = _x(dtype, B, H, L, d)
    om = ref.hadamard_omega(seed, H, m, d).astype(np.float64)
    want = np.stack([np.stack([ref.features_relu(xs[b, h], om[h]) for h in range(H)]) for b in range(B)])
    phi, ls = favor.features_hadamard(x, seed, m, stabilize=True, feature="relu")
    err = _rel(phi.cpu().numpy().astype(np.float64), want)
    print(f"[fwht] relu {dtype} d={d} m={m}: rel L2 {err:.3e}", flush=True)
    assert err <= TOL
    assert float(ls.abs().max()) == 0.0


def test_fwht_agrees_with_dense_projection():
    """The dense entry point fed the device-generated Hadamard projection
    gives the same features within its bf16-projection tolerance."""
    B, H, L, d, m, seed = 1, 4, 500, 64, 256, 8
    x, _ = _x("bf16", B, H, L, d)
    om = favor.hadamard_omega(seed, H, m, d, device=DEV)
    dense, _ = favor.features(x, om)
    fast, _ = favor.features_hadamard(x, seed, m)
    err = _rel(dense.double().cpu().numpy(), fast.double().cpu().numpy())
    print(f"[fwht] dense vs transform (bf16 projection): rel L2 {err:.3e} (tol 2e-2)", flush=True)
    assert err <= 2e-2


def test_fwht_empty_and_one_token():
    x = torch.zeros((1, 2, 0, 64), dtype=torch.bfloat16, device=DEV)
    phi, _ = favor.features_hadamard(x, 1, 128)
    assert phi.shape == (1, 2, 0, 128)
    x1, xs = _x("bf16", 1, 1, 1, 64)
    om = ref.hadamard_omega(1, 1, 128, 64).astype(np.float64)
    phi, _ = favor.features_hadamard(x1, 1, 128)
    assert _rel(phi.cpu().numpy()[0, 0].astype(np.float64), ref.features(xs[0, 0], om[0])) <= TOL
