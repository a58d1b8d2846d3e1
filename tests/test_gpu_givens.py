"""GPU parity of the structured (Givens) orthogonal projection generated on
the device (favor_givens_omega): equal to the oracle's construction up to the
last fp32 rounding (both sides build the block in fp64 from the same Philox
draws), and attention over it matching the oracle."""

import numpy as np
import pytest
import torch

import oracle.native as native
import oracle.reference as ref
import positive_random_feature_amd as favor
from positive_random_feature_amd.workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("seed,H,m,d,rot", [(0, 1, 32, 16, 0), (3, 2, 40, 16, 0), (9, 2, 256, 64, 0),
                                             (5, 2, 512, 128, 0), (1, 3, 7, 5, 0), (2, 1, 64, 64, 1),
                                             (4, 2, 48, 32, 700), (6, 1, 3, 2, 3)])
def test_device_projection_equals_oracle(seed, H, m, d, rot):
    got = favor.givens_omega(seed, H, m, d, rotations=rot, device="cuda:0").cpu().numpy()
    want = ref.givens_omega(seed, H, m, d, rotations=rot)
    # the two sides round the same fp64 value to fp32; libm-level differences
    # in cos, sin, log and the summation order of the lengths can move a
    # value across a rounding boundary: one fp32 ulp at most
    ulp = np.spacing(np.abs(want).astype(np.float32))
    diff = np.abs(got.astype(np.float64) - want.astype(np.float64))
    print(f"[givens] seed={seed} H={H} m={m} d={d} rot={rot}: max |diff| / ulp = {float((diff / ulp).max()):.2f}, "
          f"exactly equal {float((diff == 0).mean()):.4f}", flush=True)
    assert np.all(diff <= ulp)
    assert float((diff == 0).mean()) > 0.99


@pytest.mark.parametrize("d,m", [(64, 256), (128, 512)])
@pytest.mark.parametrize("op", ["bidir", "causal"])
def test_attention_over_givens_projection(d, m, op):
    w = WORKLOADS["causal_bf16_8k"].replace(d=d, m=m, omega_per_head=True)
    B, H, L = 1, 4, 700
    inp = make_inputs(w, B=B, H=H, L=L)
    om_dev = favor.givens_omega(13, H, m, d, device="cuda:0")
    q, k, v = (torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to("cuda:0") for b in (inp.q_bits, inp.k_bits, inp.v_bits))
    fn = favor.bidir if op == "bidir" else favor.causal
    got = fn(q, k, v, om_dev)
    torch.cuda.synchronize()
    om = ref.givens_omega(13, H, m, d)
    want = (native.bidir if op == "bidir" else native.causal)(inp.q, inp.k, inp.v, om)
    got = got.float().cpu().numpy().astype(np.float64)
    err = float(np.linalg.norm(got - want) / np.linalg.norm(want))
    print(f"[givens] {op} d={d} m={m}: rel L2 {err:.3e} (tol 2e-2)", flush=True)
    assert err <= 2e-2
