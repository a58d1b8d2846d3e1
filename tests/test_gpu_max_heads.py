"""GPU parity at the largest supported number of (batch, head) pairs,
B*H = 65535: the kernels give each pair one grid row, so every launch of a
call runs at the hardware's grid-dimension limit.  Short sequences keep the
oracle cheap; forced two-segment plans put the segment-sum, merge and output
or scan kernels at the limit, the automatic plans the one-segment paths.
Every element against the fp64 oracle, the whole output and every head
within the bar (2e-2 for bf16 inputs)."""

import os
import sys

import numpy as np
import pytest
import torch

import oracle.native as native
import oracle.reference as ref
import positive_random_feature_amd as favor
from positive_random_feature_amd.workloads import WORKLOADS, make_inputs

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from bf16_rounding import features_bf16_operand, fp32_feature_bound  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
BH = 65535
TOL = 2e-2


def _inputs(d, m, L, seed):
    w = WORKLOADS["causal_bf16_8k"].replace(d=d, m=m, omega_per_head=False)
    inp = make_inputs(w, B=BH, H=1, L=L, seed=seed)
    dev = [torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(DEV) for b in (inp.q_bits, inp.k_bits, inp.v_bits)]
    om = ref.orf_omega(seed, 1, m, d)[0]
    return inp, dev, om


def _check(tag, got, want):
    err = float(np.linalg.norm(got - want) / np.linalg.norm(want))
    diff = (got - want).reshape(BH, -1)
    per_head = np.linalg.norm(diff, axis=1) / np.linalg.norm(want.reshape(BH, -1), axis=1)
    print(f"[max-heads] {tag}: rel L2 {err:.3e}, worst head {per_head.max():.3e}", flush=True)
    assert np.isfinite(got).all()
    assert err <= TOL and per_head.max() <= TOL


@pytest.mark.parametrize("op,d,m,L,segments", [
    ("bidir", 16, 32, 64, 2),    # segment sums, merge, output pass: grid rows = 65535
    ("bidir", 16, 32, 40, 0),    # automatic plan: the key-split one-kernel path
    ("causal", 16, 32, 64, 2),   # segment sums, scan, chunk scan
    ("causal", 16, 32, 50, 0),   # automatic plan: one segment, no carry
    ("causal", 64, 64, 64, 0),   # the 64-token tile scan
])
def test_max_heads(op, d, m, L, segments):
    inp, (q, k, v), om = _inputs(d, m, L, seed=31 + d + m + L)
    omd = torch.from_numpy(np.ascontiguousarray(om)).to(DEV)
    print(f"[max-heads] {op} d={d} m={m} {BH}x1x{L} segments={segments}", flush=True)
    if op == "bidir":
        got = favor.bidir(q, k, v, omd, segments=segments)
    else:
        got = favor.causal(q, k, v, omd, segments=segments)
    torch.cuda.synchronize()
    got = got.float().cpu().numpy().astype(np.float64)
    want = (native.bidir if op == "bidir" else native.causal)(inp.q, inp.k, inp.v, om)
    _check(f"{op} d={d} m={m} L={L} segments={segments}", got, want)


def test_max_heads_features():
    # 64 tokens per head, so that each head's figure covers enough elements
    d, m, L = 16, 32, 64
    inp, (q, _k, _v), om = _inputs(d, m, L, seed=77)
    print(f"[max-heads] features d={d} m={m} {BH}x1x{L}", flush=True)
    phi, _ = favor.features(q, torch.from_numpy(np.ascontiguousarray(om)).to(DEV))
    torch.cuda.synchronize()
    got = phi.cpu().numpy().astype(np.float64)
    want = ref.features(inp.q, om)
    _check(f"features d={d} m={m} L={L}", got, want)
    # The one rounding the matrix cores need is that of the projection
    # operand log2(e) * omega (q is bf16 already), carried at d = 16 as a high
    # and a low bf16 part.  Against the definition evaluated in fp64 with that
    # operand, every head is within the a-priori error bound of fp32
    # arithmetic.
    emu = features_bf16_operand(inp.q.reshape(BH, L, d), om)
    diff = (got.reshape(BH, L, m) - emu).reshape(BH, -1)
    per_head = np.linalg.norm(diff, axis=1) / np.linalg.norm(emu.reshape(BH, -1), axis=1)
    bound = fp32_feature_bound(inp.q.reshape(BH, L, d), om)
    print(f"[max-heads] features against the bf16-operand definition: worst head {per_head.max():.3e} "
          f"(fp32 bound {bound:.2e})", flush=True)
    assert per_head.max() <= bound
