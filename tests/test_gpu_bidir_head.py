"""The one-kernel bidirectional path (one workgroup per head computes the
head's sums and then its outputs), taken when the launch plan gives each head
a single segment (many heads of short sequences, or an explicit one-segment
plan) and its operands fit in LDS.  Every element against the fp64 oracle,
for both dtypes, d from 16 to 128, m up to 256, shared and per-head
projections, ragged and one-token sequences, ReLU features (the bf16 d = 128,
m = 128 and fp32 d = 64, m = 128 cases do not fit and run the three kernels on
the one-segment plan); and the one-segment plan against a multi-segment plan
of the same call."""

import numpy as np
import pytest
import torch

import oracle.native as native
import oracle.reference as ref
import positive_random_feature_amd as favor
from positive_random_feature_amd.workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = {"f32": 1e-5, "bf16": 2e-2}


def _case(dtype, d, m, B, H, L, per_head, seed=5):
    w = WORKLOADS["bidir_bf16_4k" if dtype == "bf16" else "bidir_f32_tiny"].replace(d=d, m=m, omega_per_head=per_head)
    inp = make_inputs(w, B=B, H=H, L=L, seed=seed)
    om = ref.orf_omega(seed, H if per_head else 1, m, d)
    om = om if per_head else om[0]
    if dtype == "bf16":
        dev = [torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(DEV) for b in (inp.q_bits, inp.k_bits, inp.v_bits)]
    else:
        dev = [torch.from_numpy(a).to(DEV) for a in (inp.q, inp.k, inp.v)]
    return inp, om, dev


def _rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


@pytest.mark.parametrize("dtype,d,m,B,H,L,per_head,feature", [
    ("bf16", 64, 256, 8, 8, 384, False, "positive"),
    ("bf16", 64, 256, 16, 8, 512, True, "positive"),
    ("bf16", 64, 256, 16, 4, 301, True, "positive"),
    ("bf16", 128, 128, 8, 8, 200, True, "positive"),
    ("bf16", 32, 64, 4, 16, 97, False, "positive"),
    ("bf16", 16, 32, 64, 1, 33, True, "positive"),
    ("f32", 64, 128, 8, 8, 150, True, "positive"),
    ("f32", 16, 32, 2, 32, 1, False, "positive"),
    ("bf16", 64, 256, 8, 8, 129, True, "relu"),
])
def test_one_kernel_path_matches_oracle(dtype, d, m, B, H, L, per_head, feature):
    inp, om, (q, k, v) = _case(dtype, d, m, B, H, L, per_head)
    got = favor.bidir(q, k, v, torch.from_numpy(np.ascontiguousarray(om)).to(DEV), feature=feature)
    got = got.float().cpu().numpy().astype(np.float64)
    if feature == "relu":
        want = ref.bidir(inp.q, inp.k, inp.v, om, kind="relu")
    else:
        want = native.bidir(inp.q, inp.k, inp.v, om)
    err = _rel(got, want)
    # every head on its own as well
    worst = max(_rel(got[b, h], want[b, h]) for b in range(B) for h in range(H))
    print(f"[bidir_head] {dtype} d={d} m={m} {B}x{H}x{L} per_head={per_head} {feature}: rel L2 {err:.3e}, "
          f"worst head {worst:.3e}", flush=True)
    assert err <= TOL[dtype] and worst <= TOL[dtype]


@pytest.mark.parametrize("segments", [2, 5])
def test_one_segment_plan_against_more_segments(segments):
    """Forcing one segment on a few heads takes the one-kernel path too; its
    result agrees with the multi-segment plan of the same call (bf16
    rounding of the merged operand aside)."""
    inp, om, (q, k, v) = _case("bf16", 64, 256, 1, 2, 700, True)
    omd = torch.from_numpy(om).to(DEV)
    one = favor.bidir(q, k, v, omd, segments=1).float()
    many = favor.bidir(q, k, v, omd, segments=segments).float()
    want = native.bidir(inp.q, inp.k, inp.v, om)
    assert _rel(one.cpu().numpy().astype(np.float64), want) <= TOL["bf16"]
    assert float((one - many).norm() / many.norm()) <= 1e-2


def test_one_kernel_path_empty():
    q = torch.zeros((8, 8, 0, 64), dtype=torch.bfloat16, device=DEV)
    om = favor.orf_omega(1, 1, 256, 64)[0].contiguous().to(DEV)
    out = favor.bidir(q, q, q, om)
    assert out.shape == q.shape
