"""The key-split one-kernel bidirectional path for 32 features (d <= 64 in
bf16, d <= 32 in fp32), taken when the launch plan gives each head one
segment: the eight waves of a head's workgroup split the keys, each with its
own shift, and their sums meet rescaled to the largest before the output
pass.  Every element against the fp64 oracle for both dtypes and every d,
ragged lengths around the 32-token chunks and the eight waves, shared and
per-head projections, ReLU features, and keys whose spikes make the waves'
shifts differ and rise after their first chunk.  The one-segment plans with
m = 64, and fp32 with d = 64, run the feature-split one-kernel path and are
checked here as well."""

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


def _rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def _run(dtype, d, m, B, H, L, per_head, feature="positive", seed=11, spike=None):
    w = WORKLOADS["bidir_bf16_4k" if dtype == "bf16" else "bidir_f32_tiny"].replace(d=d, m=m, omega_per_head=per_head)
    inp = make_inputs(w, B=B, H=H, L=L, seed=seed)
    k = inp.k.copy()
    if spike is not None:
        # a few keys scaled by a power of two (exact in bf16): their
        # projections dominate, so the waves that hold them raise their shift
        for t, f in spike:
            if t < L:
                k[:, :, t, :] *= f
    om = ref.orf_omega(seed, H if per_head else 1, m, d)
    om = om if per_head else om[0]
    if dtype == "bf16":
        kb = np.ascontiguousarray(k).view(np.uint32) >> 16  # k stays bf16-representable
        dev = [torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(DEV)
               for b in (inp.q_bits, kb.astype(np.uint16), inp.v_bits)]
    else:
        dev = [torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in (inp.q, k, inp.v)]
    got = favor.bidir(*dev, torch.from_numpy(np.ascontiguousarray(om)).to(DEV), feature=feature, segments=1)
    got = got.float().cpu().numpy().astype(np.float64)
    if feature == "relu":
        want = ref.bidir(inp.q, k, inp.v, om, kind="relu")
    else:
        want = native.bidir(inp.q, k, inp.v, om)
    err = _rel(got, want)
    worst = max(_rel(got[b, h], want[b, h]) for b in range(B) for h in range(H))
    print(f"[bidir_small] {dtype} d={d} m={m} {B}x{H}x{L} per_head={per_head} {feature} spike={spike is not None}: "
          f"rel L2 {err:.3e}, worst head {worst:.3e}", flush=True)
    assert err <= TOL[dtype] and worst <= TOL[dtype]
    return got


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [16, 32, 64])
@pytest.mark.parametrize("m", [32, 64])
def test_every_shape(dtype, d, m):
    _run(dtype, d, m, 2, 3, 300, per_head=(d == 32))


@pytest.mark.parametrize("dtype,d,m", [("bf16", 64, 32), ("f32", 16, 32)])
@pytest.mark.parametrize("L", [1, 31, 32, 33, 255, 256, 257, 2000])
def test_lengths(dtype, d, m, L):
    _run(dtype, d, m, 1, 2, L, per_head=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_relu(dtype):
    _run(dtype, 32, 32, 2, 2, 517, per_head=False, feature="relu")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_wave_shifts_differ_and_rise(dtype):
    # wave 5's first chunk, and wave 2's second chunk (tokens 320..351)
    d = 64 if dtype == "bf16" else 32
    _run(dtype, d, 32, 1, 2, 700, per_head=True, spike=[(5 * 32 + 3, 4.0), (2 * 32 + 256 + 7, 8.0)])


def test_against_segmented_plan():
    """The one-segment result agrees with the three-kernel plan of the same
    call (bf16 rounding of the merged operand aside)."""
    w = WORKLOADS["bidir_bf16_4k"].replace(d=64, m=32)
    inp = make_inputs(w, B=2, H=4, L=1500, seed=3)
    q, k, v = (torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(DEV)
               for b in (inp.q_bits, inp.k_bits, inp.v_bits))
    om = torch.from_numpy(ref.orf_omega(3, 1, 32, 64)[0]).to(DEV)
    one = favor.bidir(q, k, v, om, segments=1).float()
    many = favor.bidir(q, k, v, om, segments=6).float()
    assert float((one - many).norm() / many.norm()) <= 1e-2


@pytest.mark.parametrize("B,H", [(16, 8), (127, 1)])
def test_plan_limit(B, H):
    """The automatic plan at its limit for 32 features: 128 heads of 4096
    tokens take the key-split kernel (one segment per head), 127 heads of
    the same length keep the segmented kernels; every element against the
    oracle either way."""
    w = WORKLOADS["bidir_bf16_4k"].replace(d=32, m=32, omega_per_head=False)
    inp = make_inputs(w, B=B, H=H, L=4096, seed=21)
    om = ref.orf_omega(21, 1, 32, 32)[0]
    q, k, v = (torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(DEV)
               for b in (inp.q_bits, inp.k_bits, inp.v_bits))
    got = favor.bidir(q, k, v, torch.from_numpy(np.ascontiguousarray(om)).to(DEV))
    got = got.float().cpu().numpy().astype(np.float64)
    want = native.bidir(inp.q, inp.k, inp.v, om)
    err = _rel(got, want)
    worst = max(_rel(got[b, h], want[b, h]) for b in range(B) for h in range(H))
    print(f"[bidir_small] plan limit {B}x{H}x4096 d=32 m=32: rel L2 {err:.3e}, worst head {worst:.3e}", flush=True)
    assert err <= TOL["bf16"] and worst <= TOL["bf16"]
