"""Split invariance on the GPU: causal and bidirectional FAVOR+ give the
oracle's result whatever the chunk length and however each head is cut into
segments ("paperlayer.ai" summary of arXiv:2009.14794v4, A.2: the prefix sums
parallelise over any split, so chunk and segment counts change only the
rounding).  Every element is compared with the plain-C oracle; bar 2e-2 rel
L2 for bf16 inputs, 1e-5 for fp32, also on every 64-token tile."""

import numpy as np
import pytest
import torch

import oracle.native as native
import oracle.reference as ref
import positive_random_feature_amd as favor
from positive_random_feature_amd.workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}


def _dev():
    return torch.device("cuda:0")


def _to_dev(inp, dtype):
    if dtype == "bf16":
        return [torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(_dev()) for b in (inp.q_bits, inp.k_bits, inp.v_bits)]
    return [torch.from_numpy(a).to(_dev()) for a in (inp.q, inp.k, inp.v)]


def _rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def _worst_tile(got, want, tile=64):
    worst = 0.0
    B, H, L, _ = want.shape
    for b in range(B):
        for h in range(H):
            for t0 in range(0, L, tile):
                w = want[b, h, t0:t0 + tile]
                worst = max(worst, float(np.linalg.norm(got[b, h, t0:t0 + tile] - w) / np.linalg.norm(w)))
    return worst


def _case(base, d, m, B, H, L, dtype="bf16", seed=None):
    w = WORKLOADS[base].replace(d=d, m=m) if dtype == "bf16" else WORKLOADS["bidir_f32_tiny"].replace(
        d=d, m=m, omega_per_head=True)
    inp = make_inputs(w, B=B, H=H, L=L, seed=seed)
    om = ref.orf_omega(w.seed, H, m, d)
    return w, inp, om, _to_dev(inp, w.dtype), torch.from_numpy(om).to(_dev())


CAUSAL = [  # (d, m, chunks, segment counts, B, H, L)
    (64, 256, (64, 32), (1, 2, 3, 7, 16, 40, 0), 1, 2, 3000),
    (64, 128, (64, 32), (1, 5, 0), 2, 1, 2100),
    (64, 64, (64, 32), (1, 3, 0), 1, 2, 777),
    (128, 512, (32,), (1, 3, 8, 0), 1, 2, 1500),
    (128, 256, (32,), (1, 4, 0), 1, 2, 1300),
    (32, 64, (32,), (1, 5, 0), 1, 2, 1000),
]


@pytest.mark.parametrize("d,m,chunks,segs,B,H,L", CAUSAL)
def test_causal_chunk_and_segment_invariance(d, m, chunks, segs, B, H, L):
    w, inp, om, (q, k, v), om_d = _case("causal_bf16_8k", d, m, B, H, L)
    want = native.causal(inp.q, inp.k, inp.v, om)
    outs = {}
    for chunk in chunks:
        for seg in segs:
            got = favor.causal(q, k, v, om_d, chunk=chunk, segments=seg).float().cpu().numpy().astype(np.float64)
            err, tile = _rel(got, want), _worst_tile(got, want)
            print(f"[plan] causal d={d} m={m} {B}x{H}x{L} chunk={chunk} segments={seg}: rel L2 {err:.3e}, "
                  f"worst tile {tile:.3e}", flush=True)
            assert np.isfinite(got).all()
            assert err <= TOL["bf16"] and tile <= TOL["bf16"]
            outs[(chunk, seg)] = got
    # the splits agree with one another far more closely than with the bar
    first = next(iter(outs.values()))
    for key, o in outs.items():
        assert _rel(o, first) <= 1e-2, key


@pytest.mark.parametrize("d,m,segs,B,H,L", [(64, 256, (1, 2, 5, 13, 0), 2, 2, 2500),
                                             (128, 512, (1, 3, 0), 1, 2, 1200),
                                             (16, 32, (1, 4, 0), 1, 3, 500)])
def test_bidir_segment_invariance(d, m, segs, B, H, L):
    w, inp, om, (q, k, v), om_d = _case("bidir_bf16_4k", d, m, B, H, L)
    want = native.bidir(inp.q, inp.k, inp.v, om)
    for seg in segs:
        got = favor.bidir(q, k, v, om_d, segments=seg).float().cpu().numpy().astype(np.float64)
        err, tile = _rel(got, want), _worst_tile(got, want)
        print(f"[plan] bidir d={d} m={m} {B}x{H}x{L} segments={seg}: rel L2 {err:.3e}, worst tile {tile:.3e}",
              flush=True)
        assert err <= TOL["bf16"] and tile <= TOL["bf16"]


@pytest.mark.parametrize("op", ["bidir", "causal"])
@pytest.mark.parametrize("segs", [1, 3, 0])
def test_fp32_segment_invariance(op, segs):
    w, inp, om, (q, k, v), om_d = _case("bidir_f32_tiny", 32, 64, 1, 2, 700, dtype="f32")
    fn = favor.bidir if op == "bidir" else favor.causal
    got = fn(q, k, v, om_d, segments=segs).cpu().numpy().astype(np.float64)
    want = (native.bidir if op == "bidir" else native.causal)(inp.q, inp.k, inp.v, om)
    err = _rel(got, want)
    print(f"[plan] fp32 {op} segments={segs}: rel L2 {err:.3e}", flush=True)
    assert err <= TOL["f32"]


def test_workspace_follows_plan():
    """A workspace sized for one segment is too small for the default plan:
    the binding sizes it from the plan, and the library refuses a short one."""
    w, inp, om, (q, k, v), om_d = _case("causal_bf16_8k", 64, 256, 1, 2, 2000)
    shp = favor._shape(q, om_d)
    small = torch.empty(favor.workspace_bytes(2, shp, 0, 1), dtype=torch.uint8, device=_dev())
    assert small.numel() < favor.workspace_bytes(2, shp)
    favor.causal(q, k, v, om_d, segments=1, workspace=small)   # enough for one segment
    with pytest.raises(ValueError, match="workspace"):
        favor.causal(q, k, v, om_d, workspace=small)


@pytest.mark.parametrize("d,m,dtype,relu", [(64, 256, "bf16", False), (64, 256, "bf16", True), (128, 256, "bf16", False),
                                              (32, 64, "bf16", False), (32, 64, "f32", False)])
def test_causal_one_segment_per_head(d, m, dtype, relu):
    """Causal calls with one segment per head and no carried state skip the
    merge pass: the scan starts from a zero state with the segment-sum
    pass's key shifts, and that pass packs the projection operands.  256
    heads take that plan automatically; every element against the oracle
    (the tile scan, the d = 128 scan and the generic one), and equal to the
    same call forced to two segments up to rounding."""
    B, H, L = 32, 8, 150
    _, inp, om, (q, k, v), omd = _case("causal_bf16_8k", d, m, B, H, L, dtype=dtype)
    feature = "relu" if relu else "positive"
    got = favor.causal(q, k, v, omd, feature=feature).float()
    two = favor.causal(q, k, v, omd, feature=feature, segments=2).float()
    g = got.cpu().numpy().astype(np.float64)
    want = ref.causal(inp.q, inp.k, inp.v, om, kind="relu") if relu else native.causal(inp.q, inp.k, inp.v, om)
    err, worst = _rel(g, want), _worst_tile(g, want)
    print(f"[plan] causal one segment per head d={d} m={m} {dtype} {feature} {B}x{H}x{L}: rel L2 {err:.3e}, "
          f"worst tile {worst:.3e}", flush=True)
    assert err <= TOL[dtype] and worst <= TOL[dtype]
    assert float((got - two).norm() / two.norm()) <= (1e-2 if dtype == "bf16" else 1e-5)
