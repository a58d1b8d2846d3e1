"""GPU parity of the generalised (ReLU) features, phi(x) = m^-1/2 max(omega.x, 0)
(FAVOR+ with the ReLU kernel function, the "Performer-ReLU" of the pages),
through the C ABI against the fp64 oracle, on every kernel path: the d = 64
tile scan, the d = 128 scan, the generic chunk scan, fp32, and the features
entry point.  Bar (relative L2): 1e-5 for fp32 inputs, 2e-2 for bf16."""

import numpy as np
import pytest
import torch

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


def _rel(got, want):
    return float(np.linalg.norm(got - want) / np.linalg.norm(want))


def _log(name, err, tol):
    print(f"[relu] {name}: rel L2 {err:.3e} (tol {tol})", flush=True)


SHAPES = [("bf16", 64, 256), ("bf16", 64, 128), ("bf16", 128, 512), ("bf16", 128, 256), ("bf16", 32, 64),
          ("bf16", 16, 32), ("bf16", 64, 512), ("f32", 32, 64), ("f32", 16, 32), ("f32", 64, 256)]


@pytest.mark.parametrize("dtype,d,m", SHAPES)
@pytest.mark.parametrize("op", ["bidir", "causal"])
@pytest.mark.parametrize("B,H,L", [(1, 2, 333), (2, 8, 1000)])
def test_relu_every_element(dtype, d, m, op, B, H, L):
    base = WORKLOADS["causal_bf16_8k" if dtype == "bf16" else "bidir_f32_tiny"]
    w = base.replace(d=d, m=m, omega_per_head=True)
    inp = make_inputs(w, B=B, H=H, L=L)
    om = ref.orf_omega(w.seed, H, m, d)
    q, k, v = _to_dev(inp, dtype)
    fn = favor.bidir if op == "bidir" else favor.causal
    got = fn(q, k, v, torch.from_numpy(om).to(_dev()), feature="relu")
    torch.cuda.synchronize()
    got = got.float().cpu().numpy().astype(np.float64)
    want = (ref.bidir if op == "bidir" else ref.causal)(inp.q, inp.k, inp.v, om, kind="relu")
    err = _rel(got, want)
    _log(f"{op} {dtype} d={d} m={m} {B}x{H}x{L}", err, TOL[dtype])
    assert err <= TOL[dtype]


@pytest.mark.parametrize("name", ["bidir_bf16_4k", "causal_bf16_8k", "causal_bf16_64k"])
def test_relu_full_size_sampled(name):
    """Full-size workloads with ReLU features; the oracle evaluates sampled
    rows of a few heads one by one."""
    w = WORKLOADS[name]
    inp = make_inputs(w)
    om = ref.orf_omega(w.seed, w.H if w.omega_per_head else 1, w.m, w.d)
    om_dev = om if w.omega_per_head else om[0]
    q, k, v = _to_dev(inp, w.dtype)
    fn = favor.bidir if w.op == "bidir" else favor.causal
    got = fn(q, k, v, torch.from_numpy(om_dev).to(_dev()), feature="relu")
    torch.cuda.synchronize()
    got = got.float().cpu().numpy()
    assert np.isfinite(got).all()
    rng = np.random.default_rng(9)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 511, 512, w.L - 1], rng.integers(0, w.L, size=24)]))
    rows_fn = ref.bidir_rows if w.op == "bidir" else ref.causal_rows
    errs = []
    for b, h in ((0, 0), (w.B - 1, w.H - 1), (0, w.H // 2)):
        omh = om[h] if w.omega_per_head else om[0]
        want = rows_fn(inp.q[b, h], inp.k[b, h], inp.v[b, h], omh, rows, kind="relu")
        errs.append(_rel(got[b, h, rows].astype(np.float64), want))
    _log(f"{name} sampled", max(errs), TOL[w.dtype])
    assert max(errs) <= TOL[w.dtype]


@pytest.mark.parametrize("dtype,d,m", [("bf16", 64, 256), ("f32", 16, 32), ("bf16", 128, 512)])
def test_relu_features_entry_point(dtype, d, m):
    base = WORKLOADS["causal_bf16_8k" if dtype == "bf16" else "bidir_f32_tiny"]
    w = base.replace(d=d, m=m, omega_per_head=True)
    inp = make_inputs(w, B=1, H=2, L=77)
    om = ref.orf_omega(w.seed, 2, m, d)
    x = _to_dev(inp, dtype)[0]
    phi, ls = favor.features(x, torch.from_numpy(om).to(_dev()), stabilize=True, feature="relu")
    torch.cuda.synchronize()
    want = np.stack([ref.features_relu(inp.q[0, h], om[h]) for h in range(2)])[None]
    err = _rel(phi.cpu().numpy().astype(np.float64), want)
    _log(f"features {dtype} d={d} m={m}", err, TOL[dtype])
    assert err <= TOL[dtype]
    assert torch.count_nonzero(ls).item() == 0
