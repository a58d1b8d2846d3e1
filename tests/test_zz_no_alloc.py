"""favor_causal_noalloc, the causal entry point that allocates nothing (its
workspace is the library's static per-GPU scratch array), against
favor_causal with a caller-allocated workspace on the same inputs.  Both run
the same kernels with the same launch plan, so the outputs must be
bit-identical (hence within the 2e-2 bf16 / 1e-5 fp32 bar); checked on
several calls in a row, each later one smaller than the first, so that a
stale scratch from the previous call would show."""

import ctypes

import numpy as np
import pytest
import torch

import oracle.reference as ref
import positive_random_feature_amd as favor
from positive_random_feature_amd import _lib
from positive_random_feature_amd.workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _case(name, B, H, L, d=None, m=None, seed=None):
    w = WORKLOADS[name]
    if d is not None:
        w = w.replace(d=d, m=m, omega_per_head=True)
    inp = make_inputs(w, B=B, H=H, L=L, seed=seed)
    om = ref.orf_omega(5, H, w.m, w.d)
    if w.dtype == "bf16":
        t = [torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(DEV) for b in (inp.q_bits, inp.k_bits, inp.v_bits)]
    else:
        t = [torch.from_numpy(a).to(DEV) for a in (inp.q, inp.k, inp.v)]
    return w, t, torch.from_numpy(om).to(DEV)


def _rel(a, b):
    return float((a.double() - b.double()).norm() / b.double().norm())


# (workload, B, H, L, d, m, chunk): the first call is the largest
CALLS = [
    ("causal_bf16_8k", 2, 8, 8192, None, None, 0),    # 2 x 8 x 8192, d 64, m 256: ~34 MB of scratch
    ("causal_bf16_8k", 1, 2, 1000, None, None, 0),    # smaller, same path
    ("causal_bf16_8k", 1, 3, 777, None, None, 32),    # 32-token chunks
    ("causal_bf16_8k", 1, 2, 333, 128, 512, 0),       # the d = 128 scan
    ("bidir_f32_tiny", 1, 1, 256, None, None, 0),     # fp32
]


def test_noalloc_matches_causal_on_consecutive_calls():
    for i, (name, B, H, L, d, m, chunk) in enumerate(CALLS):
        w, (q, k, v), om = _case(name, B, H, L, d, m, seed=20 + i)
        print(f"[noalloc] call {i}: {name} {B}x{H}x{L} d={w.d} m={w.m} chunk={chunk}", flush=True)
        want = favor.causal(q, k, v, om, chunk=chunk)
        out = torch.full_like(q, float("nan"))
        favor.causal_noalloc(q, k, v, om, out, chunk=chunk)
        torch.cuda.synchronize()
        tol = 2e-2 if w.dtype == "bf16" else 1e-5
        err = _rel(out, want)
        print(f"[noalloc] call {i}: rel L2 against favor_causal {err:.3e} (bar {tol}), "
              f"bit-identical {torch.equal(out, want)}", flush=True)
        assert err <= tol
        assert torch.equal(out, want)


def test_noalloc_rejects_shapes_beyond_the_scratch():
    """A shape whose workspace exceeds the scratch array is refused with
    FAVOR_ERR_WORKSPACE before anything is launched (the output keeps its
    contents)."""
    lib = _lib.load()
    shp = _lib.shape(1, 256, 128, 128, 512, _lib.FAVOR_BF16, 512 * 128)
    need = lib.favor_workspace_bytes(_lib.FAVOR_OP_CAUSAL, ctypes.byref(shp), 0)
    assert need > _lib.FAVOR_NOALLOC_SCRATCH_BYTES
    q = torch.zeros(1, 256, 128, 128, dtype=torch.bfloat16, device=DEV)
    om = torch.zeros(256, 512, 128, device=DEV)
    out = torch.full_like(q, 7.0)
    with pytest.raises(favor.FavorError) as e:
        favor.causal_noalloc(q, q, q, om, out)
    assert e.value.status == 3
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
