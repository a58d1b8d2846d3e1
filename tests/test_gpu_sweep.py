"""GPU parity over a seeded random sweep of the supported shapes.

Each case draws the input dtype, head size d, feature count m, operation
(bidirectional or causal), feature map (positive or ReLU), batch, heads, a
ragged sequence length and whether the projection is shared or per head, and
compares every output element with the fp64 oracle.  The draws reach every
launch plan of the library (the 64-token tile scan, the two-workgroup d = 128
scan and the generic chunk scan for causal attention; the output pass with
its operands in LDS or read from memory) at lengths that are not multiples of
the tile sizes.  Further draws take lengths at and around the tile, chunk
and segment edges with forced chunk lengths and segment counts, and cut
causal sequences in two calls that carry the state across the cut.  Bar as
in the other parity tests: relative L2 1e-5 for fp32 inputs, 2e-2 for bf16
inputs, for the whole output and for every head.
"""

import numpy as np
import pytest
import torch

import oracle.native as native
import oracle.reference as ref
import positive_random_feature_amd as favor
from positive_random_feature_amd.workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}
N_CASES = 40


def _draw_cases(n, seed=20261202):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dtype = str(rng.choice(["bf16", "bf16", "f32"]))
        d = int(rng.choice([16, 32, 64, 128] if dtype == "bf16" else [16, 32, 64]))
        op = str(rng.choice(["bidir", "causal"]))
        feature = str(rng.choice(["positive", "positive", "relu"]))
        if op == "causal":
            ms = [32, 64, 128, 256, 512]
            if dtype == "f32" and d == 64:
                ms = ms[:-1]
        else:
            ms = list(range(32, 257, 32)) + [320, 384, 448, 512]
        m = int(rng.choice(ms))
        B = int(rng.integers(1, 3))
        H = int(rng.integers(1, 4))
        # the ReLU causal oracle walks the tokens in Python: shorter sequences
        L = int(rng.integers(1, 400 if (feature == "relu" and op == "causal") else 1200))
        per_head = bool(rng.integers(0, 2))
        cases.append((i, dtype, d, m, op, feature, B, H, L, per_head))
    return cases


CASES = _draw_cases(N_CASES)


def _id(c):
    i, dtype, d, m, op, feature, B, H, L, per_head = c
    return f"{i}-{op}-{feature}-{dtype}-d{d}-m{m}-{B}x{H}x{L}-{'perhead' if per_head else 'shared'}"


def _to_dev(inp, dtype, dev):
    if dtype == "bf16":
        return [torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(dev) for b in (inp.q_bits, inp.k_bits, inp.v_bits)]
    return [torch.from_numpy(a).to(dev) for a in (inp.q, inp.k, inp.v)]


@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_random_shape(case):
    i, dtype, d, m, op, feature, B, H, L, per_head = case
    print(f"[sweep] {_id(case)}", flush=True)
    base = WORKLOADS["causal_bf16_8k" if dtype == "bf16" else "bidir_f32_tiny"]
    w = base.replace(d=d, m=m, omega_per_head=per_head)
    inp = make_inputs(w, B=B, H=H, L=L, seed=5000 + i)
    om = ref.orf_omega(7000 + i, H if per_head else 1, m, d)
    om = om if per_head else om[0]
    dev = torch.device("cuda:0")
    q, k, v = _to_dev(inp, dtype, dev)
    fn = favor.bidir if op == "bidir" else favor.causal
    got = fn(q, k, v, torch.from_numpy(om).to(dev), feature=feature)
    torch.cuda.synchronize()
    got = got.float().cpu().numpy().astype(np.float64)
    if feature == "positive":
        want = (native.bidir if op == "bidir" else native.causal)(inp.q, inp.k, inp.v, om)
    else:
        want = (ref.bidir if op == "bidir" else ref.causal)(inp.q, inp.k, inp.v, om, kind="relu")
    assert np.isfinite(want).all()
    err = float(np.linalg.norm(got - want) / np.linalg.norm(want))
    print(f"[sweep] {_id(case)}: rel L2 {err:.3e} (tol {TOL[dtype]})", flush=True)
    assert err <= TOL[dtype]


def _draw_many_head_cases(n, seed=20261203):
    """Bidirectional calls with many heads of short sequences: the range where
    the automatic plan gives each head one segment and the call runs as one
    kernel (key-split for m = 32, feature-split where its operands fit), and
    just around it."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dtype = str(rng.choice(["bf16", "bf16", "f32"]))
        d = int(rng.choice([16, 32, 64, 128] if dtype == "bf16" else [16, 32, 64]))
        feature = str(rng.choice(["positive", "positive", "relu"]))
        m = int(rng.choice([32, 32, 64, 128, 256]))
        B = int(rng.integers(8, 40))
        H = int(rng.integers(8, 9))
        L = int(rng.integers(1, 640))
        per_head = bool(rng.integers(0, 2))
        cases.append((100 + i, dtype, d, m, "bidir", feature, B, H, L, per_head))
    return cases


MANY_HEAD_CASES = _draw_many_head_cases(16)


@pytest.mark.parametrize("case", MANY_HEAD_CASES, ids=[_id(c) for c in MANY_HEAD_CASES])
def test_random_many_head_shape(case):
    test_random_shape(case)


_BOUNDARY_LENGTHS = [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 383, 384, 385,
                     511, 512, 513, 1023, 1024, 1025]


def _draw_plan_cases(n, seed=20261204):
    """Lengths at and around the 16-, 32- and 64-token tiles, chunks and
    segment edges, with the chunk length and the segment count drawn as
    well (forced plans, as a caller may choose them), every element
    against the oracle."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dtype = str(rng.choice(["bf16", "bf16", "f32"]))
        d = int(rng.choice([16, 32, 64, 128] if dtype == "bf16" else [16, 32, 64]))
        op = str(rng.choice(["bidir", "causal"]))
        feature = str(rng.choice(["positive", "positive", "relu"]))
        if op == "causal":
            ms = [32, 64, 128, 256, 512]
            if dtype == "f32" and d == 64:
                ms = ms[:-1]
        else:
            ms = list(range(32, 257, 32)) + [320, 384, 448, 512]
        m = int(rng.choice(ms))
        B = int(rng.integers(1, 3))
        H = int(rng.integers(1, 4))
        L = int(rng.choice(_BOUNDARY_LENGTHS))
        per_head = bool(rng.integers(0, 2))
        chunk = 0
        if op == "causal":
            chunk = int(rng.choice([0, 32] + ([64] if (dtype == "bf16" and d == 64 and m in (64, 128, 256)) else [])))
        segments = int(rng.choice([0, int(rng.integers(1, 41))]))
        cases.append((200 + i, dtype, d, m, op, feature, B, H, L, per_head, chunk, segments))
    return cases


PLAN_CASES = _draw_plan_cases(48)


def _plan_id(c):
    return _id(c[:10]) + f"-chunk{c[10]}-seg{c[11]}"


@pytest.mark.parametrize("case", PLAN_CASES, ids=[_plan_id(c) for c in PLAN_CASES])
def test_random_boundary_length_and_plan(case):
    i, dtype, d, m, op, feature, B, H, L, per_head, chunk, segments = case
    print(f"[sweep] {_plan_id(case)}", flush=True)
    base = WORKLOADS["causal_bf16_8k" if dtype == "bf16" else "bidir_f32_tiny"]
    w = base.replace(d=d, m=m, omega_per_head=per_head)
    inp = make_inputs(w, B=B, H=H, L=L, seed=5000 + i)
    om = ref.orf_omega(7000 + i, H if per_head else 1, m, d)
    om = om if per_head else om[0]
    dev = torch.device("cuda:0")
    q, k, v = _to_dev(inp, dtype, dev)
    omd = torch.from_numpy(np.ascontiguousarray(om)).to(dev)
    if op == "bidir":
        got = favor.bidir(q, k, v, omd, feature=feature, segments=segments)
    else:
        got = favor.causal(q, k, v, omd, chunk=chunk, feature=feature, segments=segments)
    torch.cuda.synchronize()
    got = got.float().cpu().numpy().astype(np.float64)
    if feature == "positive":
        want = (native.bidir if op == "bidir" else native.causal)(inp.q, inp.k, inp.v, om)
    else:
        want = (ref.bidir if op == "bidir" else ref.causal)(inp.q, inp.k, inp.v, om, kind="relu")
    assert np.isfinite(want).all()
    err = float(np.linalg.norm(got - want) / np.linalg.norm(want))
    worst = max(float(np.linalg.norm(got[b, h] - want[b, h]) / np.linalg.norm(want[b, h]))
                for b in range(B) for h in range(H))
    print(f"[sweep] {_plan_id(case)}: rel L2 {err:.3e}, worst head {worst:.3e} (tol {TOL[dtype]})", flush=True)
    assert err <= TOL[dtype] and worst <= TOL[dtype]


def _draw_split_cases(n, seed=20261205):
    """Sequences cut at a random point and run as two calls that carry the
    state across the cut: the concatenated outputs against the oracle's
    single pass over the whole sequence."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dtype = str(rng.choice(["bf16", "bf16", "f32"]))
        d = int(rng.choice([16, 32, 64, 128] if dtype == "bf16" else [16, 32, 64]))
        ms = [32, 64, 128, 256, 512]
        if dtype == "f32" and d == 64:
            ms = ms[:-1]
        m = int(rng.choice(ms))
        B = int(rng.integers(1, 3))
        H = int(rng.integers(1, 4))
        L = int(rng.integers(2, 2500))
        split = int(rng.integers(1, L))
        per_head = bool(rng.integers(0, 2))
        chunk = int(rng.choice([0, 32] + ([64] if (dtype == "bf16" and d == 64 and m in (64, 128, 256)) else [])))
        cases.append((300 + i, dtype, d, m, B, H, L, split, per_head, chunk))
    return cases


SPLIT_CASES = _draw_split_cases(24)


def _split_id(c):
    i, dtype, d, m, B, H, L, split, per_head, chunk = c
    return f"{i}-{dtype}-d{d}-m{m}-{B}x{H}x{L}-cut{split}-{'perhead' if per_head else 'shared'}-chunk{chunk}"


@pytest.mark.parametrize("case", SPLIT_CASES, ids=[_split_id(c) for c in SPLIT_CASES])
def test_random_carried_state_split(case):
    i, dtype, d, m, B, H, L, split, per_head, chunk = case
    print(f"[sweep] {_split_id(case)}", flush=True)
    base = WORKLOADS["causal_bf16_8k" if dtype == "bf16" else "bidir_f32_tiny"]
    w = base.replace(d=d, m=m, omega_per_head=per_head)
    inp = make_inputs(w, B=B, H=H, L=L, seed=6000 + i)
    om = ref.orf_omega(8000 + i, H if per_head else 1, m, d)
    om = om if per_head else om[0]
    dev = torch.device("cuda:0")
    q, k, v = _to_dev(inp, dtype, dev)
    omd = torch.from_numpy(np.ascontiguousarray(om)).to(dev)
    first, state = favor.causal(*(x[:, :, :split].contiguous() for x in (q, k, v)), omd, chunk=chunk,
                                return_state=True)
    second = favor.causal(*(x[:, :, split:].contiguous() for x in (q, k, v)), omd, chunk=chunk, state=state)
    torch.cuda.synchronize()
    got = torch.cat([first, second], dim=2).float().cpu().numpy().astype(np.float64)
    want = native.causal(inp.q, inp.k, inp.v, om)
    err = float(np.linalg.norm(got - want) / np.linalg.norm(want))
    worst = max(float(np.linalg.norm(got[b, h] - want[b, h]) / np.linalg.norm(want[b, h]))
                for b in range(B) for h in range(H))
    print(f"[sweep] {_split_id(case)}: rel L2 {err:.3e}, worst head {worst:.3e} (tol {TOL[dtype]})", flush=True)
    assert err <= TOL[dtype] and worst <= TOL[dtype]
