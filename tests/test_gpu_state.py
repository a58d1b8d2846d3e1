"""GPU parity of causal FAVOR+ with a carried prefix state (favor_causal_state
through the C ABI) against the fp64 oracle: a sequence processed in pieces,
each call continuing from the previous call's state, matches the oracle's
single pass, and the returned state matches the oracle's prefix sums.

Bar (relative L2): 1e-5 for fp32 inputs, 2e-2 for bf16 inputs."""

import math

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


def _rel(got, want):
    return float(np.linalg.norm(got - want) / np.linalg.norm(want))


def _true_state(st, m, d):
    """(G, z) in true units from a library state tensor."""
    S, z, s = favor.state_parts(st.double().cpu(), m, d)
    scale = torch.exp(s)[..., None]
    return (S * scale[..., None]).numpy(), (z * scale).numpy()


def _log(name, err, tol):
    print(f"[state] {name}: rel L2 {err:.3e} (tol {tol})", flush=True)


CASES = [("bf16", 64, 256), ("bf16", 128, 512), ("bf16", 32, 64), ("bf16", 128, 256), ("f32", 32, 64),
         ("f32", 64, 256)]


@pytest.mark.parametrize("dtype,d,m", CASES)
@pytest.mark.parametrize("splits", [(357,), (64, 700), (1, 2, 999)])
def test_pieces_continue_the_sequence(dtype, d, m, splits):
    base = WORKLOADS["causal_bf16_8k" if dtype == "bf16" else "bidir_f32_tiny"]
    w = base.replace(d=d, m=m, omega_per_head=True)
    B, H, L = 1, 2, 1000
    inp = make_inputs(w, B=B, H=H, L=L)
    om = ref.orf_omega(w.seed, H, m, d)
    q, k, v = _to_dev(inp, dtype)
    om_t = torch.from_numpy(om).to(_dev())
    cuts = [0, *splits, L]
    outs, st = [], None
    for a, b in zip(cuts[:-1], cuts[1:]):
        o, st = favor.causal(q[:, :, a:b].contiguous(), k[:, :, a:b].contiguous(), v[:, :, a:b].contiguous(), om_t,
                             state=st, return_state=True)
        outs.append(o)
    torch.cuda.synchronize()
    got = torch.cat(outs, dim=2).float().cpu().numpy().astype(np.float64)
    want = native.causal(inp.q, inp.k, inp.v, om)
    err = _rel(got, want)
    _log(f"{dtype} d={d} m={m} pieces {cuts}", err, TOL[dtype])
    assert err <= TOL[dtype]
    _, (G, z) = ref.causal_with_state(inp.q, inp.k, inp.v, om)
    Gg, zg = _true_state(st, m, d)
    eg, ez = _rel(Gg, G), _rel(zg, z)
    _log(f"{dtype} d={d} m={m} final state G, z", max(eg, ez), TOL[dtype])
    assert eg <= TOL[dtype] and ez <= TOL[dtype]


@pytest.mark.parametrize("d,m", [(64, 256), (128, 512), (32, 64)])
def test_state_in_from_the_oracle(d, m):
    """A state built by the oracle from a prefix of keys (stored with a
    shift), continued on the GPU, gives the oracle's continuation."""
    w = WORKLOADS["causal_bf16_8k"].replace(d=d, m=m, omega_per_head=True)
    B, H, Lp, L = 1, 2, 300, 500
    inp = make_inputs(w, B=B, H=H, L=Lp + L, seed=3)
    om = ref.orf_omega(w.seed, H, m, d)
    pre = [a[:, :, :Lp] for a in (inp.q, inp.k, inp.v)]
    post = [a[:, :, Lp:] for a in (inp.q, inp.k, inp.v)]
    _, (G, z) = ref.causal_with_state(*pre, om)
    want, _ = ref.causal_with_state(*post, om, (G, z))
    shift = np.log(np.max(z, axis=-1))  # store relative to the largest z
    st = np.concatenate([(G / np.exp(shift)[..., None, None]).reshape(B, H, m * d),
                         z / np.exp(shift)[..., None], shift[..., None]], axis=-1).astype(np.float32)
    q, k, v = _to_dev(inp, "bf16")
    om_t = torch.from_numpy(om).to(_dev())
    out = favor.causal(q[:, :, Lp:].contiguous(), k[:, :, Lp:].contiguous(), v[:, :, Lp:].contiguous(), om_t,
                       state=torch.from_numpy(st).to(_dev()))
    torch.cuda.synchronize()
    err = _rel(out.float().cpu().numpy().astype(np.float64), want)
    _log(f"state from the oracle d={d} m={m}", err, 2e-2)
    assert err <= 2e-2


def test_state_large_norms():
    """Entries of q, k at 3 d^-1/4 (exponents far outside fp32 range without
    shifts), three pieces."""
    w = WORKLOADS["causal_bf16_8k"].replace(qk_scale=3.0)
    B, H, L = 1, 2, 900
    inp = make_inputs(w, B=B, H=H, L=L)
    om = ref.orf_omega(w.seed, H, w.m, w.d)
    q, k, v = _to_dev(inp, "bf16")
    om_t = torch.from_numpy(om).to(_dev())
    outs, st = [], None
    for a, b in ((0, 200), (200, 650), (650, 900)):
        o, st = favor.causal(q[:, :, a:b].contiguous(), k[:, :, a:b].contiguous(), v[:, :, a:b].contiguous(), om_t,
                             state=st, return_state=True)
        outs.append(o)
    torch.cuda.synchronize()
    got = torch.cat(outs, dim=2).float().cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    err = _rel(got, native.causal(inp.q, inp.k, inp.v, om))
    _log("large-norm pieces", err, 2e-2)
    assert err <= 2e-2
    S, z, s = favor.state_parts(st.cpu(), w.m, w.d)
    assert torch.isfinite(S).all() and torch.isfinite(z).all() and torch.isfinite(s).all()


def test_state_matches_plain_call():
    """Without a state in, favor_causal_state gives favor_causal's output bit
    for bit (same kernels, same plan)."""
    w = WORKLOADS["causal_bf16_8k"]
    inp = make_inputs(w, B=2, H=8, L=2000)
    om = ref.orf_omega(w.seed, 8, w.m, w.d)
    q, k, v = _to_dev(inp, "bf16")
    om_t = torch.from_numpy(om).to(_dev())
    a = favor.causal(q, k, v, om_t)
    b, st = favor.causal(q, k, v, om_t, return_state=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert math.isfinite(float(st[..., -1].max()))


# Every configuration of the one-launch path for calls of at most 32 tokens
# per head that carry a state (features per wave x waves: 32 x 1, 64 x 1..8,
# 32 x 2..4 for bf16 d = 128, 32 x 2..8 for fp32 d = 64), d = 16 with its
# split projection operand, and shapes without that path (bf16, d = 128,
# m = 256 and 512), which keep the three kernels.
DECODE_CASES = [("bf16", 16, 32), ("bf16", 16, 512), ("bf16", 32, 64), ("bf16", 64, 64), ("bf16", 64, 128),
                ("bf16", 64, 256), ("bf16", 64, 512), ("bf16", 128, 64), ("bf16", 128, 128), ("bf16", 128, 256),
                ("bf16", 128, 512), ("f32", 16, 128), ("f32", 32, 512), ("f32", 64, 64), ("f32", 64, 128),
                ("f32", 64, 256)]


@pytest.mark.parametrize("dtype,d,m", DECODE_CASES)
def test_decode_steps(dtype, d, m):
    """A prefix in one call, then decode steps of 1 token (and a few of 2 to
    32) per call, each continuing from the previous state, for 32 heads: the
    outputs match the oracle's single pass and the final state its prefix
    sums."""
    base = WORKLOADS["causal_bf16_8k" if dtype == "bf16" else "bidir_f32_tiny"]
    w = base.replace(d=d, m=m, omega_per_head=True)
    B, H = 4, 8
    steps = [50] + [1] * 12 + [17, 32, 1, 5, 2]
    L = sum(steps)
    inp = make_inputs(w, B=B, H=H, L=L, seed=d + m)
    om = ref.orf_omega(7 + d + m, H, m, d)
    q, k, v = _to_dev(inp, dtype)
    om_t = torch.from_numpy(om).to(_dev())
    outs, st, t = [], None, 0
    for n in steps:
        o, st = favor.causal(q[:, :, t:t + n].contiguous(), k[:, :, t:t + n].contiguous(),
                             v[:, :, t:t + n].contiguous(), om_t, state=st, return_state=True)
        outs.append(o)
        t += n
    torch.cuda.synchronize()
    got = torch.cat(outs, dim=2).float().cpu().numpy().astype(np.float64)
    want = native.causal(inp.q, inp.k, inp.v, om)
    err = _rel(got, want)
    worst = max(_rel(got[b, h], want[b, h]) for b in range(B) for h in range(H))
    _log(f"decode steps {dtype} d={d} m={m}: worst head {worst:.3e}, whole", err, TOL[dtype])
    assert err <= TOL[dtype] and worst <= TOL[dtype]
    _, (G, z) = ref.causal_with_state(inp.q, inp.k, inp.v, om)
    Gg, zg = _true_state(st, m, d)
    eg, ez = _rel(Gg, G), _rel(zg, z)
    _log(f"decode steps {dtype} d={d} m={m} final state G, z", max(eg, ez), TOL[dtype])
    assert eg <= TOL[dtype] and ez <= TOL[dtype]


def test_decode_large_norms():
    """Decode steps with entries of q, k at 3 d^-1/4: keys that raise the
    shift far above the carried one, rescaling the state each step."""
    w = WORKLOADS["causal_bf16_8k"].replace(qk_scale=3.0, omega_per_head=True)
    B, H = 2, 8
    steps = [3] + [1] * 20 + [32]
    L = sum(steps)
    inp = make_inputs(w, B=B, H=H, L=L, seed=5)
    om = ref.orf_omega(w.seed, H, w.m, w.d)
    q, k, v = _to_dev(inp, "bf16")
    om_t = torch.from_numpy(om).to(_dev())
    outs, st, t = [], None, 0
    for n in steps:
        o, st = favor.causal(q[:, :, t:t + n].contiguous(), k[:, :, t:t + n].contiguous(),
                             v[:, :, t:t + n].contiguous(), om_t, state=st, return_state=True)
        outs.append(o)
        t += n
    torch.cuda.synchronize()
    got = torch.cat(outs, dim=2).float().cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    err = _rel(got, native.causal(inp.q, inp.k, inp.v, om))
    _log("large-norm decode steps", err, 2e-2)
    assert err <= 2e-2
    S, z, s = favor.state_parts(st.cpu(), w.m, w.d)
    assert torch.isfinite(S).all() and torch.isfinite(z).all() and torch.isfinite(s).all()


def test_decode_first_and_last_call():
    """A first call with no state in (state out only) and a last call with no
    state out, both of a few tokens, against the oracle."""
    w = WORKLOADS["causal_bf16_8k"].replace(omega_per_head=True)
    B, H = 3, 4
    inp = make_inputs(w, B=B, H=H, L=37, seed=9)
    om = ref.orf_omega(w.seed, H, w.m, w.d)
    q, k, v = _to_dev(inp, "bf16")
    om_t = torch.from_numpy(om).to(_dev())
    a, st = favor.causal(q[:, :, :7].contiguous(), k[:, :, :7].contiguous(), v[:, :, :7].contiguous(), om_t,
                         return_state=True)
    b = favor.causal(q[:, :, 7:].contiguous(), k[:, :, 7:].contiguous(), v[:, :, 7:].contiguous(), om_t, state=st)
    torch.cuda.synchronize()
    got = torch.cat([a, b], dim=2).float().cpu().numpy().astype(np.float64)
    err = _rel(got, native.causal(inp.q, inp.k, inp.v, om))
    _log("decode first and last call", err, 2e-2)
    assert err <= 2e-2
