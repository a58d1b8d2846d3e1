"""Memory and NaN safety of the kernels on the GPU.

- Canaries: out, workspace and state buffers are sub-views of larger
  allocations whose padding holds a sentinel pattern; after each call at a
  ragged length the padding is unchanged (nothing written out of bounds),
  the inputs are unchanged (nothing written into them), and the result still
  matches the oracle.
- NaN propagation, with positive and with ReLU features: a NaN in one row of
  the inputs gives NaN exactly where the exact formula (the fp64 oracle on
  the same inputs) gives it: a NaN key
  poisons every output of its head that attends to it (bidirectional: all
  rows; causal: rows at or after it), a NaN query only its own row, a NaN in
  one value element that column of the rows that attend to it.  One
  documented exception: in causal attention a non-finite value element also
  reaches the earlier rows of its own scan chunk (same column), because the
  intra-chunk product multiplies the masked score 0 by it (0 * NaN = NaN), as
  in masked matrix-product attention kernels generally.
"""

import ctypes

import numpy as np
import pytest
import torch

import oracle.native as native
import oracle.reference as ref
import positive_random_feature_amd as favor
from positive_random_feature_amd import _lib
from positive_random_feature_amd.workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
PAD = 4096  # elements (bf16/fp32) or bytes (workspace) on each side; keeps every alignment


def _to_dev(inp, dtype):
    if dtype == "bf16":
        return [torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(DEV) for b in (inp.q_bits, inp.k_bits, inp.v_bits)]
    return [torch.from_numpy(a).to(DEV) for a in (inp.q, inp.k, inp.v)]


def _rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def _padded(n, dtype, fill):
    big = torch.empty(n + 2 * PAD, dtype=dtype, device=DEV)
    if dtype == torch.uint8:
        big.fill_(fill)
    else:
        big.view(torch.int16 if dtype == torch.bfloat16 else torch.int32).fill_(fill)
    return big, big[PAD:PAD + n]


def _pads_intact(big, n, fill):
    b = big if big.dtype == torch.uint8 else big.view(torch.int16 if big.dtype == torch.bfloat16 else torch.int32)
    head, tail = b[:PAD], b[PAD + n:]
    return bool((head == fill).all()) and bool((tail == fill).all())


SHAPES = [  # (base workload, d, m, B, H, L, dtype)
    ("causal_bf16_8k", 64, 256, 1, 3, 1000, "bf16"),
    ("causal_bf16_8k", 64, 256, 2, 1, 97, "bf16"),
    ("causal_bf16_8k", 128, 512, 1, 2, 333, "bf16"),
    ("causal_bf16_8k", 32, 64, 1, 2, 65, "bf16"),
    ("bidir_f32_tiny", 16, 32, 1, 2, 131, "f32"),
    ("bidir_f32_tiny", 64, 256, 1, 1, 1, "f32"),
    ("causal_bf16_8k", 32, 32, 1, 2, 300, "bf16"),     # bidirectional: the key-split one-kernel path
    ("causal_bf16_8k", 64, 256, 16, 8, 200, "bf16"),   # bidirectional: the feature-split one-kernel path
]


@pytest.mark.parametrize("base,d,m,B,H,L,dtype", SHAPES)
@pytest.mark.parametrize("op", ["bidir", "causal", "causal_state"])
def test_canaries(base, d, m, B, H, L, dtype, op):
    w = WORKLOADS[base].replace(d=d, m=m, omega_per_head=True)
    inp = make_inputs(w, B=B, H=H, L=L, seed=11)
    om = ref.orf_omega(3, H, m, d)
    q, k, v = _to_dev(inp, dtype)
    om_d = torch.from_numpy(om).to(DEV)
    before = [t.clone() for t in (q, k, v, om_d)]
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    fill = 0x5A5A if dtype == "bf16" else 0x5A5A5A5A
    n = B * H * L * d
    out_big, out_flat = _padded(n, tdt, fill)
    out = out_flat.view(B, H, L, d)
    shp = favor._shape(q, om_d)
    opcode = _lib.FAVOR_OP_BIDIR if op == "bidir" else _lib.FAVOR_OP_CAUSAL
    need = favor.workspace_bytes(opcode, shp)
    ws_big, ws = _padded(need, torch.uint8, 0xA5)
    ws.fill_(0x3C)  # the workspace body: arbitrary contents are allowed
    if op == "bidir":
        favor.bidir(q, k, v, om_d, out=out, workspace=ws)
    elif op == "causal":
        favor.causal(q, k, v, om_d, out=out, workspace=ws)
    else:
        ns = favor.state_floats(m, d)
        st_big, st_flat = _padded(B * H * ns, torch.float32, 0x5A5A5A5A)
        st = st_flat.view(B, H, ns)
        status = _lib.load().favor_causal_state(ctypes.byref(shp), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                                om_d.data_ptr(), out.data_ptr(), 0, None, st.data_ptr(), ws.data_ptr(),
                                                ws.numel(), torch.cuda.current_stream().cuda_stream)
        _lib.check(status, "favor_causal_state")
        torch.cuda.synchronize()
        assert _pads_intact(st_big, B * H * ns, 0x5A5A5A5A), "state_out padding overwritten"
    torch.cuda.synchronize()
    assert _pads_intact(out_big, n, fill), "out padding overwritten"
    assert _pads_intact(ws_big, need, 0xA5), "workspace padding overwritten"
    for a, b in zip(before, (q, k, v, om_d)):
        assert torch.equal(a, b), "an input was modified"
    got = out.float().cpu().numpy().astype(np.float64)
    want = (native.bidir if op == "bidir" else native.causal)(inp.q, inp.k, inp.v, om)
    err = _rel(got, want)
    print(f"[safety] canaries {op} d={d} m={m} {B}x{H}x{L} {dtype}: rel L2 {err:.3e}", flush=True)
    assert err <= (2e-2 if dtype == "bf16" else 1e-5)


def _nan_case(d, m, B, H, L, where, t, col=0):
    w = WORKLOADS["causal_bf16_8k"].replace(d=d, m=m)
    inp = make_inputs(w, B=B, H=H, L=L, seed=8)
    from positive_random_feature_amd.workloads import bf16_bits_to_f32
    bits = {"q": inp.q_bits.copy(), "k": inp.k_bits.copy(), "v": inp.v_bits.copy()}
    if where == "v":
        bits["v"][0, 1, t, col] = 0x7FC0  # one value element of head 1
    else:
        bits[where][0, 1, t, :] = 0x7FC0  # one whole row of head 1
    vals = [bf16_bits_to_f32(bits[x]) for x in "qkv"]
    dev = [torch.from_numpy(bits[x].view(np.int16)).view(torch.bfloat16).to(DEV) for x in "qkv"]
    om = ref.orf_omega(0, H, m, d)
    return vals, dev, om


@pytest.mark.parametrize("d,m", [(64, 256), (128, 512), (32, 64)])
@pytest.mark.parametrize("op", ["bidir", "causal"])
@pytest.mark.parametrize("where,t", [("k", 700), ("k", 0), ("q", 455), ("v", 1234), ("k", 1999)])
def test_nan_propagation(d, m, op, where, t):
    B, H, L = 1, 3, 2000
    vals, dev, om = _nan_case(d, m, B, H, L, where, t, col=d // 2 + 3)
    fn = favor.bidir if op == "bidir" else favor.causal
    got = fn(*dev, torch.from_numpy(om).to(DEV)).float().cpu().numpy().astype(np.float64)
    with np.errstate(invalid="ignore"):
        want = (native.bidir if op == "bidir" else native.causal)(*vals, om)
    nan_want, nan_got = np.isnan(want), np.isnan(got)
    if op == "causal" and where == "v":
        # the documented exception: the masked score times the NaN value
        chunk = 64 if (d, m) == (64, 256) else 32
        c0 = (t // chunk) * chunk
        nan_want = nan_want.copy()
        nan_want[0, 1, c0:t, d // 2 + 3] = True
    print(f"[safety] NaN in {where}[{t}] {op} d={d} m={m}: {int(nan_want.sum())} NaN expected, "
          f"{int(nan_got.sum())} produced", flush=True)
    assert nan_want.any()
    np.testing.assert_array_equal(nan_got, nan_want)
    ok = ~nan_want
    assert np.isfinite(got[ok]).all()
    assert _rel(got[ok], want[ok]) <= 2e-2


@pytest.mark.parametrize("d,m", [(64, 256), (128, 512), (32, 64)])
@pytest.mark.parametrize("op", ["bidir", "causal"])
@pytest.mark.parametrize("where,t", [("k", 700), ("q", 455), ("v", 1234)])
def test_nan_propagation_relu(d, m, op, where, t):
    """ReLU features keep a NaN too: max(NaN, 0) is NaN in the exact formula
    (the numpy oracle's maximum), so a NaN key row spreads as with positive
    features instead of dropping out as a zero feature vector."""
    B, H, L = 1, 3, 2000
    vals, dev, om = _nan_case(d, m, B, H, L, where, t, col=d // 2 + 3)
    fn = favor.bidir if op == "bidir" else favor.causal
    got = fn(*dev, torch.from_numpy(om).to(DEV), feature="relu").float().cpu().numpy().astype(np.float64)
    with np.errstate(invalid="ignore"):
        want = (ref.bidir if op == "bidir" else ref.causal)(*vals, om, kind="relu")
    nan_want, nan_got = np.isnan(want), np.isnan(got)
    if op == "causal" and where == "v":
        chunk = 64 if (d, m) == (64, 256) else 32
        c0 = (t // chunk) * chunk
        nan_want = nan_want.copy()
        nan_want[0, 1, c0:t, d // 2 + 3] = True
    print(f"[safety] NaN in {where}[{t}] {op} relu d={d} m={m}: {int(nan_want.sum())} NaN expected, "
          f"{int(nan_got.sum())} produced", flush=True)
    assert nan_want.any()
    np.testing.assert_array_equal(nan_got, nan_want)
    ok = ~nan_want
    assert np.isfinite(got[ok]).all()
    assert _rel(got[ok], want[ok]) <= 2e-2


@pytest.mark.parametrize("d,m", [(32, 32), (64, 256)])
@pytest.mark.parametrize("where,t", [("k", 300), ("q", 255), ("v", 411)])
def test_nan_propagation_relu_one_kernel(d, m, where, t):
    """ReLU NaN patterns through the one-kernel bidirectional paths."""
    B, H, L = 1, 3, 500
    vals, dev, om = _nan_case(d, m, B, H, L, where, t, col=d // 2 + 3)
    got = favor.bidir(*dev, torch.from_numpy(om).to(DEV), feature="relu", segments=1)
    got = got.float().cpu().numpy().astype(np.float64)
    with np.errstate(invalid="ignore"):
        want = ref.bidir(*vals, om, kind="relu")
    nan_want, nan_got = np.isnan(want), np.isnan(got)
    print(f"[safety] NaN in {where}[{t}] one-kernel bidir relu d={d} m={m}: {int(nan_want.sum())} NaN expected, "
          f"{int(nan_got.sum())} produced", flush=True)
    assert nan_want.any()
    np.testing.assert_array_equal(nan_got, nan_want)
    ok = ~nan_want
    assert np.isfinite(got[ok]).all()
    assert _rel(got[ok], want[ok]) <= 2e-2


@pytest.mark.parametrize("d,m", [(32, 32), (64, 256)])
@pytest.mark.parametrize("where,t", [("k", 300), ("k", 0), ("q", 255), ("v", 411), ("k", 499)])
def test_nan_propagation_one_kernel(d, m, where, t):
    """The same NaN pattern through the one-kernel bidirectional paths (a
    one-segment plan: m = 32 runs the key-split kernel, m = 256 the
    feature-split one): a NaN key reaches every row of its head, a NaN query
    only its row, a NaN value that column of every row."""
    B, H, L = 1, 3, 500
    vals, dev, om = _nan_case(d, m, B, H, L, where, t, col=d // 2 + 3)
    got = favor.bidir(*dev, torch.from_numpy(om).to(DEV), segments=1).float().cpu().numpy().astype(np.float64)
    with np.errstate(invalid="ignore"):
        want = native.bidir(*vals, om)
    nan_want, nan_got = np.isnan(want), np.isnan(got)
    print(f"[safety] NaN in {where}[{t}] one-kernel bidir d={d} m={m}: {int(nan_want.sum())} NaN expected, "
          f"{int(nan_got.sum())} produced", flush=True)
    assert nan_want.any()
    np.testing.assert_array_equal(nan_got, nan_want)
    ok = ~nan_want
    assert np.isfinite(got[ok]).all()
    assert _rel(got[ok], want[ok]) <= 2e-2


@pytest.mark.parametrize("feature", ["positive", "relu"])
@pytest.mark.parametrize("api", ["dense", "hadamard"])
@pytest.mark.parametrize("stabilize", [False, True])
def test_nan_propagation_features(feature, api, stabilize):
    """One NaN element of x makes that row's features NaN (every projection
    of the row involves it) and leaves every other row finite, as in the
    exact formula."""
    B, H, L, d, m = 1, 2, 100, 64, 256
    w = WORKLOADS["causal_bf16_8k"].replace(d=d, m=m)
    inp = make_inputs(w, B=B, H=H, L=L, seed=5)
    bits = inp.q_bits.copy()
    bits[0, 1, 37, 11] = 0x7FC0
    x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    if api == "dense":
        om = torch.from_numpy(ref.orf_omega(2, H, m, d)).to(DEV)
        phi, _ = favor.features(x, om, stabilize=stabilize, feature=feature)
    else:
        phi, _ = favor.features_hadamard(x, 2, m, stabilize=stabilize, feature=feature)
    phi = phi.cpu().numpy()
    nan = np.isnan(phi)
    print(f"[safety] NaN in x features {feature} {api} stabilize={stabilize}: {int(nan.sum())} NaN "
          f"(expected {m})", flush=True)
    want = np.zeros_like(nan)
    want[0, 1, 37, :] = True
    np.testing.assert_array_equal(nan, want)
    assert np.isfinite(phi[~want]).all()
