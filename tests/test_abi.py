"""C-ABI contract tests that run without a GPU: the library loads, exports
every entry point the header declares, validates arguments before any HIP
call, and its host-side projection generator matches the oracle's."""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle.reference as ref
from positive_random_feature_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3

# fake, 256-byte-aligned device addresses: validation rejects the call before
# any of them is touched
P_Q, P_K, P_V, P_O, P_OM, P_WS = (0x10000000 * (i + 1) for i in range(6))
P_S1, P_S2 = 0x70000000, 0x78000000  # fake state buffers, far from the others


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from positive_random_feature_amd import build
        build.build()
    return _lib.load()


def shp(B=1, H=2, L=64, d=64, m=256, dtype=_lib.FAVOR_BF16, stride=0, feature=_lib.FAVOR_FEATURE_POSITIVE):
    return _lib.shape(B, H, L, d, m, dtype, stride, feature)


def test_exports_every_declared_symbol(lib):
    header = open(os.path.join(ROOT, "include", "favor.h")).read()
    names = set(re.findall(r"\b(favor_[a-z_]+)\s*\(", header))
    assert {"favor_features", "favor_bidir", "favor_causal", "favor_workspace_bytes", "favor_orf_omega",
            "favor_status_string"} <= names
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code in range(5):
        assert lib.favor_status_string(code)
    assert lib.favor_status_string(0) == b"ok"


def test_workspace_bytes(lib):
    s = shp()
    for op in (0, 1, 2):
        assert lib.favor_workspace_bytes(op, ctypes.byref(s), 0) > 0
    assert lib.favor_workspace_bytes(7, ctypes.byref(s), 0) == 0
    assert lib.favor_workspace_bytes(1, ctypes.byref(shp(d=48)), 0) == 0
    assert lib.favor_workspace_bytes(1, None, 0) == 0
    # grows with the number of heads
    assert lib.favor_workspace_bytes(2, ctypes.byref(shp(H=8)), 0) > lib.favor_workspace_bytes(2, ctypes.byref(s), 0)


def _bidir(lib, s, q=P_Q, k=P_K, v=P_V, om=P_OM, o=P_O, ws=P_WS, nbytes=1 << 40):
    return lib.favor_bidir(ctypes.byref(s) if s is not None else None, q, k, v, om, o, ws, nbytes, None)


def _causal(lib, s, chunk=0, q=P_Q, k=P_K, v=P_V, om=P_OM, o=P_O, ws=P_WS, nbytes=1 << 40):
    return lib.favor_causal(ctypes.byref(s) if s is not None else None, q, k, v, om, o, chunk, ws, nbytes, None)


@pytest.mark.parametrize("fn", [_bidir, _causal])
def test_validation(lib, fn):
    assert fn(lib, None) == INVALID
    assert fn(lib, shp(B=0)) == INVALID
    assert fn(lib, shp(H=-1)) == INVALID
    assert fn(lib, shp(L=-5)) == INVALID
    assert fn(lib, shp(d=48)) == UNSUPPORTED
    assert fn(lib, shp(d=256)) == UNSUPPORTED
    assert fn(lib, shp(m=33)) == UNSUPPORTED
    assert fn(lib, shp(m=544)) == UNSUPPORTED
    assert fn(lib, shp(m=288)) == UNSUPPORTED
    assert fn(lib, shp(dtype=7)) == UNSUPPORTED
    assert fn(lib, shp(stride=5)) == INVALID
    assert fn(lib, shp(), q=None) == INVALID
    assert fn(lib, shp(), om=None) == INVALID
    assert fn(lib, shp(), o=None) == INVALID
    assert fn(lib, shp(), q=P_Q + 8) == INVALID          # 16-byte alignment
    assert fn(lib, shp(), o=P_Q) == INVALID              # out aliases q
    assert fn(lib, shp(), o=P_V + 64) == INVALID         # out overlaps v
    assert fn(lib, shp(), o=P_OM) == INVALID             # out overlaps omega
    for p in (P_Q, P_K, P_V, P_OM):                     # the workspace overlaps an input
        assert fn(lib, shp(), ws=p) == INVALID
    assert fn(lib, shp(), ws=P_K - 256) == INVALID       # ... partly
    assert fn(lib, shp(), ws=None) == WORKSPACE
    assert fn(lib, shp(), ws=P_WS + 16) == WORKSPACE     # 256-byte alignment
    need = lib.favor_workspace_bytes(1 if fn is _bidir else 2, ctypes.byref(shp()), 0)
    assert fn(lib, shp(), nbytes=need - 1) == WORKSPACE
    assert fn(lib, shp(L=0), q=None, k=None, v=None, o=None, ws=None, nbytes=0) == OK  # L = 0: no-op
    assert fn(lib, shp(B=1 << 16, H=1 << 8, L=1 << 8, d=64)) == UNSUPPORTED            # > 2^31 elements
    # more than 65535 (batch, head) pairs: unsupported even where the element
    # count fits, rejected before any pointer is looked at
    assert fn(lib, shp(B=65536, H=1, L=1, d=16), q=None, o=None, ws=None) == UNSUPPORTED
    assert fn(lib, shp(B=257, H=256, L=4, d=16), q=None, o=None, ws=None) == UNSUPPORTED
    assert lib.favor_workspace_bytes(1 if fn is _bidir else 2, ctypes.byref(shp(B=65536, H=1, L=1, d=16)), 0) == 0
    assert lib.favor_workspace_bytes(1 if fn is _bidir else 2, ctypes.byref(shp(B=65535, H=1, L=1, d=16)), 0) > 0


def documented_support(dtype, d, m, op):
    """The supported set as include/favor.h states it."""
    if d not in (16, 32, 64, 128) or (dtype == _lib.FAVOR_F32 and d > 64):
        return False
    if op == 2:
        return m in (32, 64, 128, 256, 512) and not (dtype == _lib.FAVOR_F32 and d == 64 and m == 512)
    return m >= 32 and ((m <= 256 and m % 32 == 0) or (m <= 512 and m % 64 == 0))


def test_support_matrix_matches_header(lib):
    # every (dtype, d, m, op) over a grid wider than the supported set: the
    # library accepts (nonzero workspace) exactly what the header documents
    for dtype in (_lib.FAVOR_F32, _lib.FAVOR_BF16):
        for d in (8, 16, 24, 32, 48, 64, 96, 128, 256):
            for m in range(16, 577, 16):
                for op in (0, 1, 2):
                    for feature in (_lib.FAVOR_FEATURE_POSITIVE, _lib.FAVOR_FEATURE_RELU):
                        s = shp(d=d, m=m, dtype=dtype, feature=feature)
                        got = lib.favor_workspace_bytes(op, ctypes.byref(s), 0) > 0
                        assert got == documented_support(dtype, d, m, op), (dtype, d, m, op, feature)


def test_causal_chunk_and_lds_limits(lib):
    # A one-byte workspace makes an accepted shape stop at the workspace
    # check (WORKSPACE), before anything is launched.
    # chunk: 0, 32, and 64 where the shape has the 64-token tile scan
    # (bf16, d=64, m in {64, 128, 256})
    for m in (64, 128, 256):
        assert _causal(lib, shp(m=m), chunk=64, nbytes=1) == WORKSPACE
        assert _causal(lib, shp(m=m), chunk=32, nbytes=1) == WORKSPACE
    for chunk in (16, 48, 128, 96):
        assert _causal(lib, shp(), chunk=chunk, nbytes=1) == UNSUPPORTED
    assert _causal(lib, shp(m=32), chunk=64, nbytes=1) == UNSUPPORTED
    assert _causal(lib, shp(d=128, m=512), chunk=64, nbytes=1) == UNSUPPORTED
    assert _causal(lib, shp(dtype=_lib.FAVOR_F32), chunk=64, nbytes=1) == UNSUPPORTED
    assert _causal(lib, shp(d=32, m=64), chunk=32, nbytes=1) == WORKSPACE
    assert _causal(lib, shp(d=32, m=64), chunk=64, nbytes=1) == UNSUPPORTED
    assert _causal(lib, shp(m=512), chunk=32, nbytes=1) == WORKSPACE
    assert _causal(lib, shp(), chunk=-1) == UNSUPPORTED
    assert _causal(lib, shp(m=96)) == UNSUPPORTED      # causal: m in {32, 64, 128, 256, 512}
    assert _bidir(lib, shp(m=96), nbytes=1) == WORKSPACE
    assert _bidir(lib, shp(d=128, dtype=_lib.FAVOR_F32)) == UNSUPPORTED
    # fp32 d=128 m=512: the causal state does not fit one workgroup's LDS
    assert _causal(lib, shp(d=128, m=512, dtype=_lib.FAVOR_F32)) == UNSUPPORTED


def test_features_validation(lib):
    s = shp()
    f = lib.favor_features
    assert f(ctypes.byref(s), None, P_OM, P_O, None, 0, P_WS, 1 << 40, None) == INVALID
    assert f(ctypes.byref(s), P_Q, P_OM, P_O, None, 1, P_WS, 1 << 40, None) == INVALID   # log_scale needed
    assert f(ctypes.byref(s), P_Q, P_OM, P_Q, None, 0, P_WS, 1 << 40, None) == INVALID   # phi overlaps x
    assert f(ctypes.byref(s), P_Q, P_OM, P_O, None, 0, P_WS, 16, None) == WORKSPACE
    assert f(ctypes.byref(s), P_Q, P_OM, P_OM, None, 0, P_WS, 1 << 40, None) == INVALID  # phi overlaps omega
    assert f(ctypes.byref(s), P_Q, P_OM, P_O, P_Q, 1, P_WS, 1 << 40, None) == INVALID   # log_scale overlaps x
    for ws in (P_Q, P_OM, P_O):                                                          # ws overlaps x, omega, phi
        assert f(ctypes.byref(s), P_Q, P_OM, P_O, None, 0, ws, 1 << 40, None) == INVALID
    assert f(ctypes.byref(s), P_Q, P_OM, P_O, P_S1, 1, P_S1, 1 << 40, None) == INVALID  # ... or log_scale


@pytest.mark.parametrize("seed,H,m,d", [(0, 1, 32, 16), (0, 8, 256, 64), (3, 2, 40, 16), (11, 1, 512, 128), (5, 3, 10, 4)])
def test_orf_omega_matches_oracle(lib, seed, H, m, d):
    """The library's host generator (same published Philox4x64-10 and the same
    construction) reproduces the oracle's projection."""
    out = np.empty((H, m, d), dtype=np.float32)
    assert lib.favor_orf_omega(seed, H, m, d, out.ctypes.data) == OK
    want = ref.orf_omega(seed, H, m, d)
    np.testing.assert_allclose(out, want, rtol=2e-7, atol=2e-7)


def test_orf_omega_invalid(lib):
    out = np.empty(16, dtype=np.float32)
    assert lib.favor_orf_omega(0, 1, 4, 4, None) == INVALID
    assert lib.favor_orf_omega(0, 0, 4, 4, out.ctypes.data) == INVALID
    assert lib.favor_orf_omega(0, 1, -4, 4, out.ctypes.data) == INVALID




def _causal_state(lib, s, si=P_S1, so=P_S2, chunk=0, o=P_O, ws=P_WS, nbytes=1 << 40):
    return lib.favor_causal_state(ctypes.byref(s) if s is not None else None, P_Q, P_K, P_V, P_OM, o, chunk, si, so,
                                  ws, nbytes, None)


def test_causal_state_validation(lib):
    """Carried-state arguments are checked before anything is launched."""
    assert _causal_state(lib, None) == INVALID
    assert _causal_state(lib, shp(), so=P_S1) == INVALID             # state_out aliases state_in
    assert _causal_state(lib, shp(), so=P_S1 + 64) == INVALID        # ... or overlaps it
    assert _causal_state(lib, shp(), so=P_O) == INVALID              # state_out overlaps out
    assert _causal_state(lib, shp(), so=P_WS + 1024) == INVALID      # ... or the workspace
    assert _causal_state(lib, shp(), si=None, so=P_Q) == INVALID     # ... or q
    assert _causal_state(lib, shp(), si=P_WS + 1024, so=None) == INVALID  # state_in inside the workspace
    assert _causal_state(lib, shp(), si=P_S1 + 2) == INVALID         # 4-byte alignment
    assert _causal_state(lib, shp(), so=P_S2 + 2) == INVALID
    assert _causal_state(lib, shp(), chunk=16) == UNSUPPORTED        # chunk as for favor_causal
    assert _causal_state(lib, shp(d=32, m=64), chunk=64) == UNSUPPORTED
    assert _causal_state(lib, shp(), si=P_O, so=None) == INVALID     # state_in overlaps out
    assert _causal_state(lib, shp(), nbytes=1) == WORKSPACE
    assert _causal_state(lib, shp(L=0), o=None, ws=None, nbytes=0) == OK  # L = 0: no-op, nothing written


def test_feature_kind_validation(lib):
    assert _bidir(lib, shp(feature=2)) == UNSUPPORTED
    assert _causal(lib, shp(feature=-1)) == UNSUPPORTED
    assert _bidir(lib, shp(feature=_lib.FAVOR_FEATURE_RELU), nbytes=1) == WORKSPACE   # accepted up to the workspace
    assert _causal(lib, shp(feature=_lib.FAVOR_FEATURE_RELU), nbytes=1) == WORKSPACE
    assert _causal_state(lib, shp(feature=_lib.FAVOR_FEATURE_RELU)) == UNSUPPORTED  # no carried state for ReLU
    # the struct the binding passes has the header's layout
    assert ctypes.sizeof(_lib.FavorShape) == 40


def test_hadamard_omega_validation(lib):
    f = lib.favor_hadamard_omega
    assert f(0, 1, 32, 16, None, None) == INVALID
    assert f(0, 1, 32, 16, P_OM + 4, None) == INVALID    # 16-byte alignment
    assert f(0, 0, 32, 16, P_OM, None) == INVALID
    assert f(0, 1, 0, 16, P_OM, None) == INVALID
    assert f(0, 1, 32, 48, P_OM, None) == UNSUPPORTED   # d must be 16, 32, 64 or 128
    assert f(0, 1 << 12, 1 << 12, 128, P_OM, None) == UNSUPPORTED  # >= 2^31 elements


def test_features_hadamard_validation(lib):
    f = lib.favor_features_hadamard

    def call(s, x=P_Q, phi=P_O, ls=None, stab=0):
        return f(ctypes.byref(s), x, 1, phi, ls, stab, None)

    assert call(shp(B=1, H=1, L=0)) == OK                 # nothing to do
    assert f(None, P_Q, 1, P_O, None, 0, None) == INVALID
    assert call(shp(), x=None) == INVALID
    assert call(shp(), phi=None) == INVALID
    assert call(shp(), x=P_Q + 8) == INVALID                 # 16-byte alignment
    assert call(shp(), stab=1) == INVALID                     # stabilised: log_scale required
    assert call(shp(d=48)) == UNSUPPORTED
    assert call(shp(m=48)) == UNSUPPORTED
    assert call(shp(B=300, H=300)) == UNSUPPORTED           # one grid row per (batch, head)
    assert call(shp(), phi=P_Q) == INVALID                    # phi overlaps x


def test_givens_omega_validation(lib):
    f = lib.favor_givens_omega
    assert f(0, 1, 32, 16, 0, None, None) == INVALID
    assert f(0, 1, 32, 16, 0, P_OM + 4, None) == INVALID    # 16-byte alignment
    assert f(0, 0, 32, 16, 0, P_OM, None) == INVALID
    assert f(0, 1, 0, 16, 0, P_OM, None) == INVALID
    assert f(0, 1, 32, 16, -1, P_OM, None) == INVALID       # rotations in [0, 2^24]
    assert f(0, 1, 32, 16, (1 << 24) + 1, P_OM, None) == INVALID
    assert f(0, 1, 32, 1, 0, P_OM, None) == UNSUPPORTED     # 2 <= d <= 128
    assert f(0, 1, 32, 129, 0, P_OM, None) == UNSUPPORTED
    assert f(0, 65536, 1, 16, 0, P_OM, None) == UNSUPPORTED  # one grid row per head
    assert f(0, 1 << 12, 1 << 12, 128, 0, P_OM, None) == UNSUPPORTED  # >= 2^31 elements


def _causal_plan(lib, s, chunk=0, segments=0, ws=P_WS, nbytes=1 << 40):
    pl = _lib.plan(chunk, segments)
    return lib.favor_causal_plan(ctypes.byref(s), P_Q, P_K, P_V, P_OM, P_O, ctypes.byref(pl), ws, nbytes, None)


def _bidir_plan(lib, s, segments=0, ws=P_WS, nbytes=1 << 40, plan=True):
    pl = _lib.plan(0, segments)
    return lib.favor_bidir_plan(ctypes.byref(s), P_Q, P_K, P_V, P_OM, P_O, ctypes.byref(pl) if plan else None, ws,
                                nbytes, None)


def test_plan_validation(lib):
    """Plan overrides: segments in [0, 256], chunk as for favor_causal; the
    workspace follows the plan."""
    s = shp(B=2, H=8, L=8192)
    for fn in (_causal_plan, _bidir_plan):
        assert fn(lib, s, segments=-1) == INVALID
        assert fn(lib, s, segments=257) == INVALID
        assert fn(lib, s, segments=1, nbytes=1) == WORKSPACE
        assert fn(lib, s, segments=256, nbytes=1) == WORKSPACE
    assert _bidir_plan(lib, s, plan=False, nbytes=1) == WORKSPACE   # NULL plan: defaults
    assert _causal_plan(lib, s, chunk=16, nbytes=1) == UNSUPPORTED
    assert _causal_plan(lib, s, chunk=32, nbytes=1) == WORKSPACE
    sz = lambda op, chunk=0, seg=0: lib.favor_workspace_bytes_plan(op, ctypes.byref(s), ctypes.byref(_lib.plan(chunk, seg)))
    # the default plan is the plain entry points' plan
    assert sz(2) == lib.favor_workspace_bytes(2, ctypes.byref(s), 0)
    assert sz(1) == lib.favor_workspace_bytes(1, ctypes.byref(s), 0)
    assert lib.favor_workspace_bytes_plan(2, ctypes.byref(s), None) == sz(2)
    # fewer segments, less workspace; invalid plans report 0
    assert 0 < sz(2, seg=1) < sz(2, seg=4) < sz(2, seg=64)
    assert sz(1, seg=1) < sz(1)
    assert sz(2, chunk=16) == 0 and sz(2, seg=-3) == 0 and sz(2, seg=300) == 0
    # the workspace of the requested plan is what the call checks
    need = sz(2, seg=3)
    assert _causal_plan(lib, s, segments=3, nbytes=need - 1) == WORKSPACE



@pytest.mark.parametrize("dtype,d,m,BH,L,one", [
    (_lib.FAVOR_BF16, 64, 256, 128, 512, True),   # the one-kernel path fits
    (_lib.FAVOR_BF16, 64, 256, 64, 384, True),
    (_lib.FAVOR_BF16, 128, 64, 128, 512, True),
    (_lib.FAVOR_F32, 32, 256, 128, 512, True),
    (_lib.FAVOR_F32, 64, 256, 128, 512, False),   # does not fit: segments kept
    (_lib.FAVOR_BF16, 128, 256, 128, 512, False),
    (_lib.FAVOR_BF16, 64, 256, 32, 512, False),   # too few heads
    (_lib.FAVOR_BF16, 64, 256, 64, 512, False),
    (_lib.FAVOR_BF16, 64, 256, 128, 1024, False),  # too long
    (_lib.FAVOR_F32, 16, 32, 1, 256, True),       # 32 features: the key-split kernel
    (_lib.FAVOR_BF16, 64, 32, 8, 512, True),
    (_lib.FAVOR_BF16, 32, 32, 128, 4096, True),
    (_lib.FAVOR_BF16, 32, 32, 64, 1024, False),
    (_lib.FAVOR_F32, 64, 32, 1, 256, False),      # fp32 d = 64: not that kernel, too few heads
])
def test_bidir_plan_one_segment_only_where_one_kernel_runs(lib, dtype, d, m, BH, L, one):
    """The automatic bidirectional plan gives each head a single segment (one
    kernel per call) only for many heads of short sequences whose one-kernel
    path fits a compute unit's LDS; elsewhere it keeps the segments.  The
    plan is visible through the workspace size, which grows with it."""
    B, H = (BH // 8, 8) if BH >= 8 else (1, BH)
    s = shp(B=B, H=H, L=L, d=d, m=m, dtype=dtype)
    auto = lib.favor_workspace_bytes(1, ctypes.byref(s), 0)
    assert auto > 0
    one_seg = lib.favor_workspace_bytes_plan(1, ctypes.byref(s), ctypes.byref(_lib.plan(0, 1)))
    assert (auto == one_seg) == one
    if not one:
        assert auto > one_seg


@pytest.mark.parametrize("B,H,L,segs", [(2, 8, 512, 8), (1, 8, 1024, 16), (2, 8, 8192, 16), (1, 1, 100, 1)])
def test_causal_plan_segments_of_at_least_64_tokens(lib, B, H, L, segs):
    """The automatic causal plan keeps segments of at least 64 tokens (and
    one per compute unit otherwise); visible through the workspace size."""
    s = shp(B=B, H=H, L=L)
    auto = lib.favor_workspace_bytes(2, ctypes.byref(s), 0)
    want = lib.favor_workspace_bytes_plan(2, ctypes.byref(s), ctypes.byref(_lib.plan(0, segs)))
    assert auto == want > 0

def test_noalloc_validation(lib):
    """The entry point without a workspace validates like favor_causal and
    refuses shapes whose workspace exceeds its static scratch array, all
    before any HIP call."""
    f = lib.favor_causal_noalloc
    assert f(None, P_Q, P_K, P_V, P_OM, P_O, 0, None) == INVALID
    assert f(ctypes.byref(shp(B=0)), P_Q, P_K, P_V, P_OM, P_O, 0, None) == INVALID
    assert f(ctypes.byref(shp(d=48)), P_Q, P_K, P_V, P_OM, P_O, 0, None) == UNSUPPORTED
    assert f(ctypes.byref(shp()), P_Q, P_K, P_V, P_OM, P_O, 16, None) == UNSUPPORTED
    big = shp(B=1, H=512, L=128, d=128, m=512)
    assert lib.favor_workspace_bytes(2, ctypes.byref(big), 0) > _lib.FAVOR_NOALLOC_SCRATCH_BYTES
    assert f(ctypes.byref(big), P_Q, P_K, P_V, P_OM, P_O, 0, None) == WORKSPACE
    # the benchmarked causal workloads fit
    for s in (shp(B=2, H=8, L=8192), shp(B=1, H=16, L=65536, d=128, m=512)):
        assert 0 < lib.favor_workspace_bytes(2, ctypes.byref(s), 0) <= _lib.FAVOR_NOALLOC_SCRATCH_BYTES
