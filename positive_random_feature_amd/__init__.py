"""FAVOR+ attention on MI355X (gfx950): positive orthogonal random features,
bidirectional and causal attention, through the C ABI in include/favor.h.

Every step runs in the HIP library ``libfavor_amd.so``; this module only
checks tensors, allocates the workspace with torch and passes pointers and
the current stream.  It fails loudly when the library is missing.
"""

from __future__ import annotations

import ctypes

import torch

from . import _lib

__all__ = ["features", "features_hadamard", "bidir", "causal", "causal_noalloc", "orf_omega", "hadamard_omega", "givens_omega", "workspace_bytes", "state_floats",
           "state_parts", "FavorError"]

FavorError = _lib.FavorError

_DTYPES = {torch.bfloat16: _lib.FAVOR_BF16, torch.float32: _lib.FAVOR_F32}
_FEATURES = {"positive": _lib.FAVOR_FEATURE_POSITIVE, "relu": _lib.FAVOR_FEATURE_RELU}


def _omega_stride(omega: torch.Tensor, H: int, m: int, d: int) -> int:
    if omega.dim() == 2 and tuple(omega.shape) == (m, d):
        return 0
    if omega.dim() == 3 and tuple(omega.shape) == (1, m, d):
        return 0
    if omega.dim() == 3 and tuple(omega.shape) == (H, m, d):
        return m * d
    raise ValueError(f"omega must be [m, d], [1, m, d] or [H, m, d]; got {tuple(omega.shape)}")


def _check_inputs(tensors, omega, out=None, workspace=None):
    """q, k, v (or x), omega and the optional out and workspace: shapes,
    dtypes and layout first (host-side, before anything touches a device),
    then that every tensor is on the inputs' GPU."""
    x = tensors[0]
    dt = x.dtype
    if dt not in _DTYPES:
        raise TypeError(f"unsupported dtype {dt}")
    if x.dim() != 4:
        raise ValueError(f"inputs must be [B, H, L, d]; got {tuple(x.shape)}")
    for t in tensors:
        if tuple(t.shape) != tuple(x.shape):
            raise ValueError(f"q, k, v must have one shape; got {tuple(x.shape)} and {tuple(t.shape)}")
        if t.dtype != dt:
            raise ValueError("q, k, v must have one dtype")
        if not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous")
    if omega.dtype != torch.float32 or not omega.is_contiguous():
        raise ValueError("omega must be a contiguous float32 tensor")
    if omega.dim() not in (2, 3):
        raise ValueError(f"omega must be [m, d], [1, m, d] or [H, m, d]; got {tuple(omega.shape)}")
    _omega_stride(omega, x.shape[1], omega.shape[-2], x.shape[3])
    if out is not None and (tuple(out.shape) != tuple(x.shape) or out.dtype != dt or not out.is_contiguous()):
        raise ValueError(f"out must be a contiguous {dt} tensor of shape {tuple(x.shape)}")
    if workspace is not None and (workspace.dtype != torch.uint8 or workspace.dim() != 1
                                  or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous 1-D uint8 tensor")
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device")
    for t in list(tensors) + [omega] + [t for t in (out, workspace) if t is not None]:
        if t.device != dev:
            raise ValueError("q, k, v, omega, out and workspace must be on one device")
    return dev, dt


def _shape(x: torch.Tensor, omega: torch.Tensor, feature: str = "positive") -> _lib.FavorShape:
    """Shape descriptor; ``feature`` is "positive" (softmax-kernel features)
    or "relu" (generalised ReLU features)."""
    B, H, L, d = x.shape
    m = omega.shape[-2]
    if feature not in _FEATURES:
        raise ValueError(f"feature must be one of {sorted(_FEATURES)}")
    return _lib.shape(B, H, L, d, m, _DTYPES[x.dtype], _omega_stride(omega, H, m, d), _FEATURES[feature])


def workspace_bytes(op: int, shp: _lib.FavorShape, chunk: int = 0, segments: int = 0) -> int:
    """Workspace bytes of one call (0: invalid shape or plan)."""
    pl = _lib.plan(chunk, segments)
    return int(_lib.load().favor_workspace_bytes_plan(op, ctypes.byref(shp), ctypes.byref(pl)))


def _workspace(op: int, shp: _lib.FavorShape, dev, chunk: int = 0, segments: int = 0,
               given: torch.Tensor | None = None) -> torch.Tensor:
    n = workspace_bytes(op, shp, chunk, segments)
    if n == 0:
        raise FavorError(2, "favor_workspace_bytes_plan")
    if given is not None:
        if given.numel() < n:
            raise ValueError(f"workspace holds {given.numel()} bytes; this call needs {n}")
        return given
    return torch.empty(n, dtype=torch.uint8, device=dev)


def _stream(dev) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def features(x: torch.Tensor, omega: torch.Tensor, stabilize: bool = False, feature: str = "positive"):
    """phi(x) = m^-1/2 exp(omega x - |x|^2/2) as fp32 [B, H, L, m]
    (``feature="relu"``: m^-1/2 max(omega x, 0)).

    With ``stabilize`` the per-row maximum exponent s is taken out and
    returned as ``log_scale`` ([B, H, L]); phi * exp(log_scale) is the plain
    feature map (0 for ReLU features).  Returns (phi, log_scale or None).
    """
    dev, _ = _check_inputs([x], omega)
    shp = _shape(x, omega, feature)
    B, H, L, _d = x.shape
    phi = torch.empty((B, H, L, shp.m), dtype=torch.float32, device=dev)
    log_scale = torch.empty((B, H, L), dtype=torch.float32, device=dev) if stabilize else None
    ws = _workspace(_lib.FAVOR_OP_FEATURES, shp, dev)
    st = _lib.load().favor_features(ctypes.byref(shp), x.data_ptr(), omega.data_ptr(), phi.data_ptr(),
                                    log_scale.data_ptr() if stabilize else None, 1 if stabilize else 0,
                                    ws.data_ptr(), ws.numel(), _stream(dev))
    _lib.check(st, "favor_features")
    return phi, log_scale


def features_hadamard(x: torch.Tensor, seed: int, m: int, per_head: bool = True, stabilize: bool = False,
                      feature: str = "positive"):
    """``features`` over the structured Hadamard projection that
    ``hadamard_omega(seed, H if per_head else 1, m, d)`` would generate, built
    with fast Walsh-Hadamard transforms instead of a dense projection (the
    projection itself is never formed).  Returns (phi, log_scale or None)."""
    if x.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {x.dtype}")
    if x.dim() != 4 or not x.is_contiguous():
        raise ValueError(f"x must be a contiguous [B, H, L, d] tensor; got {tuple(x.shape)}")
    if feature not in _FEATURES:
        raise ValueError(f"feature must be one of {sorted(_FEATURES)}")
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("x must be on a GPU device")
    B, H, L, d = x.shape
    shp = _lib.shape(B, H, L, d, int(m), _DTYPES[x.dtype], int(m) * d if per_head else 0, _FEATURES[feature])
    phi = torch.empty((B, H, L, int(m)), dtype=torch.float32, device=dev)
    log_scale = torch.empty((B, H, L), dtype=torch.float32, device=dev) if stabilize else None
    st = _lib.load().favor_features_hadamard(ctypes.byref(shp), x.data_ptr(), int(seed), phi.data_ptr(),
                                             log_scale.data_ptr() if stabilize else None, 1 if stabilize else 0,
                                             _stream(dev))
    _lib.check(st, "favor_features_hadamard")
    return phi, log_scale


def bidir(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, omega: torch.Tensor,
          out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
          feature: str = "positive", segments: int = 0) -> torch.Tensor:
    """Bidirectional FAVOR+: phi(Q)(phi(K)^T V) / phi(Q)(phi(K)^T 1).
    ``segments``: token segments per head of the reduction (0 = automatic);
    with one segment per head the call runs as a single kernel where its
    operands fit on a compute unit (the automatic plan chooses that for many
    heads of short sequences, and for m = 32 up to 512 tokens, or up to 4096
    from 128 heads)."""
    dev, dt = _check_inputs([q, k, v], omega, out, workspace)
    shp = _shape(q, omega, feature)
    out = torch.empty_like(q) if out is None else out
    ws = _workspace(_lib.FAVOR_OP_BIDIR, shp, dev, 0, segments, workspace)
    pl = _lib.plan(0, segments)
    st = _lib.load().favor_bidir_plan(ctypes.byref(shp), q.data_ptr(), k.data_ptr(), v.data_ptr(), omega.data_ptr(),
                                      out.data_ptr(), ctypes.byref(pl), ws.data_ptr(), ws.numel(), _stream(dev))
    _lib.check(st, "favor_bidir_plan")
    return out


def state_floats(m: int, d: int) -> int:
    """Floats per head of a carried causal state: S [m, d], z [m], shift."""
    return m * (d + 1) + 1


def state_parts(state: torch.Tensor, m: int, d: int):
    """Views (S [..., m, d], z [..., m], shift [...]) of a state tensor
    [..., m (d + 1) + 1]; the carried sums are S e^shift and z e^shift."""
    S = state[..., : m * d].unflatten(-1, (m, d))
    z = state[..., m * d: m * (d + 1)]
    return S, z, state[..., m * (d + 1)]


def causal(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, omega: torch.Tensor, chunk: int = 0,
           out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
           state: torch.Tensor | None = None, return_state: bool = False, feature: str = "positive",
           segments: int = 0):
    """Causal FAVOR+ through the prefix-sum state G_t = sum_{s<=t} phi(k_s) v_s^T.

    ``chunk``: tokens per scan step (0 = the shape's default; 32, or 64 where
    the shape has a 64-token scan).  ``segments``: token segments per head
    (0 = automatic).
    ``state`` ([B, H, m (d + 1) + 1] float32 on the device, or None) carries
    the prefix of keys seen by earlier calls; with ``return_state`` the state
    including this call's keys is returned as well: (out, state).
    ``feature="relu"`` selects the generalised ReLU features (no carried state).
    """
    dev, dt = _check_inputs([q, k, v], omega, out, workspace)
    shp = _shape(q, omega, feature)
    out = torch.empty_like(q) if out is None else out
    lib = _lib.load()
    if state is None and not return_state:
        ws = _workspace(_lib.FAVOR_OP_CAUSAL, shp, dev, chunk, segments, workspace)
        pl = _lib.plan(chunk, segments)
        st = lib.favor_causal_plan(ctypes.byref(shp), q.data_ptr(), k.data_ptr(), v.data_ptr(), omega.data_ptr(),
                                   out.data_ptr(), ctypes.byref(pl), ws.data_ptr(), ws.numel(), _stream(dev))
        _lib.check(st, "favor_causal_plan")
        return out
    if segments:
        raise ValueError("segments cannot be chosen together with a carried state")
    ws = _workspace(_lib.FAVOR_OP_CAUSAL, shp, dev, chunk, 0, workspace)
    B, H, _L, d = q.shape
    n = state_floats(shp.m, d)
    if state is not None:
        if state.device != dev or state.dtype != torch.float32 or not state.is_contiguous() \
                or tuple(state.shape) != (B, H, n):
            raise ValueError(f"state must be a contiguous float32 [B, H, {n}] tensor on the same device")
    new_state = torch.empty((B, H, n), dtype=torch.float32, device=dev) if return_state else None
    st = lib.favor_causal_state(ctypes.byref(shp), q.data_ptr(), k.data_ptr(), v.data_ptr(), omega.data_ptr(),
                                out.data_ptr(), int(chunk), state.data_ptr() if state is not None else None,
                                new_state.data_ptr() if new_state is not None else None, ws.data_ptr(), ws.numel(),
                                _stream(dev))
    _lib.check(st, "favor_causal_state")
    return (out, new_state) if return_state else out


def causal_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, omega: torch.Tensor, out: torch.Tensor,
                   chunk: int = 0) -> torch.Tensor:
    """Causal FAVOR+ through favor_causal_noalloc: no workspace argument and
    no allocation in the call (the library's static per-GPU scratch array of
    FAVOR_NOALLOC_SCRATCH_BYTES is used); ``out`` must be provided.  Calls
    that overlap in time on one GPU race on that array."""
    dev, dt = _check_inputs([q, k, v], omega, out)
    shp = _shape(q, omega)
    st = _lib.load().favor_causal_noalloc(ctypes.byref(shp), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                          omega.data_ptr(), out.data_ptr(), int(chunk), _stream(dev))
    _lib.check(st, "favor_causal_noalloc")
    return out


def orf_omega(seed: int, n_heads: int, m: int, d: int) -> torch.Tensor:
    """Seeded orthogonal projection [n_heads, m, d] (float32, CPU tensor)."""
    out = torch.empty((n_heads, m, d), dtype=torch.float32)
    st = _lib.load().favor_orf_omega(int(seed), int(n_heads), int(m), int(d), out.data_ptr())
    _lib.check(st, "favor_orf_omega")
    return out


def hadamard_omega(seed: int, n_heads: int, m: int, d: int, device="cuda") -> torch.Tensor:
    """Structured (Hadamard) orthogonal projection [n_heads, m, d] (float32),
    generated on the device: blocks sqrt(d) H S1 H S2 H S3 with seeded +-1
    diagonals S_t."""
    dev = torch.device(device)
    out = torch.empty((n_heads, m, d), dtype=torch.float32, device=dev)
    st = _lib.load().favor_hadamard_omega(int(seed), int(n_heads), int(m), int(d), out.data_ptr(), _stream(dev))
    _lib.check(st, "favor_hadamard_omega")
    return out


def givens_omega(seed: int, n_heads: int, m: int, d: int, rotations: int = 0, device="cuda") -> torch.Tensor:
    """Structured (Givens) orthogonal projection [n_heads, m, d] (float32),
    generated on the device: each block a product of random plane rotations
    (d ceil(log2 d) of them when ``rotations`` is 0) with chi(d) row lengths."""
    dev = torch.device(device)
    out = torch.empty((n_heads, m, d), dtype=torch.float32, device=dev)
    st = _lib.load().favor_givens_omega(int(seed), int(n_heads), int(m), int(d), int(rotations), out.data_ptr(),
                                        _stream(dev))
    _lib.check(st, "favor_givens_omega")
    return out
