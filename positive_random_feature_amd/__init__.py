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

__all__ = ["features", "bidir", "causal", "orf_omega", "hadamard_omega", "workspace_bytes", "state_floats",
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


def _check_inputs(tensors, omega):
    dev = tensors[0].device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device")
    dt = tensors[0].dtype
    if dt not in _DTYPES:
        raise TypeError(f"unsupported dtype {dt}")
    for t in tensors:
        if t.device != dev or t.dtype != dt or t.dim() != 4 or not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous [B, H, L, d] tensors of one dtype on one device")
    if omega.device != dev or omega.dtype != torch.float32 or not omega.is_contiguous():
        raise ValueError("omega must be a contiguous float32 tensor on the same device")
    return dev, dt


def _shape(x: torch.Tensor, omega: torch.Tensor, feature: str = "positive") -> _lib.FavorShape:
    """Shape descriptor; ``feature`` is "positive" (softmax-kernel features)
    or "relu" (generalised ReLU features)."""
    B, H, L, d = x.shape
    m = omega.shape[-2]
    if feature not in _FEATURES:
        raise ValueError(f"feature must be one of {sorted(_FEATURES)}")
    return _lib.shape(B, H, L, d, m, _DTYPES[x.dtype], _omega_stride(omega, H, m, d), _FEATURES[feature])


def workspace_bytes(op: int, shp: _lib.FavorShape) -> int:
    return int(_lib.load().favor_workspace_bytes(op, ctypes.byref(shp), 0))


def _workspace(op: int, shp: _lib.FavorShape, dev) -> torch.Tensor:
    n = workspace_bytes(op, shp)
    if n == 0:
        raise FavorError(2, "favor_workspace_bytes")
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


def bidir(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, omega: torch.Tensor,
          out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
          feature: str = "positive") -> torch.Tensor:
    """Bidirectional FAVOR+: phi(Q)(phi(K)^T V) / phi(Q)(phi(K)^T 1)."""
    dev, dt = _check_inputs([q, k, v], omega)
    shp = _shape(q, omega, feature)
    out = torch.empty_like(q) if out is None else out
    ws = _workspace(_lib.FAVOR_OP_BIDIR, shp, dev) if workspace is None else workspace
    st = _lib.load().favor_bidir(ctypes.byref(shp), q.data_ptr(), k.data_ptr(), v.data_ptr(), omega.data_ptr(),
                                 out.data_ptr(), ws.data_ptr(), ws.numel(), _stream(dev))
    _lib.check(st, "favor_bidir")
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
           state: torch.Tensor | None = None, return_state: bool = False, feature: str = "positive"):
    """Causal FAVOR+ through the prefix-sum state G_t = sum_{s<=t} phi(k_s) v_s^T.

    ``state`` ([B, H, m (d + 1) + 1] float32 on the device, or None) carries
    the prefix of keys seen by earlier calls; with ``return_state`` the state
    including this call's keys is returned as well: (out, state).
    ``feature="relu"`` selects the generalised ReLU features (no carried state).
    """
    dev, dt = _check_inputs([q, k, v], omega)
    shp = _shape(q, omega, feature)
    out = torch.empty_like(q) if out is None else out
    ws = _workspace(_lib.FAVOR_OP_CAUSAL, shp, dev) if workspace is None else workspace
    lib = _lib.load()
    if state is None and not return_state:
        st = lib.favor_causal(ctypes.byref(shp), q.data_ptr(), k.data_ptr(), v.data_ptr(), omega.data_ptr(),
                              out.data_ptr(), int(chunk), ws.data_ptr(), ws.numel(), _stream(dev))
        _lib.check(st, "favor_causal")
        return out
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
