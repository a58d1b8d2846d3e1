"""ctypes loader for the plain-C fp64 oracle (``favor_oracle.c``).

TEST INFRASTRUCTURE ONLY: only the test suite, the smoke check and the
benchmark's CPU-baseline leg may use this module.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "favor_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile ``favor_oracle.c`` with gcc (-O2, OpenMP) into ``liboracle.so``."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        for name in ("oracle_bidir", "oracle_causal"):
            fn = getattr(lib, name)
            fn.restype = ctypes.c_int
            fn.argtypes = [ctypes.c_int] * 5 + [dp, dp, dp, dp, ctypes.c_int, dp]
        lib.oracle_features.restype = None
        lib.oracle_features.argtypes = [ctypes.c_long, ctypes.c_int, ctypes.c_int, dp, dp, dp]
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_num_threads.argtypes = []
        _lib = lib
    return _lib


def _dptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def features(x: np.ndarray, omega: np.ndarray) -> np.ndarray:
    """phi(x) for rows x[..., d] and one omega[m, d]; float64 [..., m]."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float64)
    om = np.ascontiguousarray(omega, dtype=np.float64)
    m, d = om.shape
    rows = x.reshape(-1, d)
    phi = np.empty((rows.shape[0], m), dtype=np.float64)
    lib.oracle_features(rows.shape[0], d, m, _dptr(rows), _dptr(om), _dptr(phi))
    return phi.reshape(*x.shape[:-1], m)


def _attn(name: str, q, k, v, omega) -> np.ndarray:
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    om = np.ascontiguousarray(omega, dtype=np.float64)
    B, H, L, d = q.shape
    if om.ndim == 2:
        per_head = 0
        m = om.shape[0]
    elif om.shape[0] == 1:
        per_head = 0
        om = np.ascontiguousarray(om[0])
        m = om.shape[0]
    else:
        if om.shape[0] != H:
            raise ValueError("omega must be [m, d], [1, m, d] or [H, m, d]")
        per_head = 1
        m = om.shape[1]
    out = np.empty((B, H, L, d), dtype=np.float64)
    rc = getattr(lib, name)(B, H, L, d, m, _dptr(q), _dptr(k), _dptr(v), _dptr(om), per_head, _dptr(out))
    if rc != 0:
        raise MemoryError(f"{name} failed to allocate")
    return out


def bidir(q, k, v, omega) -> np.ndarray:
    """Bidirectional FAVOR+ in plain C (fp64); inputs [B, H, L, d]."""
    return _attn("oracle_bidir", q, k, v, omega)


def causal(q, k, v, omega) -> np.ndarray:
    """Causal FAVOR+ in plain C (fp64) by the per-token prefix recurrence."""
    return _attn("oracle_causal", q, k, v, omega)
