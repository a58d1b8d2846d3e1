"""ctypes binding of the C ABI in include/favor.h (argument marshalling only)."""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfavor_amd.so")

FAVOR_F32 = 0
FAVOR_BF16 = 1
FAVOR_OP_FEATURES = 0
FAVOR_OP_BIDIR = 1
FAVOR_OP_CAUSAL = 2
FAVOR_N_STAGES = 3
FAVOR_FEATURE_POSITIVE = 0
FAVOR_FEATURE_RELU = 1
FAVOR_NOALLOC_SCRATCH_BYTES = 96 << 20

STATUS = {0: "FAVOR_OK", 1: "FAVOR_ERR_INVALID_ARG", 2: "FAVOR_ERR_UNSUPPORTED", 3: "FAVOR_ERR_WORKSPACE",
          4: "FAVOR_ERR_HIP"}


class FavorShape(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int),
        ("H", ctypes.c_int),
        ("L", ctypes.c_int),
        ("d", ctypes.c_int),
        ("m", ctypes.c_int),
        ("dtype", ctypes.c_int),
        ("omega_head_stride", ctypes.c_longlong),
        ("feature", ctypes.c_int),
    ]


class FavorPlan(ctypes.Structure):
    _fields_ = [
        ("chunk", ctypes.c_int),
        ("segments", ctypes.c_int),
    ]


class FavorError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}")


_lib = None


def load() -> ctypes.CDLL:
    """Load libfavor_amd.so; raise if it has not been built (no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with positive_random_feature_amd.build.build()")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz, sp = ctypes.c_void_p, ctypes.c_size_t, ctypes.POINTER(FavorShape)
    lib.favor_workspace_bytes.restype = sz
    lib.favor_workspace_bytes.argtypes = [ctypes.c_int, sp, ctypes.c_int]
    lib.favor_features.restype = ctypes.c_int
    lib.favor_features.argtypes = [sp, vp, vp, vp, vp, ctypes.c_int, vp, sz, vp]
    lib.favor_bidir.restype = ctypes.c_int
    lib.favor_bidir.argtypes = [sp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.favor_causal.restype = ctypes.c_int
    lib.favor_causal.argtypes = [sp, vp, vp, vp, vp, vp, ctypes.c_int, vp, sz, vp]
    pp = ctypes.POINTER(FavorPlan)
    lib.favor_workspace_bytes_plan.restype = sz
    lib.favor_workspace_bytes_plan.argtypes = [ctypes.c_int, sp, pp]
    lib.favor_bidir_plan.restype = ctypes.c_int
    lib.favor_bidir_plan.argtypes = [sp, vp, vp, vp, vp, vp, pp, vp, sz, vp]
    lib.favor_causal_plan.restype = ctypes.c_int
    lib.favor_causal_plan.argtypes = [sp, vp, vp, vp, vp, vp, pp, vp, sz, vp]
    lib.favor_causal_noalloc.restype = ctypes.c_int
    lib.favor_causal_noalloc.argtypes = [sp, vp, vp, vp, vp, vp, ctypes.c_int, vp]
    lib.favor_causal_state.restype = ctypes.c_int
    lib.favor_causal_state.argtypes = [sp, vp, vp, vp, vp, vp, ctypes.c_int, vp, vp, vp, sz, vp]
    for name, chunk in (("favor_bidir_profiled", False), ("favor_causal_profiled", True)):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [sp, vp, vp, vp, vp, vp] + ([ctypes.c_int] if chunk else []) + [vp, sz, vp,
                                                                                       ctypes.POINTER(vp), ctypes.c_int]
    lib.favor_orf_omega.restype = ctypes.c_int
    lib.favor_orf_omega.argtypes = [ctypes.c_ulonglong, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp]
    lib.favor_hadamard_omega.restype = ctypes.c_int
    lib.favor_hadamard_omega.argtypes = [ctypes.c_ulonglong, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp]
    lib.favor_features_hadamard.restype = ctypes.c_int
    lib.favor_features_hadamard.argtypes = [sp, vp, ctypes.c_ulonglong, vp, vp, ctypes.c_int, vp]
    lib.favor_givens_omega.restype = ctypes.c_int
    lib.favor_givens_omega.argtypes = [ctypes.c_ulonglong, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp,
                                       vp]
    lib.favor_status_string.restype = ctypes.c_char_p
    lib.favor_status_string.argtypes = [ctypes.c_int]
    _lib = lib
    return lib


def shape(B: int, H: int, L: int, d: int, m: int, dtype: int, omega_head_stride: int,
          feature: int = FAVOR_FEATURE_POSITIVE) -> FavorShape:
    return FavorShape(B, H, L, d, m, dtype, omega_head_stride, feature)


def plan(chunk: int = 0, segments: int = 0) -> FavorPlan:
    return FavorPlan(int(chunk), int(segments))


def check(status: int, where: str) -> None:
    if status != 0:
        raise FavorError(status, where)
