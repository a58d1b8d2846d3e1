"""The feature map with the one rounding the bf16 matrix-core path needs:
the projection operand log2(e) * omega in bf16 (round to nearest even),
everything else in fp64.  At d = 16 the library carries that operand as a
high and a low bf16 part (the padding half of the 32-deep contraction holds
the low part), so there the operand is hi + lo.  Used to check that the
library's bf16 features differ from the definition by that rounding alone
(fp32-level agreement), a much tighter statement than the 2e-2 bar against
the exact definition."""

import numpy as np

LOG2E = float(np.log2(np.e))


def round_bf16(a: np.ndarray) -> np.ndarray:
    """fp32 values of ``a`` rounded to bf16 (nearest even), as float64."""
    bits = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((bits + 0x7FFF + ((bits >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)
    return r.view(np.float32).astype(np.float64)


def projection_operand(omega: np.ndarray) -> np.ndarray:
    """log2(e) * omega as the bf16 path carries it: one bf16 value per entry,
    or at d = 16 the sum of a high and a low bf16 part (float64)."""
    v = (np.asarray(omega, dtype=np.float64) * LOG2E).astype(np.float32)
    hi = round_bf16(v)
    if omega.shape[-1] != 16:
        return hi
    return hi + round_bf16((v.astype(np.float64) - hi).astype(np.float32))


def features_bf16_operand(x: np.ndarray, omega: np.ndarray) -> np.ndarray:
    """m^-1/2 exp(omega x - |x|^2 / 2) with log2(e) omega as the bf16 path
    carries it (``projection_operand``); ``x`` [..., L, d], ``omega`` [m, d];
    float64 [..., L, m]."""
    x = np.asarray(x, dtype=np.float64)
    m = omega.shape[-2]
    o = projection_operand(omega)
    p = x @ o.T - LOG2E * 0.5 * (x * x).sum(-1)[..., None] - 0.5 * np.log2(m)
    return 2.0 ** p


def fp32_feature_bound(x: np.ndarray, omega: np.ndarray) -> float:
    """A-priori bound on the relative error of fp32 features against
    ``features_bf16_operand``: each exponent is a sum of d + 2 terms (the d
    products, the norm term and a shift), whose fp32 evaluation in any order
    is off by at most gamma_n = n u / (1 - n u) times the sum of the terms'
    magnitudes (u = 2^-24, n = d + 4 to cover the stabiliser's subtraction
    and its scale), and exp2 scales an exponent error e into a relative error
    of ln(2) e; plus a few units in the last place for the exponential and
    the final rounding."""
    x = np.asarray(x, dtype=np.float64)
    o = projection_operand(omega)
    mag = LOG2E * 0.5 * (x * x).sum(-1)[..., None] + np.abs(x) @ np.abs(o).T
    n = x.shape[-1] + 4
    u = 2.0 ** -24
    gamma = n * u / (1 - n * u)
    return float(np.log(2.0) * gamma * mag.max() + 8 * u)
