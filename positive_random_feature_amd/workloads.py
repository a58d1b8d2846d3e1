"""Seeded synthetic inputs for the FAVOR+ workloads.

This module only draws and stores numbers: Q, K and V as i.i.d. Gaussians,
scaled and rounded to the storage dtype.  It holds none of the method's
arithmetic (no features, no projection, no orthogonalisation), so that the
GPU path and the CPU oracle can both consume exactly the same arrays.

Recipe (one numpy PCG64 stream seeded ``[seed, 1]``, drawn in the order Q, K,
V, each row-major ``[B, H, L, d]`` in float64):

* Q, K ~ N(0, sigma^2) with sigma = qk_scale * d**-1/4 (qk_scale is 1, or 1.5
  for the large-norm stress workload); V ~ N(0, 1).
* float64 -> float32 (round to nearest even), then for bf16 workloads
  float32 -> bf16 (round to nearest even).  The values the kernels read are
  exactly the values returned here.

The random projection Omega is not drawn here: it comes from a seeded
orthogonal-random-feature generator (the library's for benchmarks, the
oracle's for parity tests; both implement the same counter-based generator).
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    op: str            # "bidir" or "causal"
    B: int
    H: int
    L: int
    d: int
    m: int
    dtype: str         # "f32" or "bf16"
    qk_scale: float    # sigma of Q, K entries is qk_scale * d**-0.25
    omega_per_head: bool
    seed: int = 0
    chunk: int = 0     # causal chunk length; 0 = library default

    @property
    def tokens(self) -> int:
        return self.B * self.H * self.L

    def replace(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


# The five workloads (small fp32 case; long bidirectional; long causal;
# image-length bidirectional; large-norm very long causal).
WORKLOADS = {
    "bidir_f32_tiny": Workload("bidir_f32_tiny", "bidir", 1, 1, 256, 16, 32, "f32", 1.0, False),
    "bidir_bf16_4k": Workload("bidir_bf16_4k", "bidir", 4, 8, 4096, 64, 256, "bf16", 1.0, False),
    "causal_bf16_8k": Workload("causal_bf16_8k", "causal", 2, 8, 8192, 64, 256, "bf16", 1.0, True),
    "bidir_bf16_12k": Workload("bidir_bf16_12k", "bidir", 1, 8, 12288, 64, 256, "bf16", 1.0, True),
    "causal_bf16_64k": Workload("causal_bf16_64k", "causal", 1, 16, 65536, 128, 512, "bf16", 1.5, True),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    nan = np.isnan(x)
    out = rounded.astype(np.uint16)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bits to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclass
class Inputs:
    """Q, K, V as the kernels read them.

    ``q, k, v`` are float32 arrays holding exactly the stored values (already
    bf16-representable for bf16 workloads); ``q_bits`` etc. hold the bf16 bit
    patterns for bf16 workloads and are None for f32 workloads.
    """

    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    q_bits: np.ndarray | None = None
    k_bits: np.ndarray | None = None
    v_bits: np.ndarray | None = None


def make_inputs(w: Workload, B: int | None = None, H: int | None = None, L: int | None = None,
                seed: int | None = None) -> Inputs:
    """Draw Q, K, V for workload ``w`` (optionally with a smaller B, H or L)."""
    B = w.B if B is None else B
    H = w.H if H is None else H
    L = w.L if L is None else L
    seed = w.seed if seed is None else seed
    shape = (B, H, L, w.d)
    rng = np.random.Generator(np.random.PCG64([seed, 1]))
    sigma = w.qk_scale * float(w.d) ** -0.25
    out = []
    for scale in (sigma, sigma, 1.0):
        x = rng.standard_normal(size=shape, dtype=np.float64)
        x *= scale
        out.append(x.astype(np.float32))
        del x
    q, k, v = out
    if w.dtype == "bf16":
        bits = [f32_to_bf16_bits(t) for t in (q, k, v)]
        vals = [bf16_bits_to_f32(b) for b in bits]
        return Inputs(*vals, *bits)
    return Inputs(q, k, v)
