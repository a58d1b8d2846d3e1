"""The rounding helper that the tight bf16 feature checks use, pinned on the
CPU: its bf16 rounding equals torch's float32 -> bfloat16 conversion (round
to nearest even, ties included), and with a projection whose log2(e) * omega
is already bf16 it is the oracle's feature map."""

import os
import sys

import numpy as np
import torch

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from bf16_rounding import LOG2E, features_bf16_operand, projection_operand, round_bf16  # noqa: E402

import oracle.reference as ref  # noqa: E402


def test_round_bf16_matches_torch():
    rng = np.random.default_rng(3)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(10.0) ** rng.integers(-6, 6, 20000),
        # exact ties between two bf16 values: low half 0x8000, both parities
        (np.arange(1, 2001, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, -3.0e38, 1e-40], dtype=np.float32),
    ])
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(round_bf16(x), want)


def test_features_helper_is_the_definition_for_bf16_operands():
    rng = np.random.default_rng(4)
    d, m = 32, 64
    om = ref.orf_omega(9, 1, m, d)[0]
    # a projection whose log2(e) * omega is exactly bf16: no rounding left
    om_exact = round_bf16(om * LOG2E) / LOG2E
    np.testing.assert_array_equal(round_bf16(om_exact * LOG2E), round_bf16(om * LOG2E))
    assert np.max(np.abs(round_bf16(om_exact * LOG2E) - om_exact * LOG2E)) < 1e-14
    x = rng.standard_normal((50, d)) * d ** -0.25
    got = features_bf16_operand(x, om_exact)
    want = ref.features(x, om_exact)
    assert np.max(np.abs(got - want) / want) < 1e-12


def test_projection_operand_split_at_d16():
    """At d = 16 the operand is hi + lo: within 2^-16 of log2(e) omega in
    fp32 (bf16 alone: 2^-8), and exactly hi elsewhere."""
    om16 = ref.orf_omega(5, 1, 64, 16)[0]
    v = (om16 * LOG2E).astype(np.float32).astype(np.float64)
    op = projection_operand(om16)
    assert np.max(np.abs(op - v) / np.abs(v)) <= 2.0 ** -16
    assert np.max(np.abs(round_bf16(v) - v) / np.abs(v)) > 2.0 ** -12  # bf16 alone is far coarser
    om32 = ref.orf_omega(5, 1, 64, 32)[0]
    np.testing.assert_array_equal(projection_operand(om32), round_bf16(om32 * LOG2E))
