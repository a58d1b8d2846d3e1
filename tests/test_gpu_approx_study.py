"""The approximation study (tests/approx_study.py) on the GPU at the pages'
setting L = 4096, d = 16: every library output (positive features with a
Gaussian orthogonal, a Hadamard and an i.i.d. projection; ReLU features) is
compared with the oracle's bidirectional FAVOR+ on the same projection
(fp32 bar 1e-5); the trigonometric and exact-softmax references are the
oracle's.  Robust findings checked: every error finite and positive;
trigonometric features worse than positive ones by more than 10x at every m
(the pages' reason for positive features, [P1] Theoretical bounds)."""

import math
import os
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import approx_study  # noqa: E402

pytestmark = pytest.mark.gpu


def test_study_library_against_oracle_and_orderings():
    res = approx_study.run(L=4096, d=16, ms=(32, 512), seeds=2, scales=(1.0,), parity_seeds=2,
                           log=lambda s: print(s, flush=True))
    assert res["parity_worst_rel_l2"] <= 1e-5
    mse = res["scales"]["1.0"]["mse"]
    for m in (32, 512):
        for meth in approx_study.METHODS:
            assert math.isfinite(mse[m][meth]["mean"]) and mse[m][meth]["mean"] > 0
        best_trig = min(mse[m]["trig_orf"]["mean"], mse[m]["trig_iid"]["mean"])
        worst_pos = max(mse[m][x]["mean"] for x in ("positive_orf", "positive_hadamard", "positive_iid"))
        assert best_trig > 10 * worst_pos
