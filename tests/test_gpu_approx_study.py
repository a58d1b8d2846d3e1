"""The approximation study (positive_random_feature_amd.approx_study) on the
GPU: FAVOR+ attention through the library against exact softmax attention at
L = 4096, d = 16.  Checked: every error finite; trigonometric features far
worse than positive ones at every m (the pages' reason for positive
features); the Hadamard-projection error falling as m grows."""

import math

import pytest

from positive_random_feature_amd import approx_study

pytestmark = pytest.mark.gpu


def test_study_orders_methods():
    res = approx_study.run(L=4096, d=16, ms=(32, 512), seeds=4)
    mse = res["mse"]
    print(f"[study] {mse}", flush=True)
    for meth in approx_study.METHODS:
        for m in (32, 512):
            assert math.isfinite(mse[meth][m]) and mse[meth][m] > 0
    for m in (32, 512):
        best_trig = min(mse["trig_orf"][m], mse["trig_iid"][m])
        assert best_trig > 10 * max(mse["positive_orf"][m], mse["positive_hadamard"][m], mse["positive_iid"][m])
    assert mse["positive_hadamard"][512] < mse["positive_hadamard"][32]
