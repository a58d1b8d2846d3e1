"""The Python binding rejects malformed tensors on the host, before any
device is touched: mismatched q/k/v shapes, a wrong output or workspace, a
projection of the wrong shape (each would otherwise make the kernels read or
write out of bounds)."""

import pytest
import torch

import positive_random_feature_amd as favor


def _qkv(B=1, H=2, L=64, d=64, dtype=torch.bfloat16):
    return [torch.zeros(B, H, L, d, dtype=dtype) for _ in range(3)]


OM = torch.zeros(256, 64)


@pytest.mark.parametrize("fn", [favor.bidir, favor.causal])
def test_shape_mismatch(fn):
    q, k, v = _qkv()
    with pytest.raises(ValueError, match="one shape"):
        fn(q, k[:, :, :32].contiguous(), v, OM)
    with pytest.raises(ValueError, match="one shape"):
        fn(q, k, torch.zeros(1, 2, 64, 32, dtype=torch.bfloat16), OM)
    with pytest.raises(ValueError, match="one dtype"):
        fn(q, k.float(), v, OM)
    with pytest.raises(ValueError, match="contiguous"):
        fn(q, k.transpose(2, 3).contiguous().transpose(2, 3), v, OM)
    with pytest.raises(ValueError, match=r"\[B, H, L, d\]"):
        fn(q[0], k[0], v[0], OM)
    with pytest.raises(TypeError):
        fn(*(t.half() for t in (q, k, v)), OM)


@pytest.mark.parametrize("fn", [favor.bidir, favor.causal])
def test_bad_out(fn):
    q, k, v = _qkv()
    for out in (torch.zeros(1, 2, 32, 64, dtype=torch.bfloat16),   # too small
                torch.zeros(1, 2, 64, 64, dtype=torch.float32),    # wrong dtype
                torch.zeros(1, 2, 64, 128, dtype=torch.bfloat16)[..., ::2]):  # not contiguous
        with pytest.raises(ValueError, match="out must be"):
            fn(q, k, v, OM, out=out)


@pytest.mark.parametrize("fn", [favor.bidir, favor.causal])
def test_bad_workspace(fn):
    q, k, v = _qkv()
    for ws in (torch.zeros(1024, dtype=torch.float32), torch.zeros(4, 256, dtype=torch.uint8),
               torch.zeros(2048, dtype=torch.uint8)[::2]):
        with pytest.raises(ValueError, match="workspace"):
            fn(q, k, v, OM, workspace=ws)


@pytest.mark.parametrize("fn", [favor.bidir, favor.causal])
def test_bad_omega(fn):
    q, k, v = _qkv()
    for om in (torch.zeros(256, 32), torch.zeros(3, 256, 64), torch.zeros(256 * 64),
               torch.zeros(256, 64, dtype=torch.float64)):
        with pytest.raises(ValueError, match="omega"):
            fn(q, k, v, om)


@pytest.mark.parametrize("fn", [favor.bidir, favor.causal])
def test_host_tensors_rejected(fn):
    """Well-formed tensors that live in host memory are refused, not launched."""
    q, k, v = _qkv()
    with pytest.raises(ValueError, match="GPU"):
        fn(q, k, v, OM)
