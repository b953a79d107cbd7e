"""GPU parity of the Gaussian-Poisson surrogate (flashdrr API,
VolumeRaycaster.apply_poisson) against the oracle: forward values and the gradient
with respect to the transmission, on aligned and misaligned buffers, odd sizes,
values outside [0, 1] and through autograd.  The draws are the same seeded
standard normals on both sides.  Bars: fp32 evaluation of sqrt and one fma, so
|g - o| <= 1e-6 absolute on values in [0, 1]; gradients 1e-5 relative where the
value is away from the clamp edges (a draw that lands within 1e-6 of an edge may
fall on either side in fp32)."""
import numpy as np
import pytest
import torch

import ct_forward_projection_amd as drr
import oracle
from helpers import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


@pytest.mark.parametrize("n,offset", [(1_000_003, 0), (4097, 1), (3, 0), (0, 0)])
def test_surrogate_forward_and_backward(dev, n, offset):
    rng = np.random.default_rng(n + offset)
    T = rng.uniform(-0.05, 1.05, size=n + offset).astype(np.float32)
    z = rng.standard_normal(n + offset).astype(np.float32)
    g = rng.normal(size=n + offset).astype(np.float32)
    i0 = 250.0
    Tt, zt, gt = (torch.from_numpy(a).to(dev)[offset:] for a in (T, z, g))
    say(f"case: surrogate n={n} offset={offset}")
    out = drr.drr_poisson_surrogate(Tt, zt, i0)
    grad = drr.drr_poisson_surrogate_backward(Tt, zt, i0, gt)
    torch.cuda.synchronize()
    ref, ref_g = oracle.poisson_surrogate(T[offset:], z[offset:], i0, g[offset:])
    if n == 0:
        assert out.numel() == 0
        return
    o = out.cpu().double().numpy()
    err = np.abs(o - ref).max()
    v = T[offset:].astype(np.float64) + z[offset:] * np.sqrt(np.maximum(T[offset:], 0) / i0)
    away = (np.abs(v) > 1e-5) & (np.abs(v - 1) > 1e-5)
    gd = grad.cpu().double().numpy()
    gerr = (np.abs(gd - ref_g)[away] / np.maximum(np.abs(ref_g[away]), 1e-3)).max()
    say(f"surrogate n={n}: value err {err:.3e}, gradient rel err {gerr:.3e}")
    assert err <= 1e-6 and gerr <= 1e-5


def test_surrogate_autograd(dev):
    rng = np.random.default_rng(9)
    T = torch.from_numpy(rng.uniform(0, 1, size=(3, 64, 64)).astype(np.float32)).to(dev)
    z = torch.from_numpy(rng.standard_normal((3, 64, 64)).astype(np.float32)).to(dev)
    T.requires_grad_(True)
    out = drr.poisson_noise(T, z, 1e3)
    out.sum().backward()
    torch.cuda.synchronize()
    _, ref_g = oracle.poisson_surrogate(T.detach().cpu().numpy(), z.cpu().numpy(), 1e3,
                                        np.ones((3, 64, 64)))
    assert np.allclose(T.grad.cpu().double().numpy(), ref_g, rtol=1e-5, atol=1e-6)
    assert drr.poisson_noise(T, z, None) is T
