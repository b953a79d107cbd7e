"""Pins for the oracle's Gaussian-Poisson surrogate (flashdrr API,
VolumeRaycaster.apply_poisson: Gaussian noise of standard deviation sqrt(T / i0)
added to a transmission map, clamped to [0, 1]).  The standard-normal draws are an
input.  Pinned by: zero draws leave T unchanged; the noise's mean and standard
deviation over many draws (the definition of the surrogate); one draw worked by
hand; the clamp at both ends; finite differences of the map for the gradient,
including the clamped region and T <= 0."""
import math

import numpy as np
import pytest

import oracle


def test_zero_draws_are_the_identity_inside_the_unit_interval():
    T = np.linspace(0.0, 1.0, 101)
    out = oracle.poisson_surrogate(T, np.zeros_like(T), 1e4)
    assert np.array_equal(out, T)


def test_noise_has_standard_deviation_sqrt_t_over_i0():
    rng = np.random.default_rng(0)
    for t, i0 in [(0.3, 1e3), (0.05, 2e4), (0.7, 5e2)]:
        z = rng.standard_normal(400_000)
        out = oracle.poisson_surrogate(np.full_like(z, t), z, i0)
        noise = out - t
        assert abs(noise.mean()) < 5 * math.sqrt(t / i0) / math.sqrt(z.size)
        assert noise.std() == pytest.approx(math.sqrt(t / i0), rel=5e-3)


def test_one_draw_by_hand_and_the_clamp():
    out = oracle.poisson_surrogate(np.array([0.25, 0.9, 0.02, -0.1]),
                                   np.array([1.5, 3.0, -4.0, 2.0]), 100.0)
    assert out[0] == pytest.approx(0.25 + 1.5 * 0.05, rel=1e-15)       # sqrt(0.25/100) = 0.05
    assert out[1] == 1.0                                                  # 0.9 + 3 * 0.0949 > 1
    assert out[2] == 0.0                                                  # 0.02 - 4 * 0.0141 < 0
    assert out[3] == 0.0                                                  # T < 0: no noise, clamped


def test_gradient_matches_central_differences():
    rng = np.random.default_rng(1)
    T = rng.uniform(-0.05, 1.05, size=2000)
    z = rng.standard_normal(T.size)
    g = rng.normal(size=T.size)
    i0 = 300.0
    _, grad = oracle.poisson_surrogate(T, z, i0, g)
    h = 1e-7
    fd = (oracle.poisson_surrogate(T + h, z, i0) - oracle.poisson_surrogate(T - h, z, i0)) / (2 * h) * g
    # skip points within h of a kink (clamp edges, T = 0)
    v = T + z * np.sqrt(np.maximum(T, 0) / i0)
    smooth = (np.abs(v) > 1e-5) & (np.abs(v - 1) > 1e-5) & (T > 1e-5)
    assert smooth.sum() > 1500
    assert np.allclose(grad[smooth], fd[smooth], rtol=1e-6, atol=1e-8)
    assert np.all(grad[(v < 0) | (v > 1)] == 0.0)
