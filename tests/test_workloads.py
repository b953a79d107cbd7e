"""Host-side checks of the seeded input generators (no method arithmetic here)."""
import math

import numpy as np
import pytest
import torch

import workloads as W


def test_generators_are_deterministic():
    a = W.make_workload(1)
    b = W.make_workload(1)
    assert np.array_equal(a.volume, b.volume)
    assert np.array_equal(a.poses, b.poses)
    c = W.make_random_small(3)
    d = W.make_random_small(3)
    assert np.array_equal(c.volume, d.volume) and np.array_equal(c.grad_out, d.grad_out)


def test_shapes_and_dtypes():
    w = W.make_workload(1)
    assert w.volume.shape == (64, 64, 64) and w.volume.dtype == np.float32
    assert w.poses.shape == (1, 3, 4) and w.poses.dtype == np.float32
    assert (w.det_h, w.det_w, w.n_samples, w.mode) == (64, 64, 128, W.BEER_LAMBERT)
    assert w.volume.flags["C_CONTIGUOUS"]
    # sphere of mu 0.02 plus U[0, 0.005) noise everywhere
    assert 0.0 <= w.volume.min() and w.volume.max() < 0.025
    assert abs(float(w.volume[32, 32, 32]) - 0.02) < 0.0051


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.uniform(0, 1, 10000), rng.normal(0, 1e-3, 10000),
                        [0.0, 1.0, 0.02, 0.05, 1.00390625, 1.01171875]]).astype(np.float32)
    ours = W.round_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_transfer_function_knots_and_extension():
    hu = np.array([-1000.0, 0.0, 1500.0, -1500.0, 3000.0, 40.0])
    mu = W.piecewise_linear(hu, W.HU_KNOTS, W.MU_KNOTS)
    assert np.allclose(mu[:3], [0.0, 0.02, 0.05])
    # end segments extended
    assert mu[3] == pytest.approx(-0.01)
    assert mu[4] == pytest.approx(0.08)
    assert mu[5] == pytest.approx(0.02 * 1.04)


def test_random_poses_are_rotations_facing_the_origin():
    P = W.random_poses(16, 510.0, 30.0, 10.0, seed=2002)
    for p in P.astype(np.float64):
        R, t = p[:, :3], p[:, 3]
        assert np.allclose(R @ R.T, np.eye(3), atol=1e-6)
        assert np.linalg.det(R) == pytest.approx(1.0, abs=1e-6)
        C = -R.T @ t
        assert 450.0 < np.linalg.norm(C) < 570.0
        # the origin lies in front of the camera, near the optical axis
        xc = R @ np.zeros(3) + t
        assert xc[2] > 400.0 and abs(xc[0]) < 60.0 and abs(xc[1]) < 60.0


def test_helical_orbit_geometry():
    P = W.helical_poses(360, 320.0, 40.0, 1.0)
    zs = []
    for k, p in enumerate(P.astype(np.float64)):
        R, t = p[:, :3], p[:, 3]
        C = -R.T @ t
        assert math.hypot(C[0], C[1]) == pytest.approx(320.0, rel=1e-6)
        zs.append(C[2])
        # looking at the rotation axis: the axis point at the source height is straight ahead
        xc = R @ np.array([0.0, 0.0, C[2]]) + t
        assert xc[0] == pytest.approx(0.0, abs=1e-4) and xc[1] == pytest.approx(0.0, abs=1e-4)
        assert xc[2] == pytest.approx(320.0, rel=1e-6)
    assert zs[0] == pytest.approx(-20.0) and zs[-1] == pytest.approx(20.0 - 40.0 / 360, abs=1e-4)
    assert np.all(np.diff(zs) > 0)


def test_phantom_values():
    mu = W.mu_phantom(256)
    assert mu.dtype == np.float32 and mu.shape == (256, 256, 256)
    assert mu.min() >= 0.0
    assert mu[0, 0, 0] == 0.0             # air corner
    assert mu.max() <= 0.02 * 2.5 + 1e-6   # bone up to 1500 HU
    assert mu[128, 128, 128] == pytest.approx(0.02 * 1.04, abs=0.0025)  # soft tissue 40 +- 20 HU
    assert mu.max() > 0.02 * 1.7           # some bone above 700 HU


def test_workload_sizes():
    sizes = {1: (4096, 128), 3: (1048576, 512), 4: (4194304, 256)}
    for i, (rays, n) in sizes.items():
        w = W.make_workload(i)
        assert w.n_rays == rays and w.n_samples == n
    w5 = W.make_workload(5)
    assert w5.poses.shape == (360, 3, 4) and (w5.det_h, w5.det_w) == (256, 384)
    assert w5.mode == W.LINE_INTEGRAL and w5.grad_out.shape == (360, 256, 384)
