"""Pins of the oracle's cell-constant (Siddon) model against what the pages and
the mathematics fix, independently of the oracle's own code.

The model (diffct 2.1.0, "Why diffct" feature list: project/backproject are an
exact adjoint pair for the cell-constant Siddon model): every voxel is a
constant box, and a ray's line integral is sum_v mu_v l_v with l_v the exact
length of the clipped ray inside voxel v.  The oracle implements it as the
merged-crossing traversal; the pins below rebuild l_v by brute force (one slab
test per voxel box, numpy), by closed forms, or by a nearest-voxel midpoint
rule with many samples.
"""
import numpy as np
import pytest

import oracle
import workloads as W


# ----------------------------------------------------------------- brute force

def numpy_ray(K, pose, r, c):
    """Camera centre and unit direction of pixel (r, c), written out from the
    pinhole model: C = -R^T t, d = R^T K^-1 (c + 1/2, r + 1/2, 1), normalised."""
    K = np.asarray(K, dtype=np.float32).astype(np.float64)
    P = np.asarray(pose, dtype=np.float32).astype(np.float64).reshape(3, 4)
    R, t = P[:, :3], P[:, 3]
    d = R.T @ np.linalg.solve(K, np.array([c + 0.5, r + 0.5, 1.0]))
    return -R.T @ t, d / np.linalg.norm(d)


def voxel_lengths(shape, spacing, C, d):
    """Length of the ray C + t d, t >= 0, inside every voxel box, by one slab
    test per box (no traversal): l = max(0, min(exit) - max(entry, 0))."""
    nz, ny, nx = shape
    s = np.asarray(spacing, dtype=np.float32).astype(np.float64)
    n = (nx, ny, nz)
    E = np.array([n[a] * s[a] for a in range(3)])
    entry, exit_ = [], []
    for a in range(3):
        lo = np.arange(n[a]) * s[a] - E[a] / 2
        hi = lo + s[a]
        if d[a] == 0.0:
            inside = (C[a] >= lo) & (C[a] < hi)
            entry.append(np.where(inside, -np.inf, np.inf))
            exit_.append(np.where(inside, np.inf, -np.inf))
        else:
            ta, tb = (lo - C[a]) / d[a], (hi - C[a]) / d[a]
            entry.append(np.minimum(ta, tb))
            exit_.append(np.maximum(ta, tb))
    # broadcast to (nz, ny, nx)
    ent = np.maximum(np.maximum(entry[2][:, None, None], entry[1][None, :, None]),
                     entry[0][None, None, :])
    ext = np.minimum(np.minimum(exit_[2][:, None, None], exit_[1][None, :, None]),
                     exit_[0][None, None, :])
    return np.maximum(0.0, ext - np.maximum(ent, 0.0))


def dense_matrix(w):
    """A[ray, voxel] = l_v for every ray of a small workload, by brute force."""
    rows = []
    for v in range(w.n_views):
        for r in range(w.det_h):
            for c in range(w.det_w):
                C, d = numpy_ray(w.K, w.poses[v], r, c)
                rows.append(voxel_lengths(w.volume.shape, w.spacing, C, d).ravel())
    return np.array(rows)


def rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


CASES = [
    dict(seed=301, shape=(5, 6, 7), det=(4, 5), n_views=2),
    dict(seed=302, shape=(3, 8, 4), det=(6, 3), n_views=2, spacing=(0.7, 1.3, 1.1)),
    dict(seed=303, shape=(6, 6, 6), det=(5, 5), n_views=1, distance=2.0, rot_deg=80.0),
]


def small(case, mode=W.LINE_INTEGRAL):
    kw = dict(case)
    seed = kw.pop("seed")
    return W.make_random_small(seed, n_samples=1, mode=mode, **kw)


@pytest.mark.parametrize("case", CASES)
def test_siddon_forward_equals_brute_force_lengths(case):
    w = small(case)
    A = dense_matrix(w)
    assert np.count_nonzero(A.sum(axis=1)) > 0
    _, s = oracle.siddon_forward_workload(w)
    assert rel(s.ravel(), A @ w.volume.astype(np.float64).ravel()) < 1e-12


@pytest.mark.parametrize("case", CASES)
def test_siddon_adjoint_equals_brute_force_transpose(case):
    w = small(case)
    A = dense_matrix(w)
    g = w.grad_out.astype(np.float64).ravel()
    grad, _ = oracle.siddon_adjoint_workload(w)
    assert rel(grad.ravel(), A.T @ g) < 1e-12


def test_source_inside_case_starts_at_the_source():
    w = small(CASES[2])
    nz, ny, nx = w.volume.shape
    C, _ = numpy_ray(w.K, w.poses[0], 0, 0)
    sp = np.asarray(w.spacing, dtype=np.float64)
    assert np.all(np.abs(C) < 0.5 * np.array([nx, ny, nz]) * sp)


def test_siddon_beer_lambert_gradient_by_brute_force():
    """Beer-Lambert adjoint = A^T (g exp(-A mu)) with the brute-force A."""
    w = small(CASES[0], mode=W.BEER_LAMBERT)
    w.volume = (0.1 * w.volume).astype(np.float32)
    A = dense_matrix(w)
    s = A @ w.volume.astype(np.float64).ravel()
    img, _ = oracle.siddon_forward_workload(w)
    assert rel(img.ravel(), -np.expm1(-s)) < 1e-12
    grad, _ = oracle.siddon_adjoint_workload(w)
    want = A.T @ (w.grad_out.astype(np.float64).ravel() * np.exp(-s))
    assert rel(grad.ravel(), want) < 1e-12


def test_siddon_finite_differences_beer_lambert():
    """Central differences of L = sum g I in a few voxels (I is linear in mu
    inside the exponent, so the difference quotient is accurate to h^2)."""
    w = small(CASES[1], mode=W.BEER_LAMBERT)
    vol = (0.2 * w.volume).astype(np.float64)
    g = w.grad_out.astype(np.float64)
    grad, _ = oracle.siddon_adjoint(vol.astype(np.float32), vol.shape, w.spacing, w.K, w.poses,
                                    w.det_h, w.det_w, W.BEER_LAMBERT, g)
    rng = np.random.default_rng(5)
    h = 1e-3
    for idx in zip(*(rng.integers(0, n, 6) for n in vol.shape)):
        lp, lm = vol.copy(), vol.copy()
        lp[idx] += h
        lm[idx] -= h
        # fp32 volume: perturb in a way fp32 represents, then divide by the
        # perturbation actually applied
        lp32, lm32 = lp.astype(np.float32), lm.astype(np.float32)
        dh = float(lp32[idx]) - float(lm32[idx])
        ip, _ = oracle.siddon_forward(lp32, w.spacing, w.K, w.poses, w.det_h, w.det_w,
                                      W.BEER_LAMBERT)
        im, _ = oracle.siddon_forward(lm32, w.spacing, w.K, w.poses, w.det_h, w.det_w,
                                      W.BEER_LAMBERT)
        fd = float(np.sum(g * (ip - im))) / dh
        # the other voxels also moved by the fp32 rounding of vol: use the
        # unperturbed fp32 copy as the base for both sides
        assert fd == pytest.approx(grad[idx], rel=1e-6, abs=1e-9)


def test_siddon_axis_aligned_column_sum():
    """A ray parallel to z through the inside of voxel column (i, j) crosses
    every slice over its full depth: s = s_z sum_k mu[k, j, i]."""
    rng = np.random.default_rng(11)
    nz, ny, nx = 7, 5, 4
    vol = rng.uniform(0.0, 1.0, size=(nz, ny, nx)).astype(np.float32)
    sp = np.array([1.0, 1.25, 0.8], dtype=np.float32)
    E = np.array([nx, ny, nz]) * sp.astype(np.float64)
    i, j = 2, 3
    # camera on the column's axis, offset inside the voxel, 100 mm before the box
    x = (i + 0.3) * float(sp[0]) - E[0] / 2
    y = (j + 0.6) * float(sp[1]) - E[1] / 2
    Cw = np.array([x, y, -100.0])
    pose = W.pose_from_rotation_and_centre(np.eye(3), Cw)[None]
    # principal point on the centre of pixel (2, 3) so that ray is along +z
    K = np.array([[50.0, 0.0, 3.5], [0.0, 50.0, 2.5], [0.0, 0.0, 1.0]], dtype=np.float32)
    _, s = oracle.siddon_forward(vol, sp, K, pose, 5, 7, W.LINE_INTEGRAL)
    want = float(sp[2]) * vol[:, j, i].astype(np.float64).sum()
    assert s[0, 2, 3] == pytest.approx(want, rel=1e-13)
    # and reversed (camera beyond the far face looking along -z)
    Rz = np.diag([1.0, -1.0, -1.0])       # camera z axis = world -z
    Cw2 = np.array([x, y, 100.0])
    pose2 = W.pose_from_rotation_and_centre(Rz, Cw2)[None]
    _, s2 = oracle.siddon_forward(vol, sp, K, pose2, 5, 7, W.LINE_INTEGRAL)
    assert s2[0, 2, 3] == pytest.approx(want, rel=1e-13)


def test_siddon_constant_volume_gives_the_chord():
    """mu = c everywhere: sum_v c l_v = c (t1 - t0) (lengths tile the chord)."""
    w = W.make_random_small(321, shape=(9, 10, 11), n_views=3, det=(12, 9), n_samples=1,
                            mode=W.LINE_INTEGRAL)
    w.volume = np.full(w.volume.shape, 0.37, dtype=np.float32)
    _, s = oracle.siddon_forward_workload(w)
    chord = oracle.chords_workload(w)
    assert np.count_nonzero(chord) > 50
    assert rel(s, float(np.float32(0.37)) * chord) < 1e-13


def test_siddon_limit_of_nearest_voxel_midpoint_rule():
    """The N-sample midpoint rule of the cell-constant field (each sample reads
    the voxel that contains it) approaches sum mu_v l_v; each plane crossing
    misplaces at most one sample, so |s_N - s| <= crossings * max mu * dz."""
    w = W.make_random_small(331, shape=(6, 7, 8), n_views=1, det=(5, 6), n_samples=1,
                            mode=W.LINE_INTEGRAL)
    _, s = oracle.siddon_forward_workload(w)
    nz, ny, nx = w.volume.shape
    sp = np.asarray(w.spacing, dtype=np.float32).astype(np.float64)
    E = np.array([nx, ny, nz]) * sp
    vol = w.volume.astype(np.float64)
    N = 200_000
    checked = 0
    for r in range(w.det_h):
        for c in range(w.det_w):
            hit, C, d, t0, t1 = oracle.ray(w.K, w.poses[0], E, r, c)
            if not hit:
                assert s[0, r, c] == 0.0
                continue
            dz = (t1 - t0) / N
            t = t0 + (np.arange(N) + 0.5) * dz
            p = C[None, :] + t[:, None] * d[None, :]
            idx = np.floor((p + E / 2) / sp).astype(np.int64)
            idx = np.clip(idx, 0, np.array([nx, ny, nz]) - 1)
            sN = dz * vol[idx[:, 2], idx[:, 1], idx[:, 0]].sum()
            crossings = nx + ny + nz + 3
            assert abs(sN - s[0, r, c]) <= crossings * vol.max() * dz
            checked += 1
    assert checked > 10


def test_siddon_adjoint_identity_aggregate():
    """<A x, y> = <x, A^T y> over random pairs (torchtomo: report an aggregate
    residual), in fp64."""
    w = W.make_random_small(341, shape=(8, 9, 7), n_views=2, det=(11, 13), n_samples=1,
                            mode=W.LINE_INTEGRAL)
    rng = np.random.default_rng(3)
    lhs, rhs = [], []
    for _ in range(10):
        x = rng.standard_normal(w.volume.shape).astype(np.float32)
        y = rng.standard_normal((w.n_views, w.det_h, w.det_w))
        _, Ax = oracle.siddon_forward(x, w.spacing, w.K, w.poses, w.det_h, w.det_w,
                                      W.LINE_INTEGRAL)
        ATy, _ = oracle.siddon_adjoint(None, x.shape, w.spacing, w.K, w.poses, w.det_h, w.det_w,
                                       W.LINE_INTEGRAL, y)
        lhs.append(float(np.sum(Ax * y)))
        rhs.append(float(np.sum(x.astype(np.float64) * ATy)))
    lhs, rhs = np.array(lhs), np.array(rhs)
    assert np.linalg.norm(lhs - rhs) / np.linalg.norm(lhs) < 1e-12


def test_siddon_and_trilinear_agree_on_constant_and_differ_otherwise():
    """Both models integrate a constant volume to mu * chord; on a random
    volume they are different operators (guards against one calling the other)."""
    w = W.make_random_small(351, shape=(6, 6, 6), n_views=1, det=(6, 6), n_samples=64,
                            mode=W.LINE_INTEGRAL)
    _, s_sid = oracle.siddon_forward_workload(w)
    _, s_tri = oracle.forward_workload(w)
    assert np.max(np.abs(s_sid - s_tri)) > 1e-3
    w.volume = np.full(w.volume.shape, 0.5, dtype=np.float32)
    _, s_sid = oracle.siddon_forward_workload(w)
    _, s_tri = oracle.forward_workload(w)
    assert rel(s_sid, s_tri) < 1e-12
