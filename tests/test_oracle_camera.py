"""Pins for the oracle's camera conventions (``oracle.camera``): VTK camera-to-world
view matrices, the ras2ijk affine and the vertical field of view, turned into the
HZ poses and intrinsics the renderer takes.

Passages (source pages): flashdrr API, get_vtk_view_mat (camera-to-world, columns
[right, up, forward], fourth column the camera position, forward towards the focal
point); VolumeRaycaster.forward (IJK voxel space, ras2ijk); __init__ / set_fov
(vertical field of view); nanodrr introduction (P = K [R | t]).

The pins are geometric facts, not the oracle's formulas: a look-at camera sees its
focal point at the principal point, its right to the right of the image and its up
at the top; its centre is the camera position; a RAS point lands at the voxel index
ras2ijk gives; the top edge of the image is fov / 2 off the axis; and the view-matrix
gradient composed with the pose gradient equals finite differences of the rendered
image itself.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import camera
import workloads as W


def look_at(pos, focal, up, right_handed):
    f = np.asarray(focal, float) - np.asarray(pos, float)
    f /= np.linalg.norm(f)
    if right_handed:
        r = np.cross(up, f)
        r /= np.linalg.norm(r)
        u = np.cross(f, r)
    else:
        r = np.cross(f, up)
        r /= np.linalg.norm(r)
        u = np.cross(r, f)
    M = np.eye(4)
    M[:3, 0], M[:3, 1], M[:3, 2], M[:3, 3] = r, u, f, pos
    return M.astype(np.float32), r, u, f


def ras2ijk_example():
    """Voxel axes permuted and flipped relative to RAS, anisotropic voxels, an
    offset: i runs along -A (0.8 mm), j along +S (1.25 mm), k along -R (1.0 mm)."""
    A = np.zeros((4, 4))
    A[0, 1] = -1.0 / 0.8
    A[1, 2] = 1.0 / 1.25
    A[2, 0] = -1.0
    A[:3, 3] = [9.0, 4.0, 7.5]
    A[3, 3] = 1.0
    return A.astype(np.float32), np.array([0.8, 1.25, 1.0])


def project(K, pose, p):
    x = np.asarray(K) @ (pose[:, :3] @ p + pose[:, 3])
    return x[:2] / x[2], x[2]


@pytest.mark.parametrize("right_handed", [True, False])
def test_look_at_camera_sees_focal_point_at_principal_point(right_handed):
    A, s = ras2ijk_example()
    shape = (16, 12, 20)
    T, sp = camera.frame_from_ras(A, shape)
    assert np.allclose(sp, s, rtol=1e-6)
    pos, focal = np.array([300.0, -700.0, 150.0]), np.array([5.0, 10.0, -3.0])
    M, r, u, f = look_at(pos, focal, np.array([0.0, 0.0, 1.0]), right_handed)
    pose = camera.pose_from_view_matrix(M, A, shape)[0]
    K = camera.intrinsics_from_fov(20.0, 100, 140)
    to_frame = lambda X: (T @ np.append(X, 1.0))[:3]
    uv, depth = project(K, pose, to_frame(focal))
    assert np.allclose(uv, [70.0, 50.0], atol=1e-4) and depth > 0
    uv_r, _ = project(K, pose, to_frame(focal + 5.0 * r))
    uv_u, _ = project(K, pose, to_frame(focal + 5.0 * u))
    # (tolerances: the view matrix passes the fp32 interface)
    assert uv_r[0] > 70.0 + 1 and abs(uv_r[1] - 50.0) < 1e-4      # right -> larger column
    assert uv_u[1] < 50.0 - 1 and abs(uv_u[0] - 70.0) < 1e-4      # up -> smaller row
    C = -pose[:, :3].T @ pose[:, 3]
    assert np.allclose(C, to_frame(pos), atol=1e-4)
    R = pose[:, :3]
    assert np.allclose(R @ R.T, np.eye(3), atol=1e-6)


def test_ras_point_lands_at_the_voxel_index_of_ras2ijk():
    """The rendering frame's continuous index q = p / s + (n - 1) / 2 of a RAS
    point is ras2ijk applied to it (voxel centres at integers)."""
    A, s = ras2ijk_example()
    shape = (16, 12, 20)
    nz, ny, nx = shape
    T, sp = camera.frame_from_ras(A, shape)
    rng = np.random.default_rng(0)
    for X in rng.uniform(-30, 30, size=(10, 3)):
        p = (T @ np.append(X, 1.0))[:3]
        q = p / sp + np.array([(nx - 1) / 2, (ny - 1) / 2, (nz - 1) / 2])
        assert np.allclose(q, (A.astype(np.float64) @ np.append(X, 1.0))[:3], atol=1e-9)


def test_vertical_field_of_view():
    """The ray through the top edge of the image's centre column is fov/2 off the
    optical axis; the left edge of the centre row is atan((W/2) / f) off it."""
    for fov, H, Wd in [(20.0, 1024, 1024), (35.0, 200, 300)]:
        K = camera.intrinsics_from_fov(fov, H, Wd)
        d = np.linalg.solve(K, [Wd / 2.0, 0.0, 1.0])
        assert math.degrees(math.atan2(abs(d[1]), d[2])) == pytest.approx(fov / 2, rel=1e-12)
        assert K[0, 0] == K[1, 1] and K[0, 2] == Wd / 2 and K[1, 2] == H / 2


def test_view_gradient_is_exact_for_the_quadratic_map():
    """The pose is degree 2 in the view-matrix entries, so central differences do
    not depend on the step: two steps agree to rounding."""
    A, _ = ras2ijk_example()
    rng = np.random.default_rng(1)
    M, *_ = look_at(np.array([100.0, -400.0, 30.0]), np.zeros(3), np.array([0.0, 0.0, 1.0]),
                    True)
    G = rng.normal(size=(1, 3, 4))
    g1 = camera.view_matrix_gradient(M[None], A, (16, 12, 20), G)
    Vm = M.astype(np.float64)
    g2 = np.zeros_like(g1)
    h = 1e-3
    for r in range(3):
        for c in range(4):
            P, Mm = Vm.copy(), Vm.copy()
            P[r, c] += h
            Mm[r, c] -= h
            g2[0, r, c] = ((camera._pose64(P, A, (16, 12, 20)) * G[0]).sum() -
                           (camera._pose64(Mm, A, (16, 12, 20)) * G[0]).sum()) / (2 * h)
    assert np.allclose(g1, g2, rtol=1e-8, atol=1e-9 * np.abs(g1).max())
    assert not g1[:, 3].any()


def test_view_gradient_chains_the_pose_gradient_of_the_image():
    """d(sum g * image)/d(view_mat) through the pose gradient equals central
    differences of the rendered image with respect to the view matrix."""
    rng = np.random.default_rng(2)
    shape = (6, 5, 7)
    vol = rng.uniform(0.0, 1.0, size=shape).astype(np.float32)
    A, _ = ras2ijk_example()
    T, sp = camera.frame_from_ras(A, shape)
    centre_ras = np.linalg.solve(T, [0.0, 0.0, 0.0, 1.0])[:3]
    M, *_ = look_at(centre_ras + np.array([20.0, -35.0, 12.0]), centre_ras,
                    np.array([0.0, 0.0, 1.0]), True)
    K = W.intrinsics(30.0, 4.6, 3.4)
    H, Wd, N = 7, 9, 23
    g = rng.normal(size=(1, H, Wd))

    def loss(Mv):
        pose = camera._pose64(Mv, A, shape)[None]
        img, _ = oracle.forward(vol, sp.astype(np.float32), K, pose, H, Wd, N,
                                oracle.BEER_LAMBERT)
        return float((img * g).sum())

    pose = camera.pose_from_view_matrix(M, A, shape)
    gp = oracle.pose_gradient(vol, sp.astype(np.float32), K, pose, H, Wd, N,
                              oracle.BEER_LAMBERT, g)
    gv = camera.view_matrix_gradient(M[None], A, shape, gp)[0]
    Vm = M.astype(np.float64)
    h = 1e-6
    for r in range(3):
        for c in range(4):
            P, Mm = Vm.copy(), Vm.copy()
            P[r, c] += h
            Mm[r, c] -= h
            fd = (loss(P) - loss(Mm)) / (2 * h)
            assert fd == pytest.approx(gv[r, c], rel=2e-5, abs=2e-6 * np.abs(gv).max())
