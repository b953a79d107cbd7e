"""Camera conventions of the flashdrr front end, written out plainly in numpy --
TEST INFRASTRUCTURE ONLY (same rules as the rest of ``oracle``: only ``tests/``,
the smoke check and the benchmark's CPU leg import it; it shares nothing with the
HIP library).

Passages (source pages):
  * flashdrr API, get_vtk_view_mat: a camera-to-world 4 x 4 whose 3 x 3 block
    holds the camera axes as columns [right, up, forward] (forward from the camera
    towards the focal point) and whose fourth column is the camera position, all
    in RAS world coordinates.
  * flashdrr API, VolumeRaycaster.forward: the volume lives in IJK voxel space and
    a 4 x 4 affine ras2ijk maps RAS to IJK.
  * flashdrr API, VolumeRaycaster.__init__ / set_fov: fov is the vertical field of
    view in degrees from which the per-pixel ray directions are built.
  * nanodrr page, introduction: the Hartley-Zisserman pinhole camera P = K [R | t].

Readings (the pages give no formulas):
  * IJK is the continuous voxel index with voxel centres at integers, i along the
    volume's fastest axis (x), j along y, k along z;
  * the box of the rendering frame is centred on the volume, so a RAS point X
    sits at p = diag(s) (ras2ijk X - (n - 1) / 2) with s_a the voxel size along
    axis a (1 / the norm of row a of ras2ijk's linear part), which is a rigid
    map when the voxel axes are orthogonal;
  * the HZ camera's image x axis is the VTK camera's right and its image y axis
    is down, i.e. minus up, and z is forward: the world-to-camera rotation has
    rows [right; -up; forward] (whatever the handedness of [right, up, forward]);
    the 3 x 3 block is taken as orthonormal, so the rigid inverse (transpose) is
    used;
  * K = [[f, 0, W/2], [0, f, H/2], [0, 0, 1]] with f = (H / 2) / tan(fov / 2).
"""
from __future__ import annotations

import numpy as np


def intrinsics_from_fov(fov_deg: float, det_h: int, det_w: int) -> np.ndarray:
    """[fd-fov] vertical field of view -> HZ intrinsics (fp64)."""
    f = (det_h / 2.0) / np.tan(np.radians(fov_deg) / 2.0)
    return np.array([[f, 0.0, det_w / 2.0], [0.0, f, det_h / 2.0], [0.0, 0.0, 1.0]])


def frame_from_ras(ras2ijk, shape):
    """The rigid map RAS -> rendering frame as a 4 x 4 (fp64) and the voxel sizes
    (sx, sy, sz).  shape = (nz, ny, nx)."""
    A = np.asarray(ras2ijk, dtype=np.float32).astype(np.float64).reshape(4, 4)
    nz, ny, nx = shape
    s = 1.0 / np.linalg.norm(A[:3, :3], axis=1)
    c = np.array([(nx - 1) / 2.0, (ny - 1) / 2.0, (nz - 1) / 2.0])
    to_index = A
    centre = np.eye(4)
    centre[:3, 3] = -c
    scale = np.diag([s[0], s[1], s[2], 1.0])
    return scale @ centre @ to_index, s


def pose_from_view_matrix(view_mat, ras2ijk, shape) -> np.ndarray:
    """World-to-camera HZ poses (V, 3, 4) in the rendering frame for VTK
    camera-to-world view matrices (V, 4, 4) (fp64 from the fp32 inputs)."""
    Vm = np.asarray(view_mat, dtype=np.float32).astype(np.float64).reshape(-1, 4, 4)
    T, _ = frame_from_ras(ras2ijk, shape)
    T_inv = np.linalg.inv(T)                       # rendering frame -> RAS
    flip = np.diag([1.0, -1.0, 1.0, 1.0])          # VTK camera (x right, y up) -> HZ (y down)
    out = np.zeros((Vm.shape[0], 3, 4))
    for v, M in enumerate(Vm):
        w2c = np.eye(4)
        w2c[:3, :3] = M[:3, :3].T                  # rigid inverse of the camera-to-world
        w2c[:3, 3] = -M[:3, :3].T @ M[:3, 3]
        out[v] = (flip @ w2c @ T_inv)[:3]
    return out


def view_matrix_gradient(view_mat, ras2ijk, shape, grad_poses) -> np.ndarray:
    """dL/d(view_mat) (V, 4, 4) for L = sum(grad_poses * pose_from_view_matrix):
    central differences over the twelve upper entries.  The pose is a polynomial
    of degree 2 in those entries (R is linear in the rotation block, t bilinear
    in the block and the position), so a central difference is exact for any
    step up to rounding; the bottom row gets 0."""
    Vm = np.asarray(view_mat, dtype=np.float32).astype(np.float64).reshape(-1, 4, 4)
    G = np.asarray(grad_poses, dtype=np.float64).reshape(-1, 3, 4)
    out = np.zeros_like(Vm)
    h = 0.5
    for v in range(Vm.shape[0]):
        for r in range(3):
            for c in range(4):
                P, M = Vm[v].copy(), Vm[v].copy()
                P[r, c] += h
                M[r, c] -= h
                lp = float((_pose64(P, ras2ijk, shape) * G[v]).sum())
                lm = float((_pose64(M, ras2ijk, shape) * G[v]).sum())
                out[v, r, c] = (lp - lm) / (2.0 * h)
    return out


def _pose64(M, ras2ijk, shape):
    """pose_from_view_matrix on an fp64 matrix without rounding it to fp32."""
    T, _ = frame_from_ras(ras2ijk, shape)
    flip = np.diag([1.0, -1.0, 1.0, 1.0])
    w2c = np.eye(4)
    w2c[:3, :3] = M[:3, :3].T
    w2c[:3, 3] = -M[:3, :3].T @ M[:3, 3]
    return (flip @ w2c @ np.linalg.inv(T))[:3]
