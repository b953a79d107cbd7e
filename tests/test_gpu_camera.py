"""GPU parity of the flashdrr camera conventions: VTK camera-to-world view
matrices and a ras2ijk affine turned into HZ poses (``drr_poses_from_view_matrices``),
the chain rule back to the view matrices (``drr_view_matrices_backward``), and a
render driven by them with gradients to the volume and the view matrices
(``render_view_matrices``), all against ``oracle.camera`` and the oracle's forward,
adjoint and pose gradient.

Passages: flashdrr API, get_vtk_view_mat, VolumeRaycaster.forward (ras2ijk),
set_fov; nanodrr introduction (P = K [R | t]).
"""
import numpy as np
import pytest
import torch

import ct_forward_projection_amd as drr
import oracle
from oracle import camera
from helpers import forward_rel_err, normwise_err, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def ras2ijk():
    A = np.zeros((4, 4))
    A[0, 1] = -1.0 / 0.8
    A[1, 2] = 1.0 / 1.25
    A[2, 0] = -1.0
    A[:3, 3] = [9.0, 4.0, 7.5]
    A[3, 3] = 1.0
    return A.astype(np.float32)


def look_at_views(n, centre, dist, seed):
    """Random C-arm-like look-at cameras around ``centre`` (RAS), both
    handednesses of [right, up, forward]."""
    rng = np.random.default_rng(seed)
    out = []
    for v in range(n):
        d = rng.normal(size=3)
        d /= np.linalg.norm(d)
        pos = centre + dist * d
        f = centre - pos
        f /= np.linalg.norm(f)
        up = np.array([0.0, 0.0, 1.0]) + 0.2 * rng.normal(size=3)
        if v % 2:
            r = np.cross(up, f)
            r /= np.linalg.norm(r)
            u = np.cross(f, r)
        else:
            r = np.cross(f, up)
            r /= np.linalg.norm(r)
            u = np.cross(r, f)
        M = np.eye(4)
        M[:3, 0], M[:3, 1], M[:3, 2], M[:3, 3] = r, u, f, pos
        out.append(M)
    return np.stack(out).astype(np.float32)


def test_poses_and_view_gradient_match_the_oracle(dev):
    shape = (16, 12, 20)
    A = ras2ijk()
    T, sp = camera.frame_from_ras(A, shape)
    centre = np.linalg.solve(T, [0.0, 0.0, 0.0, 1.0])[:3]
    views = look_at_views(37, centre, 800.0, 1)
    vm = torch.from_numpy(views).to(dev)
    poses, spacing = drr.drr_poses_from_view_matrices(vm, A, shape)
    torch.cuda.synchronize()
    ref = camera.pose_from_view_matrix(views, A, shape)
    err = np.abs(poses.cpu().double().numpy() - ref).max() / np.abs(ref).max()
    say(f"view matrices -> poses: normwise err {err:.3e}; spacing {spacing}")
    assert err <= 1e-6 and np.allclose(spacing, sp, rtol=1e-6)
    g = np.random.default_rng(2).normal(size=(37, 3, 4)).astype(np.float32)
    gv = drr.drr_view_matrices_backward(vm, A, shape, torch.from_numpy(g).to(dev))
    torch.cuda.synchronize()
    ref_g = camera.view_matrix_gradient(views, A, shape, g)
    err_g = normwise_err(gv.cpu().double().numpy(), ref_g)
    say(f"view-matrix gradient: normwise err {err_g:.3e}")
    assert err_g <= 1e-6


def test_render_from_view_matrices_with_gradients(dev):
    """Images, volume gradient and view-matrix gradient of a render driven by
    VTK view matrices, ras2ijk and a 20 degree field of view."""
    shape = (16, 12, 20)
    A = ras2ijk()
    T, sp = camera.frame_from_ras(A, shape)
    centre = np.linalg.solve(T, [0.0, 0.0, 0.0, 1.0])[:3]
    views = look_at_views(3, centre, 90.0, 3)
    rng = np.random.default_rng(4)
    vol = rng.uniform(0.0, 0.1, size=shape).astype(np.float32)
    H, Wd, N, fov = 33, 41, 48, 20.0
    g = rng.uniform(-1, 1, size=(3, H, Wd)).astype(np.float32)
    v = torch.from_numpy(vol).to(dev).requires_grad_(True)
    vm = torch.from_numpy(views).to(dev).requires_grad_(True)
    say("case: render from view matrices, fov 20, 3 views")
    img = drr.render_view_matrices(v, vm, A, fov, H, Wd, N)
    (img * torch.from_numpy(g).to(dev)).sum().backward()
    torch.cuda.synchronize()
    # the renderer takes poses in fp32: the oracle renders the same rounding of
    # its own poses
    poses = camera.pose_from_view_matrix(views, A, shape).astype(np.float32)
    K = camera.intrinsics_from_fov(fov, H, Wd).astype(np.float32)
    spf = sp.astype(np.float32)
    ref, _ = oracle.forward(vol, spf, K, poses, H, Wd, N, oracle.BEER_LAMBERT)
    ref_gv, _ = oracle.adjoint(vol, shape, spf, K, poses, H, Wd, N, oracle.BEER_LAMBERT, g)
    gp = oracle.pose_gradient(vol, spf, K, poses, H, Wd, N, oracle.BEER_LAMBERT, g)
    ref_gm = camera.view_matrix_gradient(views, A, shape, gp)
    e_img = forward_rel_err(img.detach().cpu().double().numpy(), ref)
    e_vol = normwise_err(v.grad.cpu().double().numpy(), ref_gv)
    e_vm = normwise_err(vm.grad.cpu().double().numpy(), ref_gm)
    say(f"render from view matrices: image err {e_img:.3e}, volume gradient {e_vol:.3e}, "
        f"view-matrix gradient {e_vm:.3e}")
    assert np.abs(ref).max() > 0.05
    assert e_img <= 1e-5 and e_vol <= 1e-4 and e_vm <= 1e-4
