"""GPU parity of the brick-owned volume backward (Beer-Lambert and line
integral with the box clip, views sparse against the voxels) against the CPU
oracle's adjoint, through the C ABI.

Every case here is checked to take that path (fewer than four samples per
cell from one view).  Covered: the full 16-view 200^2 batch, ragged
anisotropic multi-view cases spanning several bricks with a ragged last one,
volumes one voxel thick, cameras inside the volume (candidate rectangles that
cover the whole detector), non-finite upstream gradients (their rays go
through float atomics), flashdrr render batches with a density factor and a
transfer function, graph replays and run-to-run determinism (integer sums in
LDS).  Bar: gradient max |g - o| / max |o| <= 1e-4 (normwise).
"""
import numpy as np
import pytest
import torch

import ct_forward_projection_amd as drr
import oracle
import workloads as W
from helpers import l2_err, normwise_err, say

pytestmark = pytest.mark.gpu

GRAD = 1e-4
BRICK_MAX_VIEW_REUSE = 4.0       # the library's threshold for the brick path


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def view_reuse(shape, H, Wd, N):
    nz, ny, nx = shape[-3:]
    return H * Wd * N / ((nx + 1) * (ny + 1) * (nz + 1))


def brick_backward(dev, w, g, s=None):
    assert view_reuse(w.volume.shape, w.det_h, w.det_w, w.n_samples) < BRICK_MAX_VIEW_REUSE
    poses = torch.from_numpy(w.poses).to(dev)
    if s is None and w.mode == W.BEER_LAMBERT:
        vol = torch.from_numpy(w.volume).to(dev)
        _, s = drr.drr_forward(vol, w.spacing, w.K, poses, w.det_h, w.det_w, w.n_samples, w.mode)
    grad = drr.drr_backward_volume(w.volume.shape, w.spacing, w.K, poses, w.det_h, w.det_w,
                                   w.n_samples, w.mode, torch.from_numpy(g).to(dev), s)
    torch.cuda.synchronize()
    return grad


def test_batch_workload_backward(dev):
    """The 16-view 200^2 x 256-sample batch over the 256^3 phantom, Beer-Lambert,
    upstream gradient U[-1, 1)."""
    w = W.make_workload(2)
    g = np.random.default_rng(2116).uniform(-1.0, 1.0, size=(16, 200, 200)).astype(np.float32)
    say("case: brick backward, 16-view 200^2 batch")
    grad = brick_backward(dev, w, g).cpu().double().numpy()
    ref, used = oracle.adjoint_workload(w, grad_out=g)
    err = normwise_err(grad, ref)
    say(f"batch brick: gradient normwise err {err:.3e}, l2 {l2_err(grad, ref):.3e} "
        f"(oracle on {used} threads)")
    assert err <= GRAD


@pytest.mark.parametrize("seed,mode,shape,views,det,n,spacing", [
    (601, W.BEER_LAMBERT, (29, 31, 27), 6, (23, 29), 19, (1.0, 1.25, 0.8)),
    (602, W.LINE_INTEGRAL, (40, 26, 37), 9, (17, 21), 33, (0.9, 1.0, 1.1)),
    (603, W.BEER_LAMBERT, (13, 50, 1), 4, (31, 9), 11, (1.0, 1.0, 1.0)),
    (604, W.LINE_INTEGRAL, (1, 18, 33), 5, (12, 40), 7, (1.0, 1.0, 1.0)),
    (605, W.LINE_INTEGRAL, (25, 25, 25), 3, (16, 16), 1, (1.0, 1.0, 1.0)),
    (606, W.BEER_LAMBERT, (37, 35, 33), 2, (11, 13), 301, (1.0, 1.0, 1.0)),
])
def test_random_sparse_cases(dev, seed, mode, shape, views, det, n, spacing):
    """Ragged volumes of several 12^3 bricks with a ragged last one per axis,
    anisotropic voxels, oblique views, N = 1 and N in the hundreds."""
    w = W.make_random_small(seed, shape=shape, n_views=views, det=det, n_samples=n, mode=mode,
                            spacing=spacing)
    say(f"case: brick seed={seed} mode={mode} shape={shape} views={views} det={det} N={n} "
        f"({view_reuse(shape, *det, n):.2f} samples per view-cell)")
    grad = brick_backward(dev, w, w.grad_out).cpu().double().numpy()
    ref, _ = oracle.adjoint_workload(w)
    err = normwise_err(grad, ref)
    say(f"brick {seed}: gradient normwise err {err:.3e}")
    assert np.abs(ref).max() > 0
    assert err <= GRAD
    assert np.all(grad[ref == 0.0] == 0.0)


def test_cameras_inside_the_volume(dev):
    """Sources inside the box: brick regions straddle the camera plane or lie
    behind it (whole-detector or empty candidate rectangles)."""
    w = W.make_random_small(611, shape=(30, 28, 26), n_views=3, det=(15, 17), n_samples=40,
                            distance=3.0, rot_deg=180.0)
    say("case: brick, cameras inside the volume")
    grad = brick_backward(dev, w, w.grad_out).cpu().double().numpy()
    ref, _ = oracle.adjoint_workload(w)
    err = normwise_err(grad, ref)
    say(f"brick inside: gradient normwise err {err:.3e}")
    assert err <= GRAD


@pytest.mark.parametrize("bad", [np.nan, np.inf, -np.inf])
def test_non_finite_upstream_gradient(dev, bad):
    """A non-finite upstream gradient goes through float atomics.  NaN: exactly
    the voxels the oracle makes NaN (every corner of every sample of that ray)
    are NaN on the GPU.  +-Inf: the voxels the ray reaches are not finite on
    both sides and, where both are infinite, of the same sign; which of them
    are NaN (Inf times a corner weight of exactly 0) is not unique: this ray
    steps onto exact integer positions in the oracle's fp64, where floor picks
    the upper cell (zero weight on its upper corner), while the fixed-point
    position sits 2^-32 below (zero weight on the lower neighbour) -- both are
    the tie reading of floor at an integer.  The other voxels match to the
    gradient bar."""
    w = W.make_random_small(612, shape=(26, 24, 28), n_views=3, det=(14, 16), n_samples=30,
                            mode=W.LINE_INTEGRAL)
    g = w.grad_out.copy()
    g[1, 6, 9] = bad
    say(f"case: brick, upstream gradient {bad}")
    grad = brick_backward(dev, w, g).cpu().double().numpy()
    ref, _ = oracle.adjoint_workload(w, grad_out=g)
    bad_ref = ~np.isfinite(ref)
    assert bad_ref.any()
    assert np.array_equal(~np.isfinite(grad), bad_ref)
    if np.isnan(bad):
        assert np.array_equal(np.isnan(grad), np.isnan(ref))
    both = np.isinf(grad) & np.isinf(ref)
    assert both.sum() >= 0.8 * np.isinf(ref).sum()
    assert np.array_equal(np.sign(grad[both]), np.sign(ref[both]))
    say(f"non-finite {bad}: {int(bad_ref.sum())} voxels, {int(np.isnan(ref).sum())} NaN in the "
        f"oracle, {int(np.isnan(grad).sum())} on the GPU")
    ok = np.isfinite(ref)
    assert normwise_err(grad[ok], ref[ok]) <= GRAD


def test_render_batches_factor_and_transfer(dev):
    """drr_render_backward_volume on 2 volumes x 2 channels, 3 views each, with a
    density factor and a per-channel transfer function (Beer-Lambert), and
    without one (line integral)."""
    rng = np.random.default_rng(613)
    B, C, shape = 2, 2, (27, 25, 29)
    K = W.intrinsics(40.0, 9.3, 8.8)
    poses = W.random_poses(6, 60.0, 40.0, 1.5, seed=620)
    sp = np.array([1.0, 1.1, 0.9], dtype=np.float32)
    H, Wd, N = 17, 19, 23
    assert view_reuse(shape, H, Wd, N) < BRICK_MAX_VIEW_REUSE
    xp = np.array([[-1000.0, 0.0, 1500.0], [-600.0, 100.0, 1200.0]], dtype=np.float32)
    yp = np.array([[0.0, 0.02, 0.05], [0.005, 0.0, 0.04]], dtype=np.float32)
    for mode, tf, f in [(W.BEER_LAMBERT, (xp, yp), 35.0), (W.LINE_INTEGRAL, None, 0.8)]:
        if tf is None:
            vol = rng.uniform(0.05, 1.0, size=(B, C) + shape).astype(np.float32)
        else:
            vol = rng.uniform(-1100.0, 1600.0, size=(B, C) + shape).astype(np.float32)
        g = rng.uniform(-1.0, 1.0, size=(6, C, H, Wd)).astype(np.float32)
        say(f"case: brick render backward mode={mode} transfer={tf is not None} f={f}")
        v = torch.from_numpy(vol).to(dev)
        P = torch.from_numpy(poses).to(dev)
        img, tau = drr.drr_render(v, sp, K, P, H, Wd, N, mode, f, drr.CLIP_BOX, 0.0, tf)
        grad = drr.drr_render_backward_volume(v, vol.shape, 0, sp, K, P, H, Wd, N, mode,
                                              torch.from_numpy(g).to(dev), img, tau, f,
                                              drr.CLIP_BOX, 0.0, tf)
        torch.cuda.synchronize()
        ref = oracle.render_adjoint(vol, sp, K, poses, H, Wd, N, mode, g, density_factor=f,
                                    clip=drr.CLIP_BOX, margin=0.0, transfer=tf)
        err = normwise_err(grad.cpu().double().numpy(), ref)
        say(f"brick render m{mode}: gradient normwise err {err:.3e}")
        assert err <= GRAD


def test_deterministic_and_graph_replays(dev):
    """Integer sums in LDS and one plain store per voxel: two eager runs are
    bit-identical, and so are replays of a captured graph (with eager work and
    other gradients written in between)."""
    w = W.make_random_small(614, shape=(33, 30, 31), n_views=4, det=(21, 19), n_samples=27,
                            mode=W.LINE_INTEGRAL)
    assert view_reuse(w.volume.shape, w.det_h, w.det_w, w.n_samples) < BRICK_MAX_VIEW_REUSE
    poses = torch.from_numpy(w.poses).to(dev)
    g = torch.from_numpy(w.grad_out).to(dev)
    nz, ny, nx = w.volume.shape
    need = drr.drr_workspace_bytes(nz, ny, nx, drr.F32, 4, 21, 19, 27, 1)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    grad = torch.empty(w.volume.shape, device=dev)

    def step():
        drr.drr_backward_volume(w.volume.shape, w.spacing, w.K, poses, 21, 19, 27,
                                drr.LINE_INTEGRAL, g, None, grad_volume=grad, workspace=ws)

    step()
    torch.cuda.synchronize()
    first = grad.clone()
    step()
    torch.cuda.synchronize()
    assert torch.equal(grad, first), "two eager runs differ"
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for i in range(3):
        grad.fill_(7.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(grad, first), f"replay {i}"
        step()
        torch.cuda.synchronize()
    ref, _ = oracle.adjoint_workload(w)
    assert normwise_err(first.cpu().double().numpy(), ref) <= GRAD
