"""GPU parity of the flashdrr front end (``drr_render`` / ``drr_render_backward_volume``
through the C ABI) against the oracle's ``render`` / ``render_adjoint``.

Covers volume and channel batches (N = B * views_per_vol views), the density
factor, all three outputs (Beer-Lambert, line integral, front-to-back alpha
compositing), both clip modes (per-ray box; per-view near/far with zero padding)
and the per-channel transfer function, on every read plan the library picks
(the caller's volume, its mapped fp32 copy, z-pair copies plain or mapped,
corner cells, zero-padded or mapped cells, LDS-staged boxes).  Bars as elsewhere: forward max |g - o| / max(|o|, 1e-3 max|o|) <= 1e-5
for fp32 (1e-2 for bf16 against the fp32 volume, 1e-5 against the bf16-rounded
one), gradients normwise <= 1e-4.
"""
import numpy as np
import pytest
import torch

import ct_forward_projection_amd as drr
import oracle
import workloads as W
from helpers import forward_rel_err, l2_err, normwise_err, say

pytestmark = pytest.mark.gpu

BL, RAW, ALPHA = drr.BEER_LAMBERT, drr.LINE_INTEGRAL, drr.ALPHA_COMPOSITE
BOX, NEAR_FAR = drr.CLIP_BOX, drr.CLIP_NEAR_FAR
FWD_F32, FWD_BF16, GRAD = 1e-5, 1e-2, 1e-4


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def knots(C):
    """Per-channel transfer functions over HU-like values (fp32, as the ABI takes them)."""
    xp = np.array([[-1000.0, 0.0, 1500.0], [-600.0, 100.0, 1200.0], [-900.0, -100.0, 800.0]],
                  dtype=np.float32)[:C]
    yp = np.array([[0.0, 0.02, 0.05], [0.005, 0.0, 0.04], [0.0, 0.03, 0.01]],
                  dtype=np.float32)[:C]
    return xp, yp


def problem(seed, B=2, C=2, vpv=2, shape=(13, 10, 17), det=(19, 23), N=37, tf=False):
    rng = np.random.default_rng(seed)
    if tf:
        vol = rng.uniform(-1100.0, 1600.0, size=(B, C) + shape).astype(np.float32)
    else:
        vol = rng.uniform(0.05, 1.0, size=(B, C) + shape).astype(np.float32)
    spacing = np.array([1.0, 1.25, 0.8], dtype=np.float32)
    H, Wd = det
    ext = max(shape[2] * 1.0, shape[1] * 1.25, shape[0] * 0.8)
    K = W.intrinsics(1.2 * max(H, Wd) * 60.0 / ext, Wd / 2.0 + 0.3, H / 2.0 - 0.2)
    poses = W.random_poses(B * vpv, 60.0, 40.0, 0.05 * ext, seed=seed + 7)
    g = rng.uniform(-1.0, 1.0, size=(B * vpv, C, H, Wd)).astype(np.float32)
    return vol, spacing, K, poses, H, Wd, N, g


def run_gpu(dev, vol, spacing, K, poses, H, Wd, N, mode, f, clip, margin, transfer, g,
            bf16_bits=None):
    if bf16_bits is not None:
        v = torch.from_numpy(bf16_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        v = torch.from_numpy(vol).to(dev)
    P = torch.from_numpy(poses).to(dev)
    img, tau = drr.drr_render(v, spacing, K, P, H, Wd, N, mode, f, clip, margin, transfer)
    grad = drr.drr_render_backward_volume(v, tuple(vol.shape), 0, spacing, K, P, H, Wd, N, mode,
                                          torch.from_numpy(g).to(dev), img, tau, f, clip, margin,
                                          transfer)
    torch.cuda.synchronize()
    return (img.cpu().double().numpy(), tau.cpu().double().numpy(),
            grad.cpu().double().numpy())


def plan_name(vol, H, Wd, N, V, mode, clip, nk, bf16=False):
    B, C, nz, ny, nx = vol.shape
    ws = drr.drr_render_workspace_bytes(B, C, nz, ny, nx, 1 if bf16 else 0, V, H, Wd, N, mode,
                                        clip, nk, 0)
    elem = 4 if (nk or not bf16) else 2
    cells = B * C * (((nx + 1) * (ny + 1) * (nz + 1) * 8 * elem + 255) // 256 * 256)
    lin = B * C * ((nx * ny * nz * 4 + 255) // 256 * 256)
    zpair = B * C * ((nx * ny * (nz - 1) * 2 * elem + 255) // 256 * 256)
    zpad = B * C * (((nx + 2) * (ny + 2) * (nz + 1) * 2 * elem + 255) // 256 * 256)
    if ws == cells:
        return "mapped cells" if nk else "cells"
    if clip == NEAR_FAR and ws == zpad:
        return "mapped padded z-pairs" if nk else "padded z-pairs"
    if ws == zpair and nz >= 2:
        return "mapped z-pairs" if nk else "z-pairs"
    if nk:
        assert ws == lin
        return "mapped linear"
    assert ws == 0
    return "caller's volume"


def check(img, tau, grad, ref, ref_tau, ref_grad, what, bar=FWD_F32):
    e_img = forward_rel_err(img, ref)
    e_tau = forward_rel_err(tau, ref_tau)
    e_g = normwise_err(grad, ref_grad)
    say(f"{what}: image err {e_img:.3e}, optical depth err {e_tau:.3e}, gradient normwise "
        f"{e_g:.3e} (l2 {l2_err(grad, ref_grad):.3e})")
    assert np.abs(ref).max() > 0 and np.abs(ref_grad).max() > 0
    assert e_img <= bar and e_tau <= bar
    assert np.all(img[ref == 0.0] == 0.0)          # nothing rendered where the oracle has 0
    assert e_g <= GRAD


@pytest.mark.parametrize("N", [37, 101])
@pytest.mark.parametrize("tf", [False, True])
@pytest.mark.parametrize("clip", [BOX, NEAR_FAR])
@pytest.mark.parametrize("mode", [BL, RAW, ALPHA])
def test_render_random_batches(dev, mode, clip, tf, N):
    """2 volumes x 2 channels, 2 views each, ragged 13 x 10 x 17 volume and
    19 x 23 detector, anisotropic voxels; N = 37 reads the z-pair copy (mapped
    with a transfer function), N = 101 reuses cells enough for the corner-cell
    copy (the near/far mode always reads zero-padded cells)."""
    seed = 300 + 10 * mode + 4 * clip + 2 * tf + (N > 50)
    vol, spacing, K, poses, H, Wd, N, g = problem(seed, N=N, tf=tf)
    C = vol.shape[1]
    transfer = knots(C) if tf else None
    f, margin = (0.9 if tf else 1.7), 3.0
    if tf:
        f *= 40.0    # the mapped mu is ~0.02/mm on a small volume: make the image non-trivial
    name = plan_name(vol, H, Wd, N, poses.shape[0], mode, clip, 3 if tf else 0)
    say(f"case: render mode={mode} clip={clip} tf={tf} N={N} plan={name} seed={seed}")
    img, tau, grad = run_gpu(dev, vol, spacing, K, poses, H, Wd, N, mode, f, clip, margin,
                             transfer, g)
    kw = dict(density_factor=f, clip=clip, margin=margin, transfer=transfer)
    ref, ref_tau = oracle.render(vol, spacing, K, poses, H, Wd, N, mode, **kw)
    ref_g = oracle.render_adjoint(vol, spacing, K, poses, H, Wd, N, mode, g, **kw)
    check(img, tau, grad, ref, ref_tau, ref_g, f"render m{mode} c{clip} tf{int(tf)} N{N}")


def test_render_bf16_hu_volume_with_transfer_function(dev):
    """bf16 HU volumes mapped by the transfer function: fp32 mapped cells, so the
    result matches the oracle on the bf16-rounded volume to the fp32 bar."""
    vol, spacing, K, poses, H, Wd, N, g = problem(351, N=64, tf=True)
    bits = W.round_to_bf16_bits(vol)
    vol_r = (bits.astype(np.uint32) << 16).view(np.float32)
    transfer = knots(2)
    for mode, clip in [(ALPHA, NEAR_FAR), (BL, BOX)]:
        say(f"case: bf16 HU + transfer mode={mode} clip={clip}")
        img, tau, grad = run_gpu(dev, vol, spacing, K, poses, H, Wd, N, mode, 30.0, clip, 2.0,
                                 transfer, g, bf16_bits=bits)
        kw = dict(density_factor=30.0, clip=clip, margin=2.0, transfer=transfer)
        ref, ref_tau = oracle.render(vol_r, spacing, K, poses, H, Wd, N, mode, **kw)
        ref_g = oracle.render_adjoint(vol_r, spacing, K, poses, H, Wd, N, mode, g, **kw)
        check(img, tau, grad, ref, ref_tau, ref_g, f"bf16 m{mode} c{clip}")
        ref32, _ = oracle.render(vol, spacing, K, poses, H, Wd, N, mode, **kw)
        assert forward_rel_err(img, ref32) <= FWD_BF16


@pytest.mark.parametrize("mode", [BL, RAW, ALPHA])
def test_render_bf16_transfer_mapped_linear(dev, mode):
    """bf16 HU volumes with a transfer function and under one sample per cell:
    the march reads the fp32 mapped linear copy (row and slice strides of fp32,
    not of the bf16 input); forward, volume gradient and pose gradient."""
    vol, spacing, K, poses, H, Wd, N, g = problem(355 + mode, det=(5, 7), N=23, tf=True)
    bits = W.round_to_bf16_bits(vol)
    vol_r = (bits.astype(np.uint32) << 16).view(np.float32)
    transfer = knots(2)
    name = plan_name(vol, H, Wd, N, poses.shape[0], mode, BOX, 3, bf16=True)
    say(f"case: bf16 HU + transfer, linear mapped copy, mode={mode} plan={name}")
    assert name == "mapped linear"
    img, tau, grad = run_gpu(dev, vol, spacing, K, poses, H, Wd, N, mode, 30.0, BOX, 0.0,
                             transfer, g, bf16_bits=bits)
    kw = dict(density_factor=30.0, clip=BOX, margin=0.0, transfer=transfer)
    ref, ref_tau = oracle.render(vol_r, spacing, K, poses, H, Wd, N, mode, **kw)
    ref_g = oracle.render_adjoint(vol_r, spacing, K, poses, H, Wd, N, mode, g, **kw)
    check(img, tau, grad, ref, ref_tau, ref_g, f"bf16 mapped linear m{mode}")
    v = torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)
    gp = drr.drr_render_backward_pose(v, spacing, K, torch.from_numpy(poses).to(dev), H, Wd, N,
                                      mode, torch.from_numpy(g).to(dev), 30.0, BOX, 0.0, transfer)
    torch.cuda.synchronize()
    ref_p = oracle.render_pose_gradient(vol_r, spacing, K, poses, H, Wd, N, mode, g,
                                        density_factor=30.0, transfer=transfer)
    got = gp.cpu().double().numpy()
    errs = [np.abs(got[i] - ref_p[i]).max() / np.abs(ref_p[i]).max() for i in range(len(ref_p))]
    say(f"bf16 mapped linear m{mode}: pose gradient per-view normwise err max {max(errs):.3e}")
    assert max(errs) <= GRAD


@pytest.mark.parametrize("tf", [False, True])
@pytest.mark.parametrize("mode", [BL, RAW, ALPHA])
def test_render_sparse_rays_read_the_volume(dev, mode, tf):
    """Under one sample per cell (5 x 7 detectors, N = 23) no copy pays: the
    march reads the caller's volume, or its mapped fp32 copy, as x-pairs;
    forward, volume gradient and pose gradient."""
    seed = 360 + 2 * mode + tf
    vol, spacing, K, poses, H, Wd, N, g = problem(seed, det=(5, 7), N=23, tf=tf)
    transfer = knots(2) if tf else None
    f = 30.0 if tf else 1.1
    name = plan_name(vol, H, Wd, N, poses.shape[0], mode, BOX, 3 if tf else 0)
    say(f"case: sparse rays mode={mode} tf={tf} plan={name} seed={seed}")
    assert name == ("mapped linear" if tf else "caller's volume")
    img, tau, grad = run_gpu(dev, vol, spacing, K, poses, H, Wd, N, mode, f, BOX, 0.0, transfer, g)
    kw = dict(density_factor=f, clip=BOX, margin=0.0, transfer=transfer)
    ref, ref_tau = oracle.render(vol, spacing, K, poses, H, Wd, N, mode, **kw)
    ref_g = oracle.render_adjoint(vol, spacing, K, poses, H, Wd, N, mode, g, **kw)
    check(img, tau, grad, ref, ref_tau, ref_g, f"sparse m{mode} tf{int(tf)}")
    gp = drr.drr_render_backward_pose(torch.from_numpy(vol).to(dev), spacing, K,
                                      torch.from_numpy(poses).to(dev), H, Wd, N, mode,
                                      torch.from_numpy(g).to(dev), f, BOX, 0.0, transfer)
    torch.cuda.synchronize()
    ref_p = oracle.render_pose_gradient(vol, spacing, K, poses, H, Wd, N, mode, g,
                                        density_factor=f, transfer=transfer)
    got = gp.cpu().double().numpy()
    errs = [np.abs(got[i] - ref_p[i]).max() / np.abs(ref_p[i]).max() for i in range(len(ref_p))]
    say(f"sparse m{mode} tf{int(tf)}: pose gradient per-view normwise err max {max(errs):.3e}")
    assert max(errs) <= GRAD


@pytest.mark.parametrize("shape,det,N,plan", [
    ((2, 9, 11), (19, 23), 5, "z-pairs"),          # one z-pair slice
    ((7, 9, 2), (19, 23), 3, "z-pairs"),           # one x-pair per row
    ((2, 2, 2), (8, 8), 2, "z-pairs"),             # both at once
    ((1, 9, 11), (19, 23), 3, "caller's volume"),  # no z-pairs in a one-voxel-deep volume
])
@pytest.mark.parametrize("tf", [False, True])
def test_render_thin_volumes(dev, shape, det, N, plan, tf):
    """Volumes two (or one) voxels thick at the reuse that picks z-pairs: every
    x and z weight is pinned or edge-clamped somewhere; forward, volume and pose
    gradients against the oracle, all three modes, with and without the
    transfer function."""
    seed = 370 + shape[0] + 3 * shape[2] + tf
    vol, spacing, K, poses, H, Wd, N, g = problem(seed, shape=shape, det=det, N=N, tf=tf)
    transfer = knots(2) if tf else None
    name = plan_name(vol, H, Wd, N, poses.shape[0], BL, BOX, 3 if tf else 0)
    say(f"case: thin volume {shape} det={det} N={N} tf={tf} plan={name}")
    expected = plan
    if tf:
        expected = "mapped linear" if plan == "caller's volume" else "mapped " + plan
    assert name == expected
    f = 30.0 if tf else 1.3
    for mode in (BL, RAW, ALPHA):
        img, tau, grad = run_gpu(dev, vol, spacing, K, poses, H, Wd, N, mode, f, BOX, 0.0,
                                 transfer, g)
        kw = dict(density_factor=f, clip=BOX, margin=0.0, transfer=transfer)
        ref, ref_tau = oracle.render(vol, spacing, K, poses, H, Wd, N, mode, **kw)
        ref_g = oracle.render_adjoint(vol, spacing, K, poses, H, Wd, N, mode, g, **kw)
        check(img, tau, grad, ref, ref_tau, ref_g, f"thin {shape} m{mode} tf{int(tf)}")
        gp = drr.drr_render_backward_pose(torch.from_numpy(vol).to(dev), spacing, K,
                                          torch.from_numpy(poses).to(dev), H, Wd, N, mode,
                                          torch.from_numpy(g).to(dev), f, BOX, 0.0, transfer)
        torch.cuda.synchronize()
        ref_p = oracle.render_pose_gradient(vol, spacing, K, poses, H, Wd, N, mode, g,
                                            density_factor=f, transfer=transfer)
        got = gp.cpu().double().numpy()
        errs = [np.abs(got[i] - ref_p[i]).max() / max(np.abs(ref_p[i]).max(), 1e-30)
                for i in range(len(ref_p))]
        say(f"thin {shape} m{mode} tf{int(tf)}: pose gradient per-view normwise err max "
            f"{max(errs):.3e}")
        assert max(errs) <= GRAD


@pytest.mark.parametrize("tf", [False, True])
def test_render_sparse_near_far_compositing(dev, tf):
    """Near/far compositing under one sample per cell: the forward reads padded
    z-pairs, while the backward's coefficient passes gather the zero-padded
    corners from the volume itself (or its mapped fp32 copy) -- no copy pays."""
    vol, spacing, K, poses, H, Wd, N, g = problem(380 + tf, det=(5, 7), N=23, tf=tf)
    B, C, nz, ny, nx = vol.shape
    transfer = knots(2) if tf else None
    ws_b = drr.drr_render_workspace_bytes(B, C, nz, ny, nx, 0, poses.shape[0], H, Wd, N, ALPHA,
                                          NEAR_FAR, 3 if tf else 0, 1)
    # with a transfer function the mapped fp32 volumes and their value bounds
    assert ws_b == (B * C * ((nx * ny * nz * 4 + 255) // 256 * 256) + 256 if tf else 0)
    say(f"case: sparse near/far compositing tf={tf}")
    f = 30.0 if tf else 1.1
    img, tau, grad = run_gpu(dev, vol, spacing, K, poses, H, Wd, N, ALPHA, f, NEAR_FAR, 3.0,
                             transfer, g)
    kw = dict(density_factor=f, clip=NEAR_FAR, margin=3.0, transfer=transfer)
    ref, ref_tau = oracle.render(vol, spacing, K, poses, H, Wd, N, ALPHA, **kw)
    ref_g = oracle.render_adjoint(vol, spacing, K, poses, H, Wd, N, ALPHA, g, **kw)
    check(img, tau, grad, ref, ref_tau, ref_g, f"sparse near/far alpha tf{int(tf)}")


@pytest.mark.parametrize("clip", [BOX, NEAR_FAR])
@pytest.mark.parametrize("shift,f", [(0.0, 1.1), (-0.3, 1.1), (0.0, -0.4)])
def test_render_compositing_backward_bound_paths(dev, clip, shift, f):
    """The compositing backward bounds its coefficients in closed form from the
    largest value of its z-pair copy when every value is finite and >= 0 and the
    density factor is >= 0; negative values (shift -0.3: values in [-0.25, 0.7))
    or a negative density factor take the pass over the samples instead.  Each
    against the oracle."""
    vol, spacing, K, poses, H, Wd, N, g = problem(400 + clip, N=37)
    vol = (vol + np.float32(shift)).astype(np.float32)
    B, C, nz, ny, nx = vol.shape
    ws_b = drr.drr_render_workspace_bytes(B, C, nz, ny, nx, 0, poses.shape[0], H, Wd, N, ALPHA,
                                          clip, 0, 1)
    assert ws_b > 0                                 # a z-pair copy and its bounds
    say(f"case: compositing backward bound clip={clip} shift={shift} f={f}")
    img, tau, grad = run_gpu(dev, vol, spacing, K, poses, H, Wd, N, ALPHA, f, clip, 3.0, None, g)
    kw = dict(density_factor=f, clip=clip, margin=3.0, transfer=None)
    ref, ref_tau = oracle.render(vol, spacing, K, poses, H, Wd, N, ALPHA, **kw)
    ref_g = oracle.render_adjoint(vol, spacing, K, poses, H, Wd, N, ALPHA, g, **kw)
    check(img, tau, grad, ref, ref_tau, ref_g, f"compositing bound clip{clip} {shift} {f}")


def test_render_compositing_backward_nan_voxel(dev):
    """A NaN voxel sets the non-finite flag of the compositing backward's value
    bounds, so the pass over the samples runs, finds the NaN coefficients of the
    rays through it (their forward image is NaN as well) and their tiles fall
    back to float atomics: exactly the voxels the oracle marks NaN are NaN on the
    GPU, and the rest match."""
    vol, spacing, K, poses, H, Wd, N, g = problem(430, N=37)
    vol[0, 1, 6, 5, 8] = np.nan
    say("case: compositing backward with a NaN voxel")
    img, tau, grad = run_gpu(dev, vol, spacing, K, poses, H, Wd, N, ALPHA, 1.1, BOX, 3.0, None, g)
    kw = dict(density_factor=1.1, clip=BOX, margin=3.0, transfer=None)
    ref_g = oracle.render_adjoint(vol, spacing, K, poses, H, Wd, N, ALPHA, g, **kw)
    assert np.isnan(ref_g).any() and not np.isnan(ref_g).all()
    assert np.array_equal(np.isnan(grad), np.isnan(ref_g))
    ok = ~np.isnan(ref_g)
    err = normwise_err(grad[ok], ref_g[ok])
    say(f"NaN voxel: {int(np.isnan(ref_g).sum())} NaN voxels, the rest normwise {err:.3e}")
    assert err <= GRAD


@pytest.mark.parametrize("N", [6, 64])
@pytest.mark.parametrize("mode", [BL, RAW, ALPHA])
def test_render_near_far_axis_aligned_and_boundary_rays(dev, mode, N):
    """Near/far rays the support test must get exactly right: with cx = cy = 7.5
    the ray through pixel (7, 7) runs along z (no step in x or y), and cameras
    shifted by 5 mm put that ray on q_x = -1 (support boundary, included, adds
    0) and q_x = n (outside, skipped).  N = 6 reads padded z-pairs, N = 64
    corner cells; forward and volume gradient against the oracle."""
    rng = np.random.default_rng(390 + mode + N)
    vol = rng.uniform(0.05, 1.0, size=(1, 1, 9, 9, 9)).astype(np.float32)
    spacing = np.ones(3, dtype=np.float32)
    K = W.intrinsics(30.0, 7.5, 7.5)
    poses = np.stack([W.pose_from_rotation_and_centre(np.eye(3), np.array([x, 0.0, -40.0]))
                      for x in (0.0, -5.0, 5.0, 2.5)]).astype(np.float32)
    H = Wd = 16
    g = rng.uniform(-1, 1, size=(4, 1, H, Wd)).astype(np.float32)
    name = plan_name(vol, H, Wd, N, 4, mode, NEAR_FAR, 0)
    say(f"case: near/far axis-aligned rays mode={mode} N={N} plan={name}")
    assert name == ("padded z-pairs" if N == 6 else "cells")
    img, tau, grad = run_gpu(dev, vol, spacing, K, poses, H, Wd, N, mode, 1.2, NEAR_FAR, 2.0,
                             None, g)
    kw = dict(density_factor=1.2, clip=NEAR_FAR, margin=2.0)
    ref, ref_tau = oracle.render(vol, spacing, K, poses, H, Wd, N, mode, **kw)
    ref_g = oracle.render_adjoint(vol, spacing, K, poses, H, Wd, N, mode, g, **kw)
    check(img, tau, grad, ref, ref_tau, ref_g, f"near/far axis m{mode} N{N}")


def test_render_graph_capture_replays_match_eager(dev):
    """drr_render and its backwards captured in a HIP graph replay to the eager
    results, four times, with eager work and synchronisations in between: near/far
    compositing with a transfer function (zero-padded z-pair copies in the
    forward's and the backward's workspaces, made by kernels) and a render that
    stages boxes, with its staged pose gradient."""
    vol, spacing, K, poses, H, Wd, N, g = problem(395, N=37, tf=True)
    v = torch.from_numpy(vol).to(dev)
    P = torch.from_numpy(poses).to(dev)
    gt = torch.from_numpy(g).to(dev)
    tf = knots(2)
    vol2, spacing2, K2, poses2, H2, Wd2, N2, g2 = problem(396, shape=(16, 16, 16), det=(96, 96),
                                                        N=37)
    assert _pose_is_staged(vol2, H2, Wd2, N2, poses2.shape[0], 0)
    v2 = torch.from_numpy(vol2).to(dev)
    P2 = torch.from_numpy(poses2).to(dev)
    g2t = torch.from_numpy(g2).to(dev)
    bufs = {}

    def step():
        img, tau = drr.drr_render(v, spacing, K, P, H, Wd, N, ALPHA, 30.0, NEAR_FAR, 2.0, tf)
        grad = drr.drr_render_backward_volume(v, tuple(vol.shape), 0, spacing, K, P, H, Wd, N,
                                              ALPHA, gt, img, tau, 30.0, NEAR_FAR, 2.0, tf)
        img2, _ = drr.drr_render(v2, spacing2, K2, P2, H2, Wd2, N2, BL, 0.8, BOX, 0.0, None)
        gp = drr.drr_render_backward_pose(v2, spacing2, K2, P2, H2, Wd2, N2, BL, g2t, 0.8, BOX,
                                          0.0, None)
        bufs.update(img=img, grad=grad, img2=img2, gp=gp)

    step()
    torch.cuda.synchronize()
    ref = {k: t.clone() for k, t in bufs.items()}
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    outs = dict(bufs)
    for i in range(4):
        for t in outs.values():
            t.fill_(-7.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(outs["img"], ref["img"]), f"replay {i}: image"
        assert torch.equal(outs["img2"], ref["img2"]), f"replay {i}: staged image"
        for k in ("grad", "gp"):
            e = normwise_err(outs[k].cpu().double().numpy(), ref[k].cpu().double().numpy())
            assert e <= 1e-6, f"replay {i}: {k} {e}"
        step()   # eager work between replays
        torch.cuda.synchronize()
    say("render graph capture: 4 replays match the eager results")


def test_render_bf16_density_without_transfer(dev):
    """bf16 densities read directly (cells keep bf16), near/far and box."""
    vol, spacing, K, poses, H, Wd, N, g = problem(352, N=101)
    bits = W.round_to_bf16_bits(vol)
    vol_r = (bits.astype(np.uint32) << 16).view(np.float32)
    for mode, clip in [(RAW, NEAR_FAR), (ALPHA, BOX)]:
        say(f"case: bf16 density mode={mode} clip={clip}")
        img, tau, grad = run_gpu(dev, vol, spacing, K, poses, H, Wd, N, mode, 1.3, clip, 4.0,
                                 None, g, bf16_bits=bits)
        kw = dict(density_factor=1.3, clip=clip, margin=4.0)
        ref, ref_tau = oracle.render(vol_r, spacing, K, poses, H, Wd, N, mode, **kw)
        ref_g = oracle.render_adjoint(vol_r, spacing, K, poses, H, Wd, N, mode, g, **kw)
        check(img, tau, grad, ref, ref_tau, ref_g, f"bf16 density m{mode} c{clip}")


def test_single_volume_render_is_drr_forward(dev):
    """One volume, one channel, f = 1, box clip, no transfer function: the same
    launches as drr_forward, bit for bit; the gradient agrees to rounding."""
    w = W.make_workload(1)
    vol = torch.from_numpy(w.volume).to(dev)
    P = torch.from_numpy(w.poses).to(dev)
    a, s = drr.drr_forward(vol, w.spacing, w.K, P, w.det_h, w.det_w, w.n_samples, BL)
    b, tau = drr.drr_render(vol, w.spacing, w.K, P, w.det_h, w.det_w, w.n_samples, BL)
    torch.cuda.synchronize()
    assert torch.equal(a, b[:, 0]) and torch.equal(s, tau[:, 0])
    g = torch.from_numpy(np.random.default_rng(5).uniform(-1, 1, size=a.shape).astype(
        np.float32)).to(dev)
    ga = drr.drr_backward_volume(w.volume.shape, w.spacing, w.K, P, w.det_h, w.det_w,
                                 w.n_samples, BL, g, s)
    gb = drr.drr_render_backward_volume(None, w.volume.shape, 0, w.spacing, w.K, P, w.det_h,
                                        w.det_w, w.n_samples, BL, g.contiguous(), b, tau)
    torch.cuda.synchronize()
    assert normwise_err(gb.cpu().double().numpy(), ga.cpu().double().numpy()) <= 1e-6


def test_batch_workload_hu_phantom_alpha_near_far(dev):
    """The 16-view 200 x 200 batch at full size, rendered flashdrr-style from the
    HU phantom: transfer function fused into the relayout, near/far clipping
    with a 30 mm margin, alpha compositing; forward on every ray, gradient on
    every voxel."""
    w = W.make_workload(2)
    hu = W.hu_phantom().astype(np.float32)
    xp = np.array([[-1000.0, 0.0, 1500.0]], dtype=np.float32)
    yp = np.array([[0.0, 0.02, 0.05]], dtype=np.float32)
    transfer = (xp, yp)
    g = np.random.default_rng(2002).uniform(-1, 1, size=(16, 1, 200, 200)).astype(np.float32)
    say("case: batch workload, HU phantom, transfer + near/far + alpha")
    img, tau, grad = run_gpu(dev, hu[None, None], w.spacing, w.K, w.poses, 200, 200,
                             w.n_samples, ALPHA, 1.0, NEAR_FAR, 30.0, transfer, g)
    kw = dict(density_factor=1.0, clip=NEAR_FAR, margin=30.0, transfer=transfer)
    ref, ref_tau = oracle.render(hu[None, None], w.spacing, w.K, w.poses, 200, 200, w.n_samples,
                                 ALPHA, **kw)
    ref_g = oracle.render_adjoint(hu[None, None], w.spacing, w.K, w.poses, 200, 200,
                                  w.n_samples, ALPHA, g, **kw)
    check(img, tau, grad, ref, ref_tau, ref_g, "batch HU alpha near/far")


def test_raycast_autograd_and_pose_broadcast(dev):
    """raycast() as an autograd function: one pose broadcast to every volume,
    and the volume gradient equals the ABI's."""
    vol, spacing, K, poses, H, Wd, N, g = problem(353, B=3, C=1, vpv=1, N=29)
    v = torch.from_numpy(vol).to(dev).requires_grad_(True)
    P = torch.from_numpy(poses[:1]).to(dev)
    img = drr.raycast(v, spacing, K, P, H, Wd, N, ALPHA, 2.0)
    gt = torch.from_numpy(g).to(dev)
    (img * gt).sum().backward()
    torch.cuda.synchronize()
    ref, _ = oracle.render(vol, spacing, K, np.repeat(poses[:1], 3, axis=0), H, Wd, N, ALPHA,
                           density_factor=2.0)
    ref_g = oracle.render_adjoint(vol, spacing, K, np.repeat(poses[:1], 3, axis=0), H, Wd, N,
                                  ALPHA, g, density_factor=2.0)
    e_img = forward_rel_err(img.detach().cpu().double().numpy(), ref)
    e_g = normwise_err(v.grad.cpu().double().numpy(), ref_g)
    say(f"raycast autograd: image err {e_img:.3e}, gradient {e_g:.3e}")
    assert e_img <= FWD_F32 and e_g <= GRAD


def test_render_edge_cases(dev):
    """Density factor 0 renders 0; a far range before near renders 0 and no
    gradient; the empty call is a no-op; one volume of one voxel."""
    vol, spacing, K, poses, H, Wd, N, g = problem(354, N=16)
    say("case: render edge cases")
    img, tau, grad = run_gpu(dev, vol, spacing, K, poses, H, Wd, N, ALPHA, 0.0, BOX, 0.0, None,
                             g)
    assert not img.any() and not tau.any()
    img, tau, grad = run_gpu(dev, vol, spacing, K, poses, H, Wd, N, BL, 1.0, NEAR_FAR, -1e4,
                             None, g)
    assert not img.any() and not grad.any()
    v = torch.from_numpy(vol).to(dev)
    out, _ = drr.drr_render(v, spacing, K, torch.zeros((0, 3, 4), device=dev), H, Wd, N)
    assert out.shape == (0, 2, H, Wd)
    one = np.full((1, 1, 1, 1, 1), 0.7, dtype=np.float32)
    img, tau, grad = run_gpu(dev, one, spacing, K, poses[:1], H, Wd, 8, RAW, 1.0, NEAR_FAR, 5.0,
                             None, g[:1, :1])
    ref, ref_tau = oracle.render(one, spacing, K, poses[:1], H, Wd, 8, RAW, clip=NEAR_FAR,
                                 margin=5.0)
    ref_g = oracle.render_adjoint(one, spacing, K, poses[:1], H, Wd, 8, RAW, g[:1, :1],
                                  clip=NEAR_FAR, margin=5.0)
    check(img, tau, grad, ref, ref_tau, ref_g, "one voxel near/far")


def check_pose_views(got, ref, what):
    errs = [np.abs(got[v] - ref[v]).max() / np.abs(ref[v]).max() for v in range(len(ref))]
    say(f"{what}: per-view normwise err max {max(errs):.3e}")
    assert all(np.abs(ref[v]).max() > 0 for v in range(len(ref)))
    assert max(errs) <= GRAD


@pytest.mark.parametrize("N", [37, 101])
@pytest.mark.parametrize("tf", [False, True])
@pytest.mark.parametrize("clip", [BOX, NEAR_FAR])
@pytest.mark.parametrize("mode", [BL, RAW, ALPHA])
def test_render_pose_gradient(dev, mode, clip, tf, N):
    """Pose gradients of batched renders (2 volumes x 2 channels, 2 views each,
    density factor, transfer function) in every mode and both clips against
    the oracle, per view normwise over the twelve entries; with the box clip
    N = 37 reads (mapped) z-pairs and N = 101 (mapped) corner cells, in the
    near/far mode zero-padded z-pairs and cells."""
    seed = 400 + 8 * mode + 4 * clip + 2 * tf + (N > 50)
    vol, spacing, K, poses, H, Wd, N, g = problem(seed, N=N, tf=tf)
    transfer = knots(2) if tf else None
    f = 30.0 if tf else 0.7
    margin = 2.0
    name = plan_name(vol, H, Wd, N, poses.shape[0], mode, clip, 3 if tf else 0)
    say(f"case: render pose gradient mode={mode} clip={clip} tf={tf} N={N} ({name})")
    P = torch.from_numpy(poses).to(dev)
    gp = drr.drr_render_backward_pose(torch.from_numpy(vol).to(dev), spacing, K, P, H, Wd, N,
                                      mode, torch.from_numpy(g).to(dev), f, clip, margin,
                                      transfer)
    torch.cuda.synchronize()
    ref = oracle.render_pose_gradient(vol, spacing, K, poses, H, Wd, N, mode, g,
                                      density_factor=f, transfer=transfer, clip=clip,
                                      margin=margin)
    check_pose_views(gp.cpu().double().numpy(), ref,
                     f"render pose gradient m{mode} c{clip} tf{int(tf)} N{N}")


def test_raycast_pose_gradient_every_mode(dev):
    """Autograd reaches the poses through raycast in every mode and both clips
    (one pose broadcast to two volumes sums both volumes' gradients)."""
    vol, spacing, K, poses, H, Wd, N, g = problem(410, B=2, C=1, vpv=1, N=33)
    v = torch.from_numpy(vol).to(dev)
    gt = torch.from_numpy(g).to(dev)
    for mode, clip in [(BL, BOX), (ALPHA, BOX), (RAW, NEAR_FAR), (ALPHA, NEAR_FAR)]:
        say(f"case: raycast pose gradient mode={mode} clip={clip}")
        P = torch.from_numpy(poses[:1]).to(dev).requires_grad_(True)
        img = drr.raycast(v, spacing, K, P, H, Wd, N, mode, 1.5, clip, 3.0)
        (img * gt).sum().backward()
        torch.cuda.synchronize()
        ref = oracle.render_pose_gradient(vol, spacing, K, np.repeat(poses[:1], 2, axis=0), H,
                                          Wd, N, mode, g, density_factor=1.5, clip=clip,
                                          margin=3.0).sum(axis=0)
        err = np.abs(P.grad.cpu().double().numpy()[0] - ref).max() / np.abs(ref).max()
        say(f"raycast pose gradient m{mode} c{clip} (broadcast pose): normwise err {err:.3e}")
        assert err <= GRAD


def test_batch_workload_hu_phantom_alpha_near_far_pose_gradient(dev):
    """The 16-view 200 x 200 batch at full size from the HU phantom (transfer
    function, near/far with a 30 mm margin, alpha compositing): pose gradient
    of every view against the oracle."""
    w = W.make_workload(2)
    hu = W.hu_phantom().astype(np.float32)
    transfer = (np.array([[-1000.0, 0.0, 1500.0]], dtype=np.float32),
                np.array([[0.0, 0.02, 0.05]], dtype=np.float32))
    g = np.random.default_rng(2003).uniform(-1, 1, size=(16, 1, 200, 200)).astype(np.float32)
    say("case: batch workload, HU phantom, transfer + near/far + alpha, pose gradient")
    gp = drr.drr_render_backward_pose(torch.from_numpy(hu[None, None]).to(dev), w.spacing, w.K,
                                      torch.from_numpy(w.poses).to(dev), 200, 200, w.n_samples,
                                      ALPHA, torch.from_numpy(g).to(dev), 1.0, NEAR_FAR, 30.0,
                                      transfer)
    torch.cuda.synchronize()
    ref = oracle.render_pose_gradient(hu[None, None], w.spacing, w.K, w.poses, 200, 200,
                                      w.n_samples, ALPHA, g, transfer=transfer, clip=NEAR_FAR,
                                      margin=30.0)
    check_pose_views(gp.cpu().double().numpy(), ref, "batch HU alpha near/far pose")


def test_train_camera_row_band_alpha_pose_gradient(dev):
    """The 1024^2 x 512 train-step camera composited, restricted to a 96-row
    band through the volume's centre (same rays; cy moved so the band is the
    whole detector; under 8 samples per cell, so the march reads the volume's
    x-pairs): pose gradient against the oracle."""
    w = W.make_workload(3)
    K = w.K.copy()
    K[1, 2] -= 464.0                  # rows 464..559 of the full detector
    g = np.ascontiguousarray(w.grad_out[:, None, 464:560, :])
    vol = w.volume[None, None]
    say("case: compositing pose gradient, 1024-wide band of the train-step camera")
    gp = drr.drr_render_backward_pose(torch.from_numpy(vol).to(dev), w.spacing, K,
                                      torch.from_numpy(w.poses).to(dev), 96, 1024, 512, ALPHA,
                                      torch.from_numpy(g).to(dev), 1.0, BOX, 0.0, None)
    torch.cuda.synchronize()
    ref = oracle.render_pose_gradient(vol, w.spacing, K, w.poses, 96, 1024, 512, ALPHA, g)
    check_pose_views(gp.cpu().double().numpy(), ref, "train band alpha pose")


def _is_staged(vol, H, Wd, N, V, mode, nk, bf16=False):
    """The forward plan stages boxes in LDS exactly when it needs no workspace
    although rays reuse cells (at least 65,536 rays, box clip)."""
    B, C, nz, ny, nx = vol.shape
    return drr.drr_render_workspace_bytes(B, C, nz, ny, nx, 1 if bf16 else 0, V, H, Wd, N, mode,
                                          BOX, nk, 0) == 0


@pytest.mark.parametrize("tf", [False, True])
@pytest.mark.parametrize("mode", [BL, RAW, ALPHA])
def test_render_staged_boxes(dev, mode, tf):
    """The LDS-staged forward (2 volumes x 2 channels, 2 views each, 96 x 96
    detector: 73,728 rays over a 16^3 volume) against the oracle, with the
    transfer function applied as the boxes are filled."""
    seed = 500 + 2 * mode + tf
    vol, spacing, K, poses, H, Wd, N, g = problem(seed, shape=(16, 16, 16), det=(96, 96), N=37,
                                                   tf=tf)
    transfer = knots(2) if tf else None
    assert _is_staged(vol, H, Wd, N, poses.shape[0], mode, 3 if tf else 0)
    f = 25.0 if tf else 0.8
    say(f"case: staged render mode={mode} tf={tf}")
    img, tau, grad = run_gpu(dev, vol, spacing, K, poses, H, Wd, N, mode, f, BOX, 0.0, transfer,
                             g)
    kw = dict(density_factor=f, transfer=transfer)
    ref, ref_tau = oracle.render(vol, spacing, K, poses, H, Wd, N, mode, **kw)
    ref_g = oracle.render_adjoint(vol, spacing, K, poses, H, Wd, N, mode, g, **kw)
    check(img, tau, grad, ref, ref_tau, ref_g, f"staged m{mode} tf{int(tf)}")


def test_render_staged_bf16(dev):
    vol, spacing, K, poses, H, Wd, N, g = problem(510, shape=(16, 16, 16), det=(96, 96), N=37)
    bits = W.round_to_bf16_bits(vol)
    vol_r = (bits.astype(np.uint32) << 16).view(np.float32)
    assert _is_staged(vol, H, Wd, N, poses.shape[0], BL, 0, bf16=True)
    say("case: staged render bf16")
    img, tau, grad = run_gpu(dev, vol, spacing, K, poses, H, Wd, N, BL, 1.0, BOX, 0.0, None, g,
                             bf16_bits=bits)
    ref, ref_tau = oracle.render(vol_r, spacing, K, poses, H, Wd, N, BL)
    ref_g = oracle.render_adjoint(vol_r, spacing, K, poses, H, Wd, N, BL, g)
    check(img, tau, grad, ref, ref_tau, ref_g, "staged bf16")


def _pose_is_staged(vol, H, Wd, N, V, nk, bf16=False):
    """The pose gradient stages boxes exactly when its workspace holds only the
    fp64 view sums (12 per view, 256-byte multiple)."""
    B, C, nz, ny, nx = vol.shape
    ws = drr.drr_render_workspace_bytes(B, C, nz, ny, nx, 1 if bf16 else 0, V, H, Wd, N, BL,
                                        BOX, nk, 2)
    return ws == (V * 12 * 8 + 255) // 256 * 256


@pytest.mark.parametrize("tf", [False, True])
@pytest.mark.parametrize("mode", [BL, RAW, ALPHA])
def test_render_staged_pose_gradient(dev, mode, tf):
    """The LDS-staged pose gradient (2 volumes x 2 channels, 2 views each,
    96 x 96 detector over a 16^3 volume, as the staged forward test), with the
    transfer function applied as the boxes are filled."""
    seed = 530 + 2 * mode + tf
    vol, spacing, K, poses, H, Wd, N, g = problem(seed, shape=(16, 16, 16), det=(96, 96), N=37,
                                                   tf=tf)
    transfer = knots(2) if tf else None
    nk = 3 if tf else 0
    assert _pose_is_staged(vol, H, Wd, N, poses.shape[0], nk)
    f = 25.0 if tf else 0.8
    say(f"case: staged pose gradient mode={mode} tf={tf}")
    gp = drr.drr_render_backward_pose(torch.from_numpy(vol).to(dev), spacing, K,
                                      torch.from_numpy(poses).to(dev), H, Wd, N, mode,
                                      torch.from_numpy(g).to(dev), f, BOX, 0.0, transfer)
    torch.cuda.synchronize()
    ref = oracle.render_pose_gradient(vol, spacing, K, poses, H, Wd, N, mode, g,
                                      density_factor=f, transfer=transfer)
    got = gp.cpu().double().numpy()
    errs = [np.abs(got[i] - ref[i]).max() / np.abs(ref[i]).max() for i in range(len(ref))]
    say(f"staged pose m{mode} tf{int(tf)}: per-view normwise err max {max(errs):.3e}")
    assert max(errs) <= GRAD


def test_render_staged_pose_gradient_bf16_and_diverging_rays(dev):
    """The staged pose gradient on a bf16 volume, and with the ~150 degree
    camera inside a 64^3 volume whose chunks fall back to global gathers."""
    vol, spacing, K, poses, H, Wd, N, g = problem(540, shape=(16, 16, 16), det=(96, 96), N=37)
    bits = W.round_to_bf16_bits(vol)
    vol_r = (bits.astype(np.uint32) << 16).view(np.float32)
    assert _pose_is_staged(vol, H, Wd, N, poses.shape[0], 0, bf16=True)
    say("case: staged pose gradient bf16")
    v = torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)
    gp = drr.drr_render_backward_pose(v, spacing, K, torch.from_numpy(poses).to(dev), H, Wd, N,
                                      BL, torch.from_numpy(g).to(dev), 1.0, BOX, 0.0, None)
    torch.cuda.synchronize()
    ref = oracle.render_pose_gradient(vol_r, spacing, K, poses, H, Wd, N, BL, g)
    got = gp.cpu().double().numpy()
    errs = [np.abs(got[i] - ref[i]).max() / np.abs(ref[i]).max() for i in range(len(ref))]
    say(f"staged pose bf16: per-view normwise err max {max(errs):.3e}")
    assert max(errs) <= GRAD

    rng = np.random.default_rng(541)
    vol = rng.uniform(0.0, 1.0, size=(1, 1, 64, 64, 64)).astype(np.float32)
    spacing = np.ones(3, dtype=np.float32)
    K = W.intrinsics(32.0, 128.0, 128.0)
    pose = W.pose_from_rotation_and_centre(np.eye(3), np.array([3.0, -2.0, -20.0]))[None]
    H = Wd = 256
    N = 80
    assert _pose_is_staged(vol, H, Wd, N, 1, 0)
    g = rng.uniform(-1, 1, size=(1, 1, H, Wd)).astype(np.float32)
    say("case: staged pose gradient, diverging rays")
    gp = drr.drr_render_backward_pose(torch.from_numpy(vol).to(dev), spacing, K,
                                      torch.from_numpy(pose).to(dev), H, Wd, N, RAW,
                                      torch.from_numpy(g).to(dev), 1.0, BOX, 0.0, None)
    torch.cuda.synchronize()
    ref = oracle.render_pose_gradient(vol, spacing, K, pose, H, Wd, N, RAW, g)
    got = gp.cpu().double().numpy()
    err = np.abs(got[0] - ref[0]).max() / np.abs(ref[0]).max()
    say(f"staged pose diverging: normwise err {err:.3e}")
    assert err <= GRAD


def test_render_staged_diverging_rays_fall_back_to_global_gathers(dev):
    """A camera inside a 64^3 volume with a ~150 degree field of view: a tile's
    rays spread over more voxels than a staged box holds even for one sample,
    so those chunks gather from global memory; the result still matches."""
    rng = np.random.default_rng(520)
    shape = (64, 64, 64)
    vol = rng.uniform(0.0, 1.0, size=(1, 1) + shape).astype(np.float32)
    spacing = np.ones(3, dtype=np.float32)
    K = W.intrinsics(32.0, 128.0, 128.0)
    pose = W.pose_from_rotation_and_centre(np.eye(3), np.array([3.0, -2.0, -20.0]))[None]
    H = Wd = 256
    N = 80
    assert _is_staged(vol, H, Wd, N, 1, RAW, 0)
    g = rng.uniform(-1, 1, size=(1, 1, H, Wd)).astype(np.float32)
    say("case: staged render, diverging rays")
    img, tau, grad = run_gpu(dev, vol, spacing, K, pose, H, Wd, N, RAW, 1.0, BOX, 0.0, None, g)
    ref, ref_tau = oracle.render(vol, spacing, K, pose, H, Wd, N, RAW)
    ref_g = oracle.render_adjoint(vol, spacing, K, pose, H, Wd, N, RAW, g)
    check(img, tau, grad, ref, ref_tau, ref_g, "staged diverging")
