"""GPU parity of the cell-constant (Siddon) projector pair against the oracle.

diffct 2.1.0, "Why diffct" feature list: project() and backproject() are an
exact adjoint pair for the cell-constant Siddon model.  The HIP pair
(drr_forward_siddon / drr_backward_volume_siddon, through the C ABI) is checked
against the oracle's merged-crossing traversal on the same seeded inputs, with
the trilinear path's bars:
  * forward, fp32 volume:   max |g - o| / max(|o|, 1e-3 max|o|) <= 1e-5
  * forward, bf16 volume:   <= 1e-2 against the fp32-volume oracle, <= 1e-5
                            against the oracle on the bf16-rounded volume
  * volume gradient:        max |g - o| / max |o| <= 1e-4 (normwise)
  * misses:                 exactly 0
"""
import numpy as np
import pytest
import torch

import ct_forward_projection_amd as drr
import oracle
import workloads as W
from helpers import check_forward, l2_err, normwise_err, say

pytestmark = pytest.mark.gpu

FWD_F32 = 1e-5
FWD_BF16 = 1e-2
GRAD = 1e-4


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def siddon_forward(w, dev, bf16=False):
    if bf16:
        vol = torch.from_numpy(w.volume_bf16.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        vol = torch.from_numpy(w.volume).to(dev)
    poses = torch.from_numpy(w.poses).to(dev)
    img, s = drr.drr_forward_siddon(vol, w.spacing, w.K, poses, w.det_h, w.det_w, w.mode)
    torch.cuda.synchronize()
    return img, s


def siddon_backward(w, dev, s, g):
    poses = torch.from_numpy(w.poses).to(dev)
    grad = drr.drr_backward_volume_siddon(w.volume.shape, w.spacing, w.K, poses, w.det_h,
                                          w.det_w, w.mode, torch.from_numpy(g).to(dev), s)
    torch.cuda.synchronize()
    return grad.cpu().double().numpy()


def check_grad(grad, ref, what):
    err = normwise_err(grad, ref)
    say(f"{what}: gradient normwise err {err:.3e}, l2 {l2_err(grad, ref):.3e}")
    assert err <= GRAD


@pytest.mark.parametrize("seed,mode,shape,det,spacing,distance", [
    (401, W.BEER_LAMBERT, (7, 9, 11), (13, 17), (1.0, 1.25, 0.8), 60.0),
    (402, W.LINE_INTEGRAL, (16, 5, 33), (40, 23), (0.7, 1.0, 1.3), 60.0),
    (403, W.BEER_LAMBERT, (1, 12, 12), (17, 33), (1.0, 1.0, 1.0), 60.0),
    (404, W.LINE_INTEGRAL, (20, 20, 1), (9, 50), (1.0, 1.0, 1.0), 60.0),
    (405, W.BEER_LAMBERT, (31, 29, 27), (65, 47), (1.0, 1.25, 0.8), 60.0),
    (406, W.LINE_INTEGRAL, (20, 20, 20), (21, 21), (1.0, 1.0, 1.0), 3.0),   # sources inside
])
def test_siddon_random_ragged(dev, seed, mode, shape, det, spacing, distance):
    """Ragged tiles, anisotropic voxels, one-voxel-thick volumes, sources inside."""
    w = W.make_random_small(seed, shape=shape, n_views=3, det=det, n_samples=1, mode=mode,
                            spacing=spacing, distance=distance)
    say(f"case: siddon random seed={seed} mode={mode} shape={shape} det={det}")
    img, s = siddon_forward(w, dev)
    ref, ref_s = oracle.siddon_forward_workload(w)
    check_forward(img, ref, FWD_F32, f"siddon {seed}", oracle.chords_workload(w))
    check_forward(s, ref_s, FWD_F32, f"siddon {seed} s")
    grad = siddon_backward(w, dev, s, w.grad_out)
    ref_g, _ = oracle.siddon_adjoint_workload(w)
    check_grad(grad, ref_g, f"siddon {seed}")


@pytest.fixture(scope="module")
def batch_workload():
    return W.make_workload(2, with_bf16=True)


def test_siddon_batch_fp32_and_bf16(dev, batch_workload):
    w = batch_workload
    say("case: siddon batch 256^3 x 16 views 200x200")
    img, _ = siddon_forward(w, dev)
    ref32, _ = oracle.siddon_forward_workload(w)
    check_forward(img, ref32, FWD_F32, "siddon batch fp32", oracle.chords_workload(w))
    img16, _ = siddon_forward(w, dev, bf16=True)
    ref16, _ = oracle.siddon_forward_workload(w, use_bf16=True)
    check_forward(img16, ref32, FWD_BF16, "siddon batch bf16 vs fp32 oracle")
    check_forward(img16, ref16, FWD_F32, "siddon batch bf16 vs bf16-rounded oracle")


def test_siddon_batch_backward_bricks(dev, batch_workload):
    """The 16-view 200^2 batch is sparse against the 256^3 voxels (about 0.6
    pieces per voxel from one view): the brick-owned backward.  Full-size
    gradient against the oracle, and bit-identical on a second run (exact
    fixed-point sums, each voxel written once)."""
    w = batch_workload
    say("case: siddon batch backward (bricks) 256^3 x 16 views 200x200")
    g = np.random.default_rng(2203).uniform(-1, 1, size=(w.n_views, w.det_h, w.det_w))
    g = g.astype(np.float32)
    _, s = siddon_forward(w, dev)
    grad = siddon_backward(w, dev, s, g)
    ref_g, _ = oracle.siddon_adjoint_workload(w, grad_out=g)
    check_grad(grad, ref_g, "siddon batch bricks")
    again = siddon_backward(w, dev, s, g)
    assert np.array_equal(grad, again)


@pytest.mark.parametrize("mode", [W.BEER_LAMBERT, W.LINE_INTEGRAL])
def test_siddon_bricks_many_views_ragged(dev, mode):
    """More views than one chunk of the brick search (40 > 16), a volume whose
    sides are not multiples of the brick, anisotropic voxels, every ray
    checked."""
    w = W.make_random_small(2211 + mode, shape=(37, 21, 45), n_views=40, det=(11, 13),
                            n_samples=1, mode=mode, spacing=(0.9, 1.3, 1.1), distance=90.0)
    say(f"case: siddon bricks 40 views 11x13 over 45x21x37 mode={mode}")
    _, s = siddon_forward(w, dev)
    grad = siddon_backward(w, dev, s, w.grad_out)
    ref_g, _ = oracle.siddon_adjoint_workload(w)
    check_grad(grad, ref_g, "siddon bricks many views")


def test_siddon_bricks_non_finite_upstream(dev):
    """NaN and +inf upstream gradients on the brick path: exactly the voxels the
    oracle makes NaN (or +inf) are, the others match it."""
    w = W.make_random_small(2221, shape=(30, 26, 34), n_views=3, det=(15, 17), n_samples=1,
                            mode=W.LINE_INTEGRAL, distance=80.0)
    g = w.grad_out.copy()
    g[0, 7, 8] = np.nan
    g[2, 4, 11] = np.inf
    _, s = siddon_forward(w, dev)
    grad = siddon_backward(w, dev, s, g)
    ref_g, _ = oracle.siddon_adjoint_workload(w, grad_out=g)
    say(f"siddon bricks non-finite: {int(np.isnan(ref_g).sum())} NaN, "
        f"{int(np.isinf(ref_g).sum())} inf voxels in the oracle")
    assert np.isnan(ref_g).any() and np.isinf(ref_g).any()
    assert np.array_equal(np.isnan(grad), np.isnan(ref_g))
    assert np.array_equal(np.isposinf(grad), np.isposinf(ref_g))
    ok = np.isfinite(ref_g)
    check_grad(grad[ok], ref_g[ok], "siddon bricks non-finite (finite voxels)")


def test_siddon_bricks_deep_attenuation(dev):
    """Beer-Lambert on the brick path with every ray that meets the volume at
    optical depth 13 or more (voxels 4.85 long in x), so its coefficient
    g exp(-s) is 1e-6 of g or less, while pixels of the bricks' candidate
    rectangles whose rays miss the volume keep y = g.  The fixed-point unit has
    to follow the rays that cross a brick: taken over all candidates it sat
    near the pieces' own size here (normwise error 6e-3)."""
    shape, det = (22, 21, 17), (22, 39)
    spacing = (4.85, 0.6, 2.54)
    w = W.make_random_small(72646, shape=shape, n_views=2, det=det, n_samples=656,
                            mode=W.BEER_LAMBERT, spacing=spacing, distance=443.0, rot_deg=0.0)
    cells = (shape[0] + 1) * (shape[1] + 1) * (shape[2] + 1)
    assert det[0] * det[1] * max(shape) / cells < 4.0          # views sparse: bricks
    say(f"case: siddon bricks deep attenuation {shape} det={det} spacing={spacing}")
    _, s = siddon_forward(w, dev)
    sv = s.cpu().double().numpy()
    hit = sv > 0
    say(f"siddon deep attenuation: {int(hit.sum())} rays meet the volume, optical depth "
        f"{sv[hit].min():.1f}..{sv[hit].max():.1f}; {int((~hit).sum())} miss")
    assert sv[hit].min() > 13.0 and (~hit).any()
    grad = siddon_backward(w, dev, s, w.grad_out)
    ref_g, _ = oracle.siddon_adjoint_workload(w)
    check_grad(grad, ref_g, "siddon bricks deep attenuation")


def test_siddon_train_size_forward_and_backward(dev):
    w = W.make_workload(3)
    say("case: siddon 256^3 1024x1024 BL fwd+bwd")
    img, s = siddon_forward(w, dev)
    ref, _ = oracle.siddon_forward_workload(w)
    check_forward(img, ref, FWD_F32, "siddon 1024", oracle.chords_workload(w))
    grad = siddon_backward(w, dev, s, w.grad_out)
    ref_g, _ = oracle.siddon_adjoint_workload(w)
    check_grad(grad, ref_g, "siddon 1024")


SAMPLED_VIEWS = np.arange(0, 360, 15)


def test_siddon_helix(dev):
    """360 views in one launch, 24 checked against the oracle; the adjoint
    identity <A x, y> = <x, A^T y> at full size on the GPU."""
    w = W.make_workload(5)
    say("case: siddon helix 128^3 360 views 256x384 RAW")
    img, _ = siddon_forward(w, dev)
    sub = w.subset_views(SAMPLED_VIEWS)
    ref, _ = oracle.siddon_forward_workload(sub)
    check_forward(img[torch.from_numpy(SAMPLED_VIEWS).to(dev)], ref, FWD_F32,
                  "siddon helix views", oracle.chords_workload(sub))
    _, s = siddon_forward(sub, dev)
    grad = siddon_backward(sub, dev, s, sub.grad_out)
    ref_g, _ = oracle.siddon_adjoint_workload(sub)
    check_grad(grad, ref_g, "siddon helix sampled")

    x = torch.from_numpy(w.volume).to(dev)
    poses = torch.from_numpy(w.poses).to(dev)
    y = torch.from_numpy(w.grad_out).to(dev)
    ax = drr.project_siddon(x, w.spacing, w.K, poses, w.det_h, w.det_w)
    aty = drr.backproject_siddon(y, w.volume.shape, w.spacing, w.K, poses, w.det_h, w.det_w)
    lhs = float((ax.double() * y.double()).sum())
    rhs = float((x.double() * aty.double()).sum())
    say(f"siddon helix: <Ax,y> = {lhs:.9e}, <x,A^T y> = {rhs:.9e}, "
        f"rel {abs(lhs - rhs) / abs(lhs):.2e}")
    assert abs(lhs - rhs) <= 1e-5 * abs(lhs)


def test_siddon_ray_in_a_voxel_plane(dev):
    """Rays parallel to two axes, one of them lying exactly in a voxel plane
    x = 0: both sides give it the voxel of higher index (floor at an exact
    integer), and the parallel axes never step."""
    rng = np.random.default_rng(41)
    vol = rng.uniform(0.0, 1.0, size=(6, 8, 10)).astype(np.float32)
    # f = 64 keeps K^-1 dyadic, so the principal ray's x and y components are
    # exactly 0 on both sides (a tiny nonzero component would decide the side)
    K = np.array([[64.0, 0.0, 3.5], [0.0, 64.0, 2.5], [0.0, 0.0, 1.0]], dtype=np.float32)
    poses = np.stack([W.pose_from_rotation_and_centre(np.eye(3), [0.0, 0.3, -80.0]),
                      W.pose_from_rotation_and_centre(np.eye(3), [1.2, -0.7, -80.0])])
    w = W.Workload("plane", vol, np.ones(3, np.float32), K, poses, 5, 7, 1, W.LINE_INTEGRAL,
                   grad_out=rng.uniform(-1, 1, size=(2, 5, 7)).astype(np.float32))
    img, s = siddon_forward(w, dev)
    ref, _ = oracle.siddon_forward_workload(w)
    check_forward(img, ref, FWD_F32, "voxel plane", oracle.chords_workload(w))
    # pixel (2, 3) of view 0 is the ray x = 0, y = 0.3 along +z: column (5, 4)
    assert float(img[0, 2, 3]) == pytest.approx(float(vol[:, 4, 5].astype(np.float64).sum()),
                                                rel=1e-6)
    grad = siddon_backward(w, dev, s, w.grad_out)
    ref_g, _ = oracle.siddon_adjoint_workload(w)
    check_grad(grad, ref_g, "voxel plane")


def test_siddon_sources_inside_wide_field_of_view(dev):
    """Sources inside the volume with a ~130 degree field of view (bricks that
    straddle the camera plane search the whole detector)."""
    rng = np.random.default_rng(51)
    vol = rng.uniform(0.0, 1.0, size=(48, 48, 48)).astype(np.float32)
    K = W.intrinsics(4.0, 8.0, 8.0)
    poses = W.random_poses(2, 2.0, 30.0, 1.0, seed=52)
    w = W.Workload("inside-wide-fov", vol, np.ones(3, np.float32), K, poses, 16, 16, 1,
                   W.LINE_INTEGRAL,
                   grad_out=rng.uniform(-1, 1, size=(2, 16, 16)).astype(np.float32))
    img, s = siddon_forward(w, dev)
    ref, _ = oracle.siddon_forward_workload(w)
    check_forward(img, ref, FWD_F32, "siddon wide fov", oracle.chords_workload(w))
    grad = siddon_backward(w, dev, s, w.grad_out)
    ref_g, _ = oracle.siddon_adjoint_workload(w)
    check_grad(grad, ref_g, "siddon wide fov")


def test_siddon_all_miss_and_empty(dev):
    w = W.make_random_small(411, n_views=2, n_samples=1)
    w.poses = np.stack([W.pose_from_rotation_and_centre(np.diag([1.0, -1.0, -1.0]),
                                                        [0.0, 0.0, -200.0])] * 2)
    img, s = siddon_forward(w, dev)
    assert torch.count_nonzero(img).item() == 0 and torch.count_nonzero(s).item() == 0
    assert not siddon_backward(w, dev, s, w.grad_out).any()
    vol = torch.rand(8, 8, 8, device=dev)
    none = torch.zeros(0, 3, 4, device=dev)
    img, _ = drr.drr_forward_siddon(vol, [1, 1, 1], W.intrinsics(10, 2, 2), none, 4, 4)
    assert img.shape == (0, 4, 4)
    grad = torch.full((8, 8, 8), 7.0, device=dev)
    drr.drr_backward_volume_siddon((8, 8, 8), [1, 1, 1], W.intrinsics(10, 2, 2), none, 4, 4,
                                   drr.LINE_INTEGRAL, torch.zeros(0, 4, 4, device=dev), None,
                                   grad_volume=grad)
    torch.cuda.synchronize()
    assert torch.count_nonzero(grad).item() == 0


def test_siddon_nan_voxel_reaches_exactly_the_rays_through_it(dev):
    """A NaN voxel makes exactly the rays that cross it (with positive length,
    per the oracle) NaN; zero-length touches do not leak it."""
    w = W.make_random_small(421, shape=(10, 11, 12), n_views=2, det=(19, 23), n_samples=1,
                            mode=W.LINE_INTEGRAL)
    w.volume[5, 6, 7] = np.nan
    img, _ = siddon_forward(w, dev)
    ref, _ = oracle.siddon_forward_workload(w)
    g = img.cpu().double().numpy()
    assert np.isnan(ref).any()
    assert np.array_equal(np.isnan(g), np.isnan(ref))
    ok = ~np.isnan(ref)
    check_forward(g[ok], ref[ok], FWD_F32, "siddon NaN voxel (finite rays)")


def test_siddon_forward_is_deterministic_and_autograd_matches(dev):
    w = W.make_random_small(431, shape=(12, 14, 16), n_views=2, det=(20, 24), n_samples=1,
                            mode=W.BEER_LAMBERT)
    a, _ = siddon_forward(w, dev)
    b, _ = siddon_forward(w, dev)
    assert torch.equal(a, b)
    vol = torch.from_numpy(w.volume).to(dev).requires_grad_(True)
    poses = torch.from_numpy(w.poses).to(dev)
    img = drr.render_siddon(vol, w.spacing, w.K, poses, w.det_h, w.det_w, w.mode)
    (img * torch.from_numpy(w.grad_out).to(dev)).sum().backward()
    ref_g, _ = oracle.siddon_adjoint_workload(w)
    check_grad(vol.grad.cpu().double().numpy(), ref_g, "siddon autograd")
