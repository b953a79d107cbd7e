"""GPU parity: the HIP library (through its C ABI) against the CPU oracle, on the
same seeded inputs.

Bars (floating point; the oracle is fp64):
  * forward, fp32 volume:   max |g - o| / max(|o|, 1e-3 max|o|) <= 1e-5
  * forward, bf16 volume:   <= 1e-2 against the oracle on the fp32 volume and
                            <= 1e-5 against the oracle on the bf16-rounded volume
                            (fp32 accumulation, no bf16 arithmetic)
  * volume gradient:        max |g - o| / max |o| <= 1e-4 (normwise)
  * misses:                 exactly 0 wherever the oracle's ray misses the box
The full-size workloads run in the launch configuration the benchmark times and
are compared with the oracle element by element, the 360-view helix included
(forward image and volume gradient); the adjoint identity is checked at that
size as well.
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


def gpu_forward(w, dev, bf16=False, stream=None):
    if bf16:
        vol = torch.from_numpy(w.volume_bf16.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        vol = torch.from_numpy(w.volume).to(dev)
    poses = torch.from_numpy(w.poses).to(dev)
    img, s = drr.drr_forward(vol, w.spacing, w.K, poses, w.det_h, w.det_w, w.n_samples, w.mode,
                             stream=stream)
    torch.cuda.synchronize()
    return img, s


def gpu_backward(w, dev, s, g):
    poses = torch.from_numpy(w.poses).to(dev)
    grad = drr.drr_backward_volume(w.volume.shape, w.spacing, w.K, poses, w.det_h, w.det_w,
                                   w.n_samples, w.mode, torch.from_numpy(g).to(dev), s)
    torch.cuda.synchronize()
    return grad.cpu().double().numpy()


# ------------------------------------------------------------------ the five workloads

def test_tiny_workload_forward(dev):
    w = W.make_workload(1)
    say("case: tiny 64^3 forward BL")
    img, s = gpu_forward(w, dev)
    ref, ref_s = oracle.forward_workload(w)
    check_forward(img, ref, FWD_F32, "tiny", oracle.chords_workload(w))
    check_forward(s, ref_s, FWD_F32, "tiny s")


def test_tiny_workload_backward(dev):
    w = W.make_workload(1)
    say("case: tiny 64^3 backward BL")
    g = np.random.default_rng(1).uniform(-1, 1, size=(1, 64, 64)).astype(np.float32)
    _, s = gpu_forward(w, dev)
    grad = gpu_backward(w, dev, s, g)
    ref, _ = oracle.adjoint_workload(w, grad_out=g)
    err = normwise_err(grad, ref)
    say(f"tiny: gradient normwise err {err:.3e}, l2 {l2_err(grad, ref):.3e}")
    assert err <= GRAD


@pytest.fixture(scope="module")
def batch_workload():
    return W.make_workload(2, with_bf16=True)


def test_nanodrr_batch_forward_fp32(dev, batch_workload):
    w = batch_workload
    say("case: batch 256^3 x 16 views 200x200 fp32")
    img, s = gpu_forward(w, dev)
    ref, _ = oracle.forward_workload(w)
    check_forward(img, ref, FWD_F32, "batch fp32", oracle.chords_workload(w))


def test_nanodrr_batch_forward_bf16(dev, batch_workload):
    w = batch_workload
    say("case: batch 256^3 x 16 views 200x200 bf16")
    img, _ = gpu_forward(w, dev, bf16=True)
    ref32, _ = oracle.forward_workload(w)
    ref16, _ = oracle.forward_workload(w, use_bf16=True)
    check_forward(img, ref32, FWD_BF16, "batch bf16 vs fp32 oracle")
    check_forward(img, ref16, FWD_F32, "batch bf16 vs bf16-rounded oracle")


def test_train_step_forward_and_backward(dev):
    w = W.make_workload(3)
    say("case: train step 256^3 1024x1024 512 samples fwd+bwd")
    img, s = gpu_forward(w, dev)
    ref, ref_s = oracle.forward_workload(w)
    check_forward(img, ref, FWD_F32, "train fwd", oracle.chords_workload(w))
    grad = gpu_backward(w, dev, s, w.grad_out)
    ref_g, _ = oracle.adjoint_workload(w)
    err = normwise_err(grad, ref_g)
    say(f"train: gradient normwise err {err:.3e}, l2 {l2_err(grad, ref_g):.3e}")
    assert err <= GRAD


def test_hires_forward(dev):
    w = W.make_workload(4)
    say("case: hires 256^3 2048x2048 256 samples fwd")
    img, _ = gpu_forward(w, dev)
    ref, _ = oracle.forward_workload(w)
    check_forward(img, ref, FWD_F32, "hires", oracle.chords_workload(w))


@pytest.fixture(scope="module")
def helix():
    return W.make_workload(5)


@pytest.mark.timeout(900)
def test_cbct_helix_forward_full(dev, helix):
    """All 360 views render in one launch (the benchmark's configuration) and
    every pixel of every view is compared with the oracle (9.06 G samples)."""
    w = helix
    say("case: helix 128^3 360 views 256x384 RAW fwd, all views against the oracle")
    img, _ = gpu_forward(w, dev)
    ref, _ = oracle.forward_workload(w)
    check_forward(img, ref, FWD_F32, "helix, 360 views", oracle.chords_workload(w))


@pytest.mark.timeout(900)
def test_cbct_helix_backward_full(dev, helix):
    """The gradient of the full 360-view launch against the oracle's, element by
    element, and the adjoint identity <A x, y> = <x, A^T y> at that size."""
    w = helix
    say("case: helix backward, 360 views, all voxels against the oracle")
    _, s = gpu_forward(w, dev)
    grad = gpu_backward(w, dev, s, w.grad_out)
    ref, used = oracle.adjoint_workload(w)
    err = normwise_err(grad, ref)
    say(f"helix 360 views: gradient normwise err {err:.3e}, l2 {l2_err(grad, ref):.3e} "
        f"(oracle on {used} threads)")
    assert err <= GRAD

    say("case: helix full-size adjoint identity")
    x = torch.from_numpy(w.volume).to(dev)
    poses = torch.from_numpy(w.poses).to(dev)
    y = torch.from_numpy(w.grad_out).to(dev)
    ax = drr.project(x, w.spacing, w.K, poses, w.det_h, w.det_w, w.n_samples)
    aty = drr.backproject(y, w.volume.shape, w.spacing, w.K, poses, w.det_h, w.det_w,
                          w.n_samples)
    lhs = float((ax.double() * y.double()).sum())
    rhs = float((x.double() * aty.double()).sum())
    say(f"helix: <Ax,y> = {lhs:.9e}, <x,A^T y> = {rhs:.9e}, rel {abs(lhs - rhs) / abs(lhs):.2e}")
    assert abs(lhs - rhs) <= 1e-5 * abs(lhs)


# ------------------------------------------------------------------ ragged and edge cases

@pytest.mark.parametrize("seed,mode,shape,det,n", [
    (1, W.BEER_LAMBERT, (7, 9, 11), (13, 17), 37),
    (2, W.LINE_INTEGRAL, (16, 5, 33), (40, 23), 64),
    (3, W.BEER_LAMBERT, (1, 12, 12), (17, 33), 5),
    (4, W.LINE_INTEGRAL, (20, 20, 1), (9, 50), 1),
    (5, W.BEER_LAMBERT, (31, 29, 27), (65, 47), 203),
])
def test_random_ragged_workloads(dev, seed, mode, shape, det, n):
    """Tiles with ragged tails, anisotropic voxels, degenerate (1-voxel-thick)
    volumes, N = 1 and N not a multiple of the unroll."""
    w = W.make_random_small(seed, shape=shape, n_views=3, det=det, n_samples=n, mode=mode)
    say(f"case: random seed={seed} mode={mode} shape={shape} det={det} N={n}")
    img, s = gpu_forward(w, dev)
    ref, ref_s = oracle.forward_workload(w)
    check_forward(img, ref, FWD_F32, f"random {seed}", oracle.chords_workload(w))
    grad = gpu_backward(w, dev, s, w.grad_out)
    ref_g, _ = oracle.adjoint_workload(w)
    err = normwise_err(grad, ref_g)
    say(f"random {seed}: gradient normwise err {err:.3e}")
    assert err <= GRAD


def test_all_rays_miss(dev):
    w = W.make_random_small(11, n_views=2)
    w.poses = np.stack([W.pose_from_rotation_and_centre(np.diag([1.0, -1.0, -1.0]),
                                                        [0.0, 0.0, -200.0])] * 2)
    say("case: all rays miss")
    img, s = gpu_forward(w, dev)
    assert torch.count_nonzero(img).item() == 0 and torch.count_nonzero(s).item() == 0
    grad = gpu_backward(w, dev, s, w.grad_out)
    assert not grad.any()


def test_source_inside_the_volume(dev):
    w = W.make_random_small(12, shape=(20, 20, 20), n_views=2, det=(21, 21), n_samples=50,
                            distance=3.0)
    say("case: sources inside the volume")
    img, s = gpu_forward(w, dev)
    ref, _ = oracle.forward_workload(w)
    check_forward(img, ref, FWD_F32, "inside")
    grad = gpu_backward(w, dev, s, w.grad_out)
    ref_g, _ = oracle.adjoint_workload(w)
    assert normwise_err(grad, ref_g) <= GRAD


def test_empty_inputs(dev):
    say("case: empty inputs")
    vol = torch.rand(8, 8, 8, device=dev)
    poses = torch.zeros(0, 3, 4, device=dev)
    img, s = drr.drr_forward(vol, [1, 1, 1], W.intrinsics(10, 2, 2), poses, 4, 4, 8)
    assert img.shape == (0, 4, 4)
    # the backward overwrites: with no rays the gradient is all zeros
    grad = torch.full((8, 8, 8), 7.0, device=dev)
    drr.drr_backward_volume((8, 8, 8), [1, 1, 1], W.intrinsics(10, 2, 2), poses, 4, 4, 8,
                            drr.LINE_INTEGRAL, torch.zeros(0, 4, 4, device=dev), None,
                            grad_volume=grad)
    torch.cuda.synchronize()
    assert torch.count_nonzero(grad).item() == 0


def test_many_samples(dev):
    w = W.make_random_small(13, shape=(10, 12, 14), n_views=1, det=(8, 8), n_samples=5000)
    say("case: N = 5000")
    img, s = gpu_forward(w, dev)
    ref, _ = oracle.forward_workload(w)
    check_forward(img, ref, FWD_F32, "N=5000")


def test_forward_is_deterministic(dev):
    w = W.make_workload(1)
    a, _ = gpu_forward(w, dev)
    b, _ = gpu_forward(w, dev)
    assert torch.equal(a, b)


def test_backward_is_stable_run_to_run(dev):
    w = W.make_random_small(14, shape=(24, 24, 24), n_views=4, det=(48, 48), n_samples=96)
    _, s = gpu_forward(w, dev)
    g1 = gpu_backward(w, dev, s, w.grad_out)
    g2 = gpu_backward(w, dev, s, w.grad_out)
    assert normwise_err(g1, g2) <= 1e-6


def test_autograd_render_matches_abi(dev):
    w = W.make_random_small(15, shape=(12, 14, 16), n_views=2, det=(20, 24), n_samples=40)
    say("case: autograd")
    vol = torch.from_numpy(w.volume).to(dev).requires_grad_(True)
    poses = torch.from_numpy(w.poses).to(dev)
    img = drr.render(vol, w.spacing, w.K, poses, w.det_h, w.det_w, w.n_samples, w.mode)
    g = torch.from_numpy(w.grad_out).to(dev)
    (img * g).sum().backward()
    ref_g, _ = oracle.adjoint_workload(w)
    assert normwise_err(vol.grad.cpu().numpy(), ref_g) <= GRAD


def test_least_squares_gradient_is_At_residual(dev):
    """diffct Quickstart: for 0.5 ||A x - y||^2, x.grad = A^T (A x - y)."""
    w = W.make_random_small(16, shape=(10, 11, 12), n_views=3, det=(15, 16), n_samples=30,
                            mode=W.LINE_INTEGRAL)
    x = torch.from_numpy(w.volume).to(dev).requires_grad_(True)
    poses = torch.from_numpy(w.poses).to(dev)
    y = torch.from_numpy(w.grad_out).to(dev)
    ax = drr.render(x, w.spacing, w.K, poses, w.det_h, w.det_w, w.n_samples, drr.LINE_INTEGRAL)
    (0.5 * (ax - y).square().sum()).backward()
    r = (ax.detach().cpu().double().numpy() - w.grad_out)
    ref, _ = oracle.adjoint(None, w.volume.shape, w.spacing, w.K, w.poses, w.det_h, w.det_w,
                            w.n_samples, W.LINE_INTEGRAL, r)
    assert normwise_err(x.grad.cpu().numpy(), ref) <= GRAD


def test_runs_on_a_non_default_stream(dev):
    w = W.make_workload(1)
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        img, _ = gpu_forward(w, dev, stream=st)
    ref, _ = oracle.forward_workload(w)
    check_forward(img, ref, FWD_F32, "side stream")


def test_graph_capture_replays_match_eager(dev):
    """Forward and backward captured in a HIP graph (torch.cuda.graph on the
    current stream) replay to the eager results, several times, with eager work
    and synchronisations in between; the gradient zeroing is a kernel, so no
    memset node is recorded."""
    w = W.make_random_small(21, shape=(20, 18, 22), n_views=2, det=(33, 29), n_samples=60)
    vol = torch.from_numpy(w.volume).to(dev)
    poses = torch.from_numpy(w.poses).to(dev)
    g = torch.from_numpy(w.grad_out).to(dev)
    out = torch.empty((2, 33, 29), device=dev)
    s = torch.empty_like(out)
    grad = torch.empty(w.volume.shape, device=dev)

    def step():
        drr.drr_forward(vol, w.spacing, w.K, poses, 33, 29, 60, w.mode, out=out, line_integral=s)
        drr.drr_backward_volume(w.volume.shape, w.spacing, w.K, poses, 33, 29, 60, w.mode, g, s,
                                grad_volume=grad)

    step()
    torch.cuda.synchronize()
    ref_img, ref_grad = out.clone(), grad.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for i in range(4):
        out.fill_(-1.0)
        grad.fill_(123.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_img), f"replay {i}: image"
        assert normwise_err(grad.cpu().numpy(), ref_grad.cpu().numpy()) <= 1e-6, f"replay {i}"
        step()   # eager work between replays
        torch.cuda.synchronize()


def test_backward_window_fallback_for_diverging_rays(dev):
    """A source inside the volume with a ~150 degree field of view: a tile's rays
    spread over the whole 48^3 volume, so even a one-sample chunk overflows the
    LDS window and the scatter takes its global-atomic path."""
    rng = np.random.default_rng(31)
    vol = rng.uniform(0.0, 1.0, size=(48, 48, 48)).astype(np.float32)
    K = W.intrinsics(4.0, 8.0, 8.0)
    poses = W.random_poses(2, 2.0, 30.0, 1.0, seed=32)
    w = W.Workload("inside-wide-fov", vol, np.ones(3, np.float32), K, poses, 16, 16, 96,
                   W.LINE_INTEGRAL,
                   grad_out=rng.uniform(-1, 1, size=(2, 16, 16)).astype(np.float32))
    say("case: diverging rays, window fallback")
    img, s = gpu_forward(w, dev)
    ref, _ = oracle.forward_workload(w)
    check_forward(img, ref, FWD_F32, "wide fov", oracle.chords_workload(w))
    grad = gpu_backward(w, dev, s, w.grad_out)
    ref_g, _ = oracle.adjoint_workload(w)
    err = normwise_err(grad, ref_g)
    say(f"wide fov: gradient normwise err {err:.3e}")
    assert err <= GRAD


def test_non_finite_upstream_gradient_propagates(dev):
    """A NaN upstream gradient cannot go through fixed point: its tile falls back
    to float atomics, and exactly the voxels the oracle marks NaN (every corner
    of every sample of that ray) are NaN on the GPU; the rest still matches."""
    w = W.make_random_small(33, shape=(12, 14, 16), n_views=1, det=(20, 24), n_samples=40,
                            mode=W.LINE_INTEGRAL)
    g = w.grad_out.copy()
    g[0, 7, 11] = np.nan
    say("case: NaN upstream gradient")
    _, s = gpu_forward(w, dev)
    grad = gpu_backward(w, dev, s, g)
    ref, _ = oracle.adjoint_workload(w, grad_out=g)
    assert np.isnan(ref).any()
    assert np.array_equal(np.isnan(grad), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert normwise_err(grad[ok], ref[ok]) <= GRAD


# ------------------------------------------------------------------ pose gradient

def gpu_pose_grad(w, dev, g, bf16=False):
    if bf16:
        vol = torch.from_numpy(w.volume_bf16.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        vol = torch.from_numpy(w.volume).to(dev)
    poses = torch.from_numpy(w.poses).to(dev)
    out = drr.drr_backward_pose(vol, w.spacing, w.K, poses, w.det_h, w.det_w, w.n_samples,
                                w.mode, torch.from_numpy(np.ascontiguousarray(g)).to(dev))
    torch.cuda.synchronize()
    return out.cpu().double().numpy()


def check_pose(gpu, ref, what):
    """Per view, max |g - o| / max |o| over the twelve entries."""
    worst = 0.0
    for v in range(ref.shape[0]):
        worst = max(worst, normwise_err(gpu[v], ref[v]))
    say(f"{what}: pose gradient normwise err {worst:.3e}")
    assert worst <= GRAD
    return worst


@pytest.mark.parametrize("seed,mode,shape,det,n", [
    (61, W.BEER_LAMBERT, (9, 10, 11), (13, 17), 37),
    (62, W.LINE_INTEGRAL, (16, 5, 33), (40, 23), 64),
    (63, W.BEER_LAMBERT, (20, 20, 1), (9, 50), 9),
    (64, W.LINE_INTEGRAL, (31, 29, 27), (65, 47), 203),
])
def test_pose_gradient_random(dev, seed, mode, shape, det, n):
    w = W.make_random_small(seed, shape=shape, n_views=3, det=det, n_samples=n, mode=mode)
    say(f"case: pose gradient seed={seed} mode={mode} shape={shape} det={det} N={n}")
    ref = oracle.pose_gradient(w.volume, w.spacing, w.K, w.poses, w.det_h, w.det_w,
                               w.n_samples, w.mode, w.grad_out)
    check_pose(gpu_pose_grad(w, dev, w.grad_out), ref, f"random {seed}")


def test_pose_gradient_batch_workload(dev, batch_workload):
    """The 16-view 200x200 batch (z-pair copies in fp32 and bf16)."""
    w = batch_workload
    g = np.random.default_rng(71).uniform(-1, 1, size=(16, 200, 200)).astype(np.float32)
    say("case: pose gradient, 16-view batch")
    ref = oracle.pose_gradient(w.volume, w.spacing, w.K, w.poses, 200, 200, 256, w.mode, g)
    check_pose(gpu_pose_grad(w, dev, g), ref, "batch fp32")
    ref16 = oracle.pose_gradient(w.volume_bf16_as_f32(), w.spacing, w.K, w.poses, 200, 200, 256,
                                 w.mode, g)
    check_pose(gpu_pose_grad(w, dev, g, bf16=True), ref16, "batch bf16")


def test_pose_gradient_train_workload_row_band(dev):
    """The 1024^2 train-step camera restricted to a 96-row band through the
    volume's centre (same rays; cy moved so the band is the whole detector)."""
    w = W.make_workload(3)
    K = w.K.copy()
    K[1, 2] -= 464.0                  # rows 464..559 of the full detector
    band = W.Workload("train-band", w.volume, w.spacing, K, w.poses, 96, 1024, 512, w.mode,
                      grad_out=np.ascontiguousarray(w.grad_out[:, 464:560, :]))
    say("case: pose gradient, 1024-wide band of the train-step camera")
    ref = oracle.pose_gradient(band.volume, band.spacing, band.K, band.poses, 96, 1024, 512,
                               band.mode, band.grad_out)
    check_pose(gpu_pose_grad(band, dev, band.grad_out), ref, "train band")


def test_pose_gradient_through_autograd(dev):
    w = W.make_random_small(65, shape=(12, 14, 16), n_views=2, det=(20, 24), n_samples=40)
    vol = torch.from_numpy(w.volume).to(dev).requires_grad_(True)
    poses = torch.from_numpy(w.poses).to(dev).requires_grad_(True)
    img = drr.render(vol, w.spacing, w.K, poses, w.det_h, w.det_w, w.n_samples, w.mode)
    (img * torch.from_numpy(w.grad_out).to(dev)).sum().backward()
    ref = oracle.pose_gradient(w.volume, w.spacing, w.K, w.poses, w.det_h, w.det_w,
                               w.n_samples, w.mode, w.grad_out)
    check_pose(poses.grad.cpu().double().numpy(), ref, "autograd")
    ref_v, _ = oracle.adjoint_workload(w)
    assert normwise_err(vol.grad.cpu().numpy(), ref_v) <= GRAD
