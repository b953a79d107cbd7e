"""GPU parity on large volumes: the 32-bit unsigned buffer offsets the library
uses for reads (and the element offsets of the gradient) above 2 GiB, and a
512^3 volume under the 1024^2 x 512-sample camera of the train step.

Bars as in test_gpu_parity: forward max |g - o| / max(|o|, 1e-3 max|o|) <= 1e-5
(misses exactly 0), gradient max |g - o| / max |o| <= 1e-4."""
import numpy as np
import pytest
import torch

import ct_forward_projection_amd as drr
import oracle
import workloads as W
from helpers import check_forward, normwise_err, say

pytestmark = pytest.mark.gpu

FWD_F32 = 1e-5
GRAD = 1e-4


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _views_along_y_and_x(distance):
    """Two cameras through the volume centre: one looking along +y (image rows
    along -z, columns along +x) and one along +x (rows along -z, columns along
    -y).  HZ rows of R: image x, image y (down), viewing direction."""
    ex, ey, ez = np.eye(3)
    r_y = np.stack([ex, -ez, ey])
    r_x = np.stack([-ey, -ez, ex])
    return np.stack([W.pose_from_rotation_and_centre(r_y, -distance * ey),
                     W.pose_from_rotation_and_centre(r_x, -distance * ex)])


@pytest.mark.timeout(900)
def test_volume_above_2gib_forward_and_backward(dev):
    """A 640 x 1024 x 1024 fp32 volume (2.68 GB, 671 M voxels): slices above
    z = 512 sit beyond 2^31 bytes.  Two small views cover the whole z range, so
    their samples read (and their gradients write) both halves."""
    shape = (640, 1024, 1024)
    rng = np.random.default_rng(501)
    # mu in [0, 0.004)/mm: optical depths of 1 to 2 over the ~1000 mm chords, so
    # neither the image saturates nor exp(-s) underflows fp32
    vol = rng.random(shape, dtype=np.float32) * np.float32(0.004)
    sp = np.ones(3, np.float32)
    poses = _views_along_y_and_x(2500.0)
    # at the near face (1988 mm) 40 rows cover +-331 mm of z (the top and bottom
    # rows leave through the z faces) and 56 columns +-464 mm across
    K = W.intrinsics(120.0, 28.0, 20.0)
    H, Wd, N = 40, 56, 256
    g = rng.uniform(-1.0, 1.0, size=(2, H, Wd)).astype(np.float32)
    w = W.Workload("large-2.7GB", vol, sp, K, poses, H, Wd, N, W.BEER_LAMBERT, grad_out=g)
    say(f"case: {shape} fp32 ({vol.nbytes / 2**30:.2f} GiB), 2 views {H}x{Wd}, N={N}, BL")
    vt = torch.from_numpy(vol).to(dev)
    pt = torch.from_numpy(poses).to(dev)
    img, s = drr.drr_forward(vt, sp, K, pt, H, Wd, N, W.BEER_LAMBERT)
    torch.cuda.synchronize()
    ref, _ = oracle.forward_workload(w)
    assert 0.3 < ref.max() < 0.99, "the image must not saturate"
    chords = oracle.chords_workload(w)
    assert (chords > 0).mean() > 0.9
    check_forward(img, ref, FWD_F32, "2.7 GB volume", chords)
    del vt
    torch.cuda.empty_cache()

    say("case: 2.7 GB volume, backward")
    grad = drr.drr_backward_volume(shape, sp, K, pt, H, Wd, N, W.BEER_LAMBERT,
                                   torch.from_numpy(g).to(dev), s)
    torch.cuda.synchronize()
    ref_g, used = oracle.adjoint_workload(w)
    gg = grad.cpu().numpy()
    del grad
    # the rays reach voxels above 2^31 bytes: the top slices have gradient
    top = np.abs(ref_g[600:]).max()
    assert top > 0.0
    err = normwise_err(gg, ref_g)
    say(f"2.7 GB volume: gradient normwise err {err:.3e} (oracle on {used} threads); "
        f"top-slices max {top:.3e}, GPU {np.abs(gg[600:]).max():.3e}")
    assert err <= GRAD
    untouched = ref_g == 0.0
    assert np.all(gg[untouched] == 0.0), "voxels no ray reaches must stay exactly 0"


@pytest.mark.timeout(900)
def test_volume_512_cubed_under_the_train_step_camera(dev):
    """512^3 fp32 (512 MiB) seen by the 1024^2 x 512-sample camera of the train
    step (20 degree vertical fov from 1000 mm): nearly every ray hits."""
    w3 = W.make_workload(3)
    shape = (512, 512, 512)
    rng = np.random.default_rng(502)
    vol = rng.random(shape, dtype=np.float32) * np.float32(0.004)   # s of 1 to 2
    w = W.Workload("train-camera-512", vol, w3.spacing, w3.K, w3.poses, w3.det_h, w3.det_w,
                   w3.n_samples, w3.mode, grad_out=w3.grad_out)
    say(f"case: 512^3 fp32, 1024x1024 x 512 samples, BL")
    vt = torch.from_numpy(vol).to(dev)
    pt = torch.from_numpy(w.poses).to(dev)
    img, s = drr.drr_forward(vt, w.spacing, w.K, pt, w.det_h, w.det_w, w.n_samples, w.mode)
    torch.cuda.synchronize()
    ref, _ = oracle.forward_workload(w)
    assert 0.3 < ref.max() < 0.99, "the image must not saturate"
    check_forward(img, ref, FWD_F32, "512^3", oracle.chords_workload(w))
    grad = drr.drr_backward_volume(shape, w.spacing, w.K, pt, w.det_h, w.det_w, w.n_samples,
                                   w.mode, torch.from_numpy(w.grad_out).to(dev), s)
    torch.cuda.synchronize()
    ref_g, used = oracle.adjoint_workload(w, max_buffer_bytes=16 << 30)
    err = normwise_err(grad.cpu().numpy(), ref_g)
    say(f"512^3: gradient normwise err {err:.3e} (oracle on {used} threads)")
    assert err <= GRAD
