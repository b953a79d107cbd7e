"""drr_forward_no_alloc (the forward for callers that cannot allocate) against
drr_forward through the C ABI: the same launches with the read copy in the
library's fixed device scratch instead of a caller workspace.  Consecutive
calls share that scratch, so the second call of each pair is smaller than the
first and must not see the first one's contents.  Bars: equal to drr_forward
bit for bit (same kernels, same inputs), and within the forward's parity bar
(1e-5 floored relative error) of the CPU oracle."""
import numpy as np
import pytest
import torch

import ct_forward_projection_amd as drr
import oracle
import workloads as W
from helpers import check_forward, say

pytestmark = pytest.mark.gpu

FWD_F32 = 1e-5


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _vol(w, dev, bf16):
    if bf16:
        return torch.from_numpy(w.volume_bf16.view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(w.volume).to(dev)


def _case(seed, shape, views, det, n, mode, bf16, dev):
    w = W.make_random_small(seed, shape=shape, n_views=views, det=det, n_samples=n, mode=mode)
    if bf16:
        w.volume_bf16 = W.round_to_bf16_bits(w.volume)
    nz, ny, nx = shape
    need = drr.drr_workspace_bytes(nz, ny, nx, drr.BF16 if bf16 else drr.F32, views, det[0],
                                   det[1], n, 0)
    say(f"case: no-alloc forward seed={seed} shape={shape} views={views} det={det} N={n} "
        f"bf16={bf16} (plan workspace {need} bytes)")
    assert 0 < need <= drr.NO_ALLOC_SCRATCH_BYTES   # the scratch is really used
    vol = _vol(w, dev, bf16)
    poses = torch.from_numpy(w.poses).to(dev)
    img_na, s_na = drr.drr_forward_no_alloc(vol, w.spacing, w.K, poses, det[0], det[1], n, mode)
    torch.cuda.synchronize()
    img, s = drr.drr_forward(vol, w.spacing, w.K, poses, det[0], det[1], n, mode)
    torch.cuda.synchronize()
    assert torch.equal(img_na, img), "image differs from drr_forward"
    assert torch.equal(s_na, s), "line integral differs from drr_forward"
    ref, _ = oracle.forward_workload(w, use_bf16=bf16)
    check_forward(img_na, ref, FWD_F32, f"no-alloc seed {seed}", oracle.chords_workload(w))
    return img_na


def test_no_alloc_forward_matches_drr_forward_on_consecutive_calls(dev):
    # z-pair plan (4 to 16 samples per cell), then a smaller z-pair plan in bf16
    _case(401, (64, 64, 64), 4, (64, 64), 128, W.BEER_LAMBERT, False, dev)
    _case(402, (36, 40, 44), 3, (48, 48), 96, W.LINE_INTEGRAL, True, dev)


def test_no_alloc_forward_corner_cells_then_smaller(dev):
    # corner-cell plan (16 or more samples per cell), then a smaller one
    _case(403, (32, 30, 34), 8, (64, 64), 64, W.BEER_LAMBERT, False, dev)
    _case(404, (20, 22, 18), 6, (40, 36), 48, W.LINE_INTEGRAL, False, dev)


def test_no_alloc_forward_rejects_a_plan_beyond_the_scratch(dev):
    vol = torch.zeros((512, 512, 512), device=dev)
    poses = torch.from_numpy(W.random_poses(64, 1200.0, 20.0, 5.0, seed=405)).to(dev)
    K = W.intrinsics(1000.0, 128.0, 128.0)
    with pytest.raises(drr.DRRError) as e:
        drr.drr_forward_no_alloc(vol, [1, 1, 1], K, poses, 256, 256, 256)
    assert e.value.status == 2 and "scratch" in str(e.value)
