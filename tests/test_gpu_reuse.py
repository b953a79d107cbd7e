"""drr_forward_reuse and drr_backward_pose_reuse through the C ABI: calls that
read the volume copy an earlier call left in the caller's workspace instead of
making it again (a registration loop over a fixed volume).  The copy depends on
the volume and the launch shape only, so a reusing call with other poses must
equal a fresh call with those poses: bit for bit for the forward (same
kernels, same inputs), within the pose gradient's fp64 view sums otherwise, and
both within the parity bars of the oracle."""
import numpy as np
import pytest
import torch

import ct_forward_projection_amd as drr
import oracle
import workloads as W
from helpers import check_forward, normwise_err, say

pytestmark = pytest.mark.gpu

FWD, GRAD = 1e-5, 1e-4


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


# (seed, shape, views, detector, samples, bf16): the z-pair copy (4 to 16
# samples per cell), the corner-cell copy (16 or more) in fp32 and bf16, and a
# staged launch (no copy: the reusing call is the plain one)
CASES = [
    (501, (48, 40, 44), 4, (48, 56), 64, False),
    (502, (48, 40, 44), 4, (48, 56), 64, True),
    (503, (20, 22, 18), 8, (40, 36), 80, False),
    (504, (20, 22, 18), 8, (40, 36), 80, True),
    (505, (24, 24, 24), 1, (272, 264), 64, False),
]


def _plan(shape, views, det, n, bf16, kind):
    nz, ny, nx = shape
    return drr.drr_workspace_bytes(nz, ny, nx, drr.BF16 if bf16 else drr.F32, views, det[0],
                                   det[1], n, kind)


def test_cases_cover_each_read_plan():
    kinds = []
    for _, (nz, ny, nx), views, det, n, bf16 in CASES:
        eb = 2 if bf16 else 4
        need = _plan((nz, ny, nx), views, det, n, bf16, 0)
        zpair = (nx * ny * (nz - 1) * 2 * eb + 255) // 256 * 256
        cells = ((nx + 1) * (ny + 1) * (nz + 1) * 8 * eb + 255) // 256 * 256
        kinds.append({zpair: "z-pairs", cells: "cells", 0: "staged"}.get(need, "?"))
    assert kinds == ["z-pairs", "z-pairs", "cells", "cells", "staged"], kinds


@pytest.mark.parametrize("seed,shape,views,det,n,bf16", CASES)
def test_reused_copy_renders_new_poses(dev, seed, shape, views, det, n, bf16):
    w = W.make_random_small(seed, shape=shape, n_views=views, det=det, n_samples=n)
    w2 = W.make_random_small(seed + 50, shape=shape, n_views=views, det=det, n_samples=n)
    if bf16:
        w2.volume_bf16 = W.round_to_bf16_bits(w.volume)
        vol = torch.from_numpy(w2.volume_bf16.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        vol = torch.from_numpy(w.volume).to(dev)
    w2.volume = w.volume                       # one volume, two sets of poses
    need = _plan(shape, views, det, n, bf16, 0)
    say(f"case: reuse forward seed={seed} shape={shape} views={views} det={det} N={n} "
        f"bf16={bf16} (copy {need} bytes)")
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    P1 = torch.from_numpy(w.poses).to(dev)
    P2 = torch.from_numpy(w2.poses).to(dev)
    args = (w.spacing, w.K)
    drr.drr_forward(vol, *args, P1, det[0], det[1], n, w.mode, workspace=ws)
    img_r, s_r = drr.drr_forward(vol, *args, P2, det[0], det[1], n, w.mode, workspace=ws,
                                 reuse_copy=True)
    img_f, s_f = drr.drr_forward(vol, *args, P2, det[0], det[1], n, w.mode)
    torch.cuda.synchronize()
    assert torch.equal(img_r, img_f) and torch.equal(s_r, s_f), "reuse differs from a fresh call"
    ref, _ = oracle.forward_workload(w2, use_bf16=bf16)
    check_forward(img_r, ref, FWD, f"reuse forward {seed}", oracle.chords_workload(w2))


@pytest.mark.parametrize("seed,shape,views,det,n,bf16", CASES)
def test_reused_copy_pose_gradient(dev, seed, shape, views, det, n, bf16):
    w = W.make_random_small(seed, shape=shape, n_views=views, det=det, n_samples=n)
    w2 = W.make_random_small(seed + 50, shape=shape, n_views=views, det=det, n_samples=n)
    if bf16:
        bits = W.round_to_bf16_bits(w.volume)
        vol = torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)
        vref = (bits.astype(np.uint32) << 16).view(np.float32).reshape(w.volume.shape)
    else:
        vol = torch.from_numpy(w.volume).to(dev)
        vref = w.volume
    need = _plan(shape, views, det, n, bf16, 2)
    say(f"case: reuse pose gradient seed={seed} shape={shape} views={views} det={det} N={n} "
        f"bf16={bf16} (workspace {need} bytes)")
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    P1 = torch.from_numpy(w.poses).to(dev)
    P2 = torch.from_numpy(w2.poses).to(dev)
    g1 = torch.from_numpy(w.grad_out).to(dev)
    g2 = torch.from_numpy(w2.grad_out).to(dev)
    args = (w.spacing, w.K)
    drr.drr_backward_pose(vol, *args, P1, det[0], det[1], n, w.mode, g1, workspace=ws)
    gp_r = drr.drr_backward_pose(vol, *args, P2, det[0], det[1], n, w.mode, g2, workspace=ws,
                                 reuse_copy=True)
    gp_f = drr.drr_backward_pose(vol, *args, P2, det[0], det[1], n, w.mode, g2)
    torch.cuda.synchronize()
    a, b = gp_r.cpu().double().numpy(), gp_f.cpu().double().numpy()
    for v in range(views):
        assert normwise_err(a[v], b[v]) <= 1e-6, "reuse differs from a fresh call"
    ref = oracle.pose_gradient(vref, w.spacing, w.K, w2.poses, det[0], det[1], n, w.mode,
                               w2.grad_out)
    worst = max(normwise_err(a[v], ref[v]) for v in range(views))
    say(f"reuse pose {seed}: normwise err {worst:.3e} (bar {GRAD:g})")
    assert worst <= GRAD


def test_reuse_without_a_workspace_is_refused(dev):
    w = W.make_random_small(506, shape=(20, 22, 18), n_views=8, det=(40, 36), n_samples=80)
    vol = torch.from_numpy(w.volume).to(dev)
    P = torch.from_numpy(w.poses).to(dev)
    with pytest.raises(ValueError):
        drr.drr_forward(vol, w.spacing, w.K, P, 40, 36, 80, reuse_copy=True)
    with pytest.raises(ValueError):
        drr.drr_backward_pose(vol, w.spacing, w.K, P, 40, 36, 80, w.mode,
                              torch.zeros((8, 40, 36), device=dev), reuse_copy=True)
