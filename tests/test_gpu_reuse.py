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


# drr_render / drr_render_backward_pose: 2 volumes x 2 channels from HU-like
# values through the transfer function (the copy holds the mapped values), the
# box clip (mapped z-pairs) and the near/far range (zero-padded copies)
KNOTS = (np.array([[-1000.0, 0.0, 1500.0], [-600.0, 100.0, 1200.0]], dtype=np.float32),
         np.array([[0.0, 0.02, 0.05], [0.005, 0.0, 0.04]], dtype=np.float32))


@pytest.mark.parametrize("clip,mode", [(drr.CLIP_BOX, drr.BEER_LAMBERT),
                                       (drr.CLIP_NEAR_FAR, drr.ALPHA_COMPOSITE)])
def test_reused_render_copy(dev, clip, mode):
    rng = np.random.default_rng(510 + clip)
    shape, det, N, f, margin = (30, 26, 34), (40, 44), 48, 30.0, 3.0
    vol = rng.uniform(-1100.0, 1600.0, size=(2, 2) + shape).astype(np.float32)
    spacing = np.array([1.0, 1.25, 0.8], dtype=np.float32)
    K = W.intrinsics(1.2 * 44 * 60.0 / 34.0, 22.3, 19.8)
    P1 = W.random_poses(6, 60.0, 30.0, 1.5, seed=511)
    P2 = W.random_poses(6, 60.0, 30.0, 1.5, seed=512)
    g = rng.uniform(-1.0, 1.0, size=(6, 2) + det).astype(np.float32)
    v = torch.from_numpy(vol).to(dev)
    gt = torch.from_numpy(g).to(dev)
    need = drr.drr_render_workspace_bytes(2, 2, *shape, drr.F32, 6, det[0], det[1], N, mode,
                                          clip, 3, 0)
    need_p = drr.drr_render_workspace_bytes(2, 2, *shape, drr.F32, 6, det[0], det[1], N, mode,
                                            clip, 3, 2)
    say(f"case: reuse render clip={clip} mode={mode} (copy {need} bytes, pose workspace {need_p})")
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_p = torch.empty(need_p, dtype=torch.uint8, device=dev)
    kw = dict(density_factor=f, clip=clip, margin=margin, transfer=KNOTS)
    args = (v, spacing, K)
    p1, p2 = torch.from_numpy(P1).to(dev), torch.from_numpy(P2).to(dev)
    drr.drr_render(*args, p1, det[0], det[1], N, mode, workspace=ws, **kw)
    img_r, tau_r = drr.drr_render(*args, p2, det[0], det[1], N, mode, workspace=ws,
                                  reuse_copy=True, **kw)
    img_f, tau_f = drr.drr_render(*args, p2, det[0], det[1], N, mode, **kw)
    drr.drr_render_backward_pose(*args, p1, det[0], det[1], N, mode, gt, workspace=ws_p, **kw)
    gp_r = drr.drr_render_backward_pose(*args, p2, det[0], det[1], N, mode, gt, workspace=ws_p,
                                        reuse_copy=True, **kw)
    gp_f = drr.drr_render_backward_pose(*args, p2, det[0], det[1], N, mode, gt, **kw)
    torch.cuda.synchronize()
    assert torch.equal(img_r, img_f) and torch.equal(tau_r, tau_f), "reuse differs from a fresh call"
    ref, _ = oracle.render(vol, spacing, K, P2, det[0], det[1], N, mode, **kw)
    check_forward(img_r, ref, FWD, f"reuse render c{clip} m{mode}")
    a, b = gp_r.cpu().double().numpy(), gp_f.cpu().double().numpy()
    ref_p = oracle.render_pose_gradient(vol, spacing, K, P2, det[0], det[1], N, mode, g, **kw)
    worst = max(normwise_err(a[i], ref_p[i]) for i in range(6))
    say(f"reuse render pose c{clip} m{mode}: normwise err {worst:.3e} (bar {GRAD:g})")
    for i in range(6):
        assert normwise_err(a[i], b[i]) <= 1e-6, "reuse differs from a fresh call"
    assert worst <= GRAD
