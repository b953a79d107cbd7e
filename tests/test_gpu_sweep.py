"""Randomised GPU parity sweeps against the oracle, over configurations drawn
across the read plans and window tiers rather than hand-picked ones.

* ``drr_forward`` / ``drr_backward_volume`` / ``drr_backward_pose`` and the
  cell-constant pair (``drr_forward_siddon`` / ``drr_backward_volume_siddon``):
  ragged small launches (split lanes), dense single views (LDS-staged boxes,
  dense windows), many views (z-pairs, corner cells, mid windows) and sparse
  views of larger volumes (brick-owned backward); sources inside the volume;
  rotations up to 180 degrees; fp32 and bf16 volumes.
* ``drr_render`` and its volume and pose backward: volume and channel batches,
  density factor, Beer-Lambert, line integral and alpha compositing, box and
  near/far clip, per-channel transfer function, fp32 and bf16.

Bars are the parity bars used elsewhere (forward floored relative 1e-5, misses
exactly 0, gradients normwise 1e-4, pose gradients per view normwise 1e-4),
with the bf16 cases compared against the oracle on the bf16-rounded volume.
One reading is added for the transfer function: its extended end segments can
map voxels to negative mu, and a line integral whose terms cancel cannot be
held to a bar relative to its own (small) value in fp32, whose rounding scales
with the terms.  There the forward is measured against the oracle's line
integral of |mu| (the same render of the mapped volume's absolute values): the
optical depth's scale is that integral, floored at 1e-3 of its largest value,
and the image's the larger of its own floored value and dI/dtau (e^-tau for
Beer-Lambert, 1 otherwise) times the optical depth's scale.  With mu >= 0 the
reading changes nothing.

The library takes the density factor and the near/far margin as fp32 and the
oracle as fp64, so both are given fp32 values: a margin rounded differently
moves every sample of a near/far view by ~1e-7 voxel, enough to carry a sample
lying within that distance of a cell face to its other side, where the
trilinear gradient jumps.
"""
import numpy as np
import pytest
import torch

import ct_forward_projection_amd as drr
import oracle
import workloads as W
from helpers import forward_rel_err, normwise_err, say

pytestmark = pytest.mark.gpu

FWD, GRAD = 1e-5, 1e-4
CHUNK = 20


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _device_volume(vol, bf16, dev):
    """The volume as the library gets it and the fp32 values the oracle gets."""
    if bf16:
        bits = W.round_to_bf16_bits(vol)
        v = torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)
        return v, (bits.astype(np.uint32) << 16).view(np.float32).reshape(vol.shape)
    return torch.from_numpy(vol).to(dev), vol


def _normwise_or_abs(g, o):
    return normwise_err(g, o) if np.abs(o).max() > 0 else float(np.abs(g).max())


# ------------------------------------------------------------------ the drr_* calls

def draw_projector(seed):
    rng = np.random.default_rng(seed)
    kind = int(rng.integers(0, 4))
    if kind == 0:        # small ragged launches: split lanes, thin volumes, N = 1
        shape = tuple(int(x) for x in rng.integers(1, 40, size=3))
        det = tuple(int(x) for x in rng.integers(1, 90, size=2))
        views, N = int(rng.integers(1, 5)), int(rng.integers(1, 300))
    elif kind == 1:      # one dense view: LDS-staged boxes, dense windows
        shape = tuple(int(x) for x in rng.integers(8, 48, size=3))
        det = (int(rng.integers(256, 330)), int(rng.integers(256, 330)))
        views, N = 1, int(rng.integers(16, 160))
    elif kind == 2:      # many views: z-pairs or corner cells
        shape = tuple(int(x) for x in rng.integers(4, 40, size=3))
        det = tuple(int(x) for x in rng.integers(16, 80, size=2))
        views, N = int(rng.integers(4, 24)), int(rng.integers(32, 256))
    else:                # views sparse against a larger volume: brick-owned backward
        shape = tuple(int(x) for x in rng.integers(40, 80, size=3))
        det = tuple(int(x) for x in rng.integers(20, 64, size=2))
        views, N = int(rng.integers(2, 10)), int(rng.integers(8, 96))
    mode = int(rng.integers(0, 2))
    spacing = tuple(float(x) for x in rng.uniform(0.5, 2.0, size=3))
    ext = max(s * n for s, n in zip(spacing, shape[::-1]))
    inside = bool(rng.uniform() < 0.15)
    distance = float(rng.uniform(0.1, 0.4) * ext) if inside else float(rng.uniform(1.0, 4.0) * ext)
    rot = float(rng.choice([10.0, 45.0, 180.0]))
    bf16 = bool(rng.uniform() < 0.25)
    w = W.make_random_small(seed, shape=shape, n_views=views, det=det, n_samples=N, mode=mode,
                            spacing=spacing, distance=distance, rot_deg=rot)
    return w, bf16, dict(kind=kind, shape=shape, det=det, views=views, N=N, mode=mode,
                         inside=inside, rot=rot, bf16=bf16)


def projector_case(dev, seed):
    w, bf16, info = draw_projector(seed)
    say(f"case: projector sweep seed={seed} {info}")
    vol, vref = _device_volume(w.volume, bf16, dev)
    P = torch.from_numpy(w.poses).to(dev)
    g = torch.from_numpy(w.grad_out).to(dev)
    args = (w.spacing, w.K, P, w.det_h, w.det_w)
    img, s = drr.drr_forward(vol, *args, w.n_samples, w.mode)
    grad = drr.drr_backward_volume(w.volume.shape, *args, w.n_samples, w.mode, g, s)
    pose = drr.drr_backward_pose(vol, *args, w.n_samples, w.mode, g)
    simg, ss = drr.drr_forward_siddon(vol, *args, w.mode)
    sgrad = drr.drr_backward_volume_siddon(w.volume.shape, *args, w.mode, g, ss)
    torch.cuda.synchronize()
    oargs = (w.spacing, w.K, w.poses, w.det_h, w.det_w)
    ref, _ = oracle.forward(vref, *oargs, w.n_samples, w.mode)
    ref_g, _ = oracle.adjoint(vref, w.volume.shape, *oargs, w.n_samples, w.mode, w.grad_out)
    ref_p = oracle.pose_gradient(vref, *oargs, w.n_samples, w.mode, w.grad_out)
    sref, _ = oracle.siddon_forward(vref, *oargs, w.mode)
    sref_g, _ = oracle.siddon_adjoint(vref, w.volume.shape, *oargs, w.mode, w.grad_out)
    chord = oracle.chords_workload(w)
    im = img.cpu().double().numpy()
    pn = pose.cpu().double().numpy()
    e = dict(fwd=forward_rel_err(im, ref),
             grad=_normwise_or_abs(grad.cpu().double().numpy(), ref_g),
             pose=max(_normwise_or_abs(pn[v], ref_p[v]) for v in range(w.n_views)),
             siddon_fwd=forward_rel_err(simg.cpu().double().numpy(), sref),
             siddon_grad=_normwise_or_abs(sgrad.cpu().double().numpy(), sref_g))
    say(f"projector sweep {seed}: " + ", ".join(f"{k} {v:.2e}" for k, v in e.items()))
    assert np.all(im[chord == 0.0] == 0.0), "misses must be exactly 0"
    assert e["fwd"] <= FWD and e["siddon_fwd"] <= FWD
    assert e["grad"] <= GRAD and e["pose"] <= GRAD and e["siddon_grad"] <= GRAD


@pytest.mark.parametrize("start", range(1000, 1100, CHUNK))
def test_projector_random_sweep(dev, start):
    for seed in range(start, start + CHUNK):
        projector_case(dev, seed)


# ------------------------------------------------------------------ the front end

KNOTS_X = np.array([[-1000.0, 0.0, 1500.0], [-600.0, 100.0, 1200.0], [-900.0, -100.0, 800.0]],
                   dtype=np.float32)
KNOTS_Y = np.array([[0.0, 0.02, 0.05], [0.005, 0.0, 0.04], [0.0, 0.03, 0.01]], dtype=np.float32)


def draw_render(seed):
    rng = np.random.default_rng(seed)
    dense = bool(rng.uniform() < 0.25)
    B, C, vpv = int(rng.integers(1, 3)), int(rng.integers(1, 4)), int(rng.integers(1, 4))
    if dense:            # one dense view per volume: staged boxes or corner cells
        B, C, vpv = 1, int(rng.integers(1, 3)), 1
        shape = tuple(int(x) for x in rng.integers(8, 40, size=3))
        det = (int(rng.integers(256, 300)), int(rng.integers(256, 300)))
        N = int(rng.integers(16, 120))
    else:
        shape = tuple(int(x) for x in rng.integers(1, 36, size=3))
        det = tuple(int(x) for x in rng.integers(1, 70, size=2))
        N = int(rng.integers(1, 200))
    mode, clip = int(rng.integers(0, 3)), int(rng.integers(0, 2))
    tf, bf16 = bool(rng.uniform() < 0.5), bool(rng.uniform() < 0.25)
    if tf:
        vol = rng.uniform(-1100.0, 1600.0, size=(B, C) + shape).astype(np.float32)
    else:
        vol = rng.uniform(0.05, 1.0, size=(B, C) + shape).astype(np.float32)
    spacing = rng.uniform(0.5, 2.0, size=3).astype(np.float32)
    H, Wd = det
    ext = max(shape[2] * spacing[0], shape[1] * spacing[1], shape[0] * spacing[2])
    inside = bool(rng.uniform() < 0.1)
    dist = float(rng.uniform(0.1, 0.4) * ext) if inside else float(rng.uniform(1.2, 4.0) * ext)
    K = W.intrinsics(1.2 * max(H, Wd) * dist / ext, Wd / 2.0 + 0.3, H / 2.0 - 0.2)
    poses = W.random_poses(B * vpv, dist, float(rng.choice([10.0, 40.0, 180.0])), 0.05 * ext,
                           seed=seed + 7)
    g = rng.uniform(-1.0, 1.0, size=(B * vpv, C, H, Wd)).astype(np.float32)
    # fp32 values, as the library takes them (the oracle takes fp64)
    f = float(np.float32(float(rng.uniform(0.3, 2.0)) * (40.0 if tf else 1.0)))
    margin = float(np.float32(rng.uniform(0.0, 10.0)))
    transfer = (KNOTS_X[:C], KNOTS_Y[:C]) if tf else None
    info = dict(dense=dense, B=B, C=C, vpv=vpv, shape=shape, det=det, N=N, mode=mode, clip=clip,
                tf=tf, bf16=bf16, inside=inside)
    return vol, spacing, K, poses, H, Wd, N, g, mode, clip, transfer, f, margin, bf16, info


def render_case(dev, seed):
    (vol, spacing, K, poses, H, Wd, N, g, mode, clip, transfer, f, margin, bf16,
     info) = draw_render(seed)
    say(f"case: render sweep seed={seed} {info}")
    v, vref = _device_volume(vol, bf16, dev)
    P = torch.from_numpy(poses).to(dev)
    gt = torch.from_numpy(g).to(dev)
    img, tau = drr.drr_render(v, spacing, K, P, H, Wd, N, mode, f, clip, margin, transfer)
    grad = drr.drr_render_backward_volume(v, tuple(vol.shape), 0, spacing, K, P, H, Wd, N, mode,
                                          gt, img, tau, f, clip, margin, transfer)
    pose = drr.drr_render_backward_pose(v, spacing, K, P, H, Wd, N, mode, gt, f, clip, margin,
                                        transfer)
    torch.cuda.synchronize()
    kw = dict(density_factor=f, clip=clip, margin=margin, transfer=transfer)
    ref, ref_tau = oracle.render(vref, spacing, K, poses, H, Wd, N, mode, **kw)
    ref_g = oracle.render_adjoint(vref, spacing, K, poses, H, Wd, N, mode, g, **kw)
    ref_p = oracle.render_pose_gradient(vref, spacing, K, poses, H, Wd, N, mode, g, **kw)
    im, ta = img.cpu().double().numpy(), tau.cpu().double().numpy()
    pn = pose.cpu().double().numpy()
    img_scale = np.maximum(np.abs(ref), 1e-3 * np.abs(ref).max())
    tau_scale = np.maximum(np.abs(ref_tau), 1e-3 * np.abs(ref_tau).max())
    if transfer is not None:
        # the line integral of |mu| (see the module docstring)
        mapped = np.stack([np.stack([W.piecewise_linear(vref[b, c].astype(np.float64),
                                                        transfer[0][c], transfer[1][c])
                                     for c in range(vol.shape[1])])
                           for b in range(vol.shape[0])])
        _, tau_abs = oracle.render(np.abs(mapped).astype(np.float32), spacing, K, poses, H, Wd,
                                   N, drr.LINE_INTEGRAL, density_factor=f, clip=clip,
                                   margin=margin)
        fl = np.maximum(tau_abs, 1e-3 * tau_abs.max())
        tau_scale = np.maximum(tau_scale, fl)
        if mode != drr.ALPHA_COMPOSITE:
            dI = np.exp(-ref_tau) if mode == drr.BEER_LAMBERT else 1.0
            img_scale = np.maximum(img_scale, dI * fl)
    e = dict(img=float((np.abs(im - ref) / img_scale).max()),
             tau=float((np.abs(ta - ref_tau) / tau_scale).max()),
             grad=_normwise_or_abs(grad.cpu().double().numpy(), ref_g),
             pose=max(_normwise_or_abs(pn[i], ref_p[i]) for i in range(ref_p.shape[0])))
    say(f"render sweep {seed}: " + ", ".join(f"{k} {x:.2e}" for k, x in e.items()))
    assert np.all(im[ref == 0.0] == 0.0), "nothing rendered where the oracle has 0"
    assert e["img"] <= FWD and e["tau"] <= FWD
    assert e["grad"] <= GRAD and e["pose"] <= GRAD


@pytest.mark.parametrize("start", range(2000, 2100, CHUNK))
def test_render_random_sweep(dev, start):
    for seed in range(start, start + CHUNK):
        render_case(dev, seed)


def test_compositing_late_samples_keep_their_weight(dev):
    """Regression: compositing's window took its fixed-point unit from the
    tile's coefficient bound alone, so the small coefficients of samples late on
    a ray (little transmittance and emission left) rounded to zero window units,
    a loss that built up on the voxels where the rays leave the volume (this
    draw: 2.4e-4 normwise on the far edge of its second volume, with views of
    4 to 16 samples per cell).  Each chunk now takes its unit from a bound on
    its own samples."""
    render_case(dev, 20806)
