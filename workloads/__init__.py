"""Seeded synthetic inputs for the cone-beam DRR workloads.

This module only *produces inputs* (volumes, voxel spacing, intrinsics K,
per-view world-to-camera poses, upstream gradients).  It holds none of the
ray-casting arithmetic: no ray generation, clipping, sampling, interpolation or
integration happens here, so both the CPU oracle and the HIP library can consume
its arrays without sharing any of the method's code.

Conventions (the plain reading of the pages where they are silent):

* Volume ``vol[k, j, i]`` has shape ``(nz, ny, nx)`` with x fastest; units are
  mm for geometry and 1/mm for attenuation mu.  The volume box is centred at the
  world origin.
* Intrinsics follow the Hartley-Zisserman pinhole model named on the nanodrr
  page (x right, y down, z forward): ``K = [[f, 0, cx], [0, f, cy], [0, 0, 1]]``
  with ``f = source-to-detector distance / detector pitch`` in pixels.
* A pose is the world-to-camera ``[R | t]`` (3x4, row-major): a world point
  ``X`` maps to ``R @ X + t`` and the camera (X-ray source) centre is
  ``-R.T @ t``.

Workloads (sizes as listed for each configuration):

1. tiny DRR forward: 64^3, centred sphere r=20 mm mu=0.02/mm plus U[0, 0.005)
   noise, one view, source 500 mm from isocentre, sdd 1000 mm, 64x64 detector
   at 2 mm pitch, 128 samples, Beer-Lambert.
2. nanodrr-style batch: 256^3 ellipsoid HU phantom mapped to mu by a
   piecewise-linear transfer function (flashdrr ``piecewise_linear_channelwise``
   semantics: end segments extended); 16 views with rotations U[-30, 30] deg per
   axis and translations N(0, 10 mm); 200x200 at 2 mm pitch, sdd 1020 mm,
   256 samples, Beer-Lambert; fp32 and bf16 copies of the volume.
3. FlashDRR train step: the workload-2 phantom, one view, 20 deg vertical
   field of view, 1024x1024, 512 samples, Beer-Lambert forward and volume
   backward with dL/dI ~ U[-1, 1].
4. high-resolution eval: as 3 with 2048x2048 and 256 samples, forward only.
5. cone-beam CT projector: 128^3 U[0, 1) volume, 360-view helical orbit
   (sid 320 mm, sdd 512 mm, 40 mm z range, one turn; the diffct quickstart),
   flat 384x256 detector at 0.8 mm pitch, raw line integrals, and the matched
   backward of a U[0, 1) sinogram.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

BEER_LAMBERT = 0
LINE_INTEGRAL = 1

VOLUME_SEED_BASE = 1000
GEOMETRY_SEED_BASE = 2000


@dataclass
class Workload:
    """One synthetic workload: every array the forward/backward consume."""

    name: str
    volume: np.ndarray                 # (nz, ny, nx) float32, C-contiguous
    spacing: np.ndarray                # (3,) float32: sx, sy, sz in mm
    K: np.ndarray                      # (3, 3) float32
    poses: np.ndarray                  # (V, 3, 4) float32 world->camera [R|t]
    det_h: int
    det_w: int
    n_samples: int
    mode: int                          # BEER_LAMBERT or LINE_INTEGRAL
    grad_out: Optional[np.ndarray] = None   # (V, H, W) float32 upstream dL/dI
    volume_bf16: Optional[np.ndarray] = None  # (nz, ny, nx) uint16 bf16 bit patterns
    notes: dict = field(default_factory=dict)

    @property
    def n_views(self) -> int:
        return int(self.poses.shape[0])

    @property
    def shape(self):
        return tuple(int(s) for s in self.volume.shape)

    @property
    def n_rays(self) -> int:
        return self.n_views * self.det_h * self.det_w

    @property
    def nominal_samples(self) -> int:
        return self.n_rays * self.n_samples

    def volume_bf16_as_f32(self) -> np.ndarray:
        """The bf16 volume widened exactly to float32 (bf16 is the top half of fp32)."""
        assert self.volume_bf16 is not None
        return (self.volume_bf16.astype(np.uint32) << np.uint32(16)).view(np.float32)

    def subset_views(self, idx) -> "Workload":
        """Same workload restricted to the views ``idx`` (for sampled comparisons)."""
        idx = np.asarray(idx)
        return Workload(
            name=f"{self.name}[views]", volume=self.volume, spacing=self.spacing, K=self.K,
            poses=np.ascontiguousarray(self.poses[idx]), det_h=self.det_h, det_w=self.det_w,
            n_samples=self.n_samples, mode=self.mode,
            grad_out=None if self.grad_out is None else np.ascontiguousarray(self.grad_out[idx]),
            volume_bf16=self.volume_bf16, notes=dict(self.notes))


# --------------------------------------------------------------------------- helpers

def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns with round-to-nearest-even (what torch's
    ``.to(torch.bfloat16)`` does).  Inputs here are finite."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    rounded = (bits + np.uint64(0x7FFF) + ((bits >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return rounded.astype(np.uint16)


def intrinsics(f: float, cx: float, cy: float) -> np.ndarray:
    return np.array([[f, 0.0, cx], [0.0, f, cy], [0.0, 0.0, 1.0]], dtype=np.float32)


def pose_from_rotation_and_centre(R: np.ndarray, C: np.ndarray) -> np.ndarray:
    """World-to-camera [R | t] with t = -R C (camera centre C)."""
    R = np.asarray(R, dtype=np.float64)
    C = np.asarray(C, dtype=np.float64)
    P = np.zeros((3, 4), dtype=np.float64)
    P[:, :3] = R
    P[:, 3] = -R @ C
    return P.astype(np.float32)


def _rot_x(a):
    c, s = math.cos(a), math.sin(a)
    return np.array([[1, 0, 0], [0, c, -s], [0, s, c]], dtype=np.float64)


def _rot_y(a):
    c, s = math.cos(a), math.sin(a)
    return np.array([[c, 0, s], [0, 1, 0], [-s, 0, c]], dtype=np.float64)


def _rot_z(a):
    c, s = math.cos(a), math.sin(a)
    return np.array([[c, -s, 0], [s, c, 0], [0, 0, 1]], dtype=np.float64)


def voxel_centres(n: int, s: float) -> np.ndarray:
    """World coordinates (mm) of the voxel centres along one axis of a box
    centred at the origin."""
    return (np.arange(n, dtype=np.float64) + 0.5) * s - 0.5 * n * s


def piecewise_linear(x: np.ndarray, xp, yp) -> np.ndarray:
    """Piecewise-linear transfer with the first and last segments extended
    (flashdrr ``piecewise_linear_channelwise``, one channel).  Builds input
    volumes, and in the GPU sweep the mapped values whose absolute line integral
    scales the forward bar where mapped values of both signs cancel."""
    xp = np.asarray(xp, dtype=np.float64)
    yp = np.asarray(yp, dtype=np.float64)
    seg = np.clip(np.searchsorted(xp, x, side="right") - 1, 0, len(xp) - 2)
    x0, x1 = xp[seg], xp[seg + 1]
    y0, y1 = yp[seg], yp[seg + 1]
    return y0 + (x - x0) * (y1 - y0) / (x1 - x0)


# Transfer-function knots: HU -> mu (1/mm), water = 0.02/mm (the sphere value of
# the tiny workload), air = 0; a straight line mu = 0.02 (1 + HU / 1000).
HU_KNOTS = (-1000.0, 0.0, 1500.0)
MU_KNOTS = (0.0, 0.02, 0.05)


def hu_phantom(n: int = 256, spacing: float = 1.0, seed: int = VOLUME_SEED_BASE + 2) -> np.ndarray:
    """Nested-ellipsoid HU phantom: air -1000, soft tissue 40 +- 20 HU, bone
    700-1500 HU.  Inside tests use voxel centres; later ellipsoids overwrite
    earlier ones.  Returns float64 HU of shape (n, n, n)."""
    rng = np.random.default_rng(seed)
    c = voxel_centres(n, spacing)
    z, y, x = np.meshgrid(c, c, c, indexing="ij")
    hu = np.full((n, n, n), -1000.0, dtype=np.float64)

    def inside(centre, semi):
        cx, cy, cz = centre
        ax, ay, az = semi
        return ((x - cx) / ax) ** 2 + ((y - cy) / ay) ** 2 + ((z - cz) / az) ** 2 <= 1.0

    body = inside((0.0, 0.0, 0.0), (110.0, 85.0, 120.0))
    tissue = 40.0 + 20.0 * rng.standard_normal(size=hu.shape)
    hu[body] = tissue[body]
    # spine: cortex then marrow
    hu[inside((0.0, 45.0, 0.0), (16.0, 16.0, 115.0))] = rng.uniform(1200.0, 1500.0)
    hu[inside((0.0, 45.0, 0.0), (9.0, 9.0, 110.0))] = rng.uniform(700.0, 900.0)
    # two lateral bones and a sternum
    hu[inside((60.0, 0.0, -40.0), (20.0, 30.0, 25.0))] = rng.uniform(700.0, 1500.0)
    hu[inside((-60.0, 0.0, -40.0), (20.0, 30.0, 25.0))] = rng.uniform(700.0, 1500.0)
    hu[inside((0.0, -65.0, 20.0), (10.0, 6.0, 50.0))] = rng.uniform(700.0, 1500.0)
    return hu


_PHANTOM_CACHE: dict = {}


def mu_phantom(n: int = 256) -> np.ndarray:
    """The HU phantom converted voxelwise (fp64) to mu and cast to float32."""
    key = n
    if key not in _PHANTOM_CACHE:
        hu = hu_phantom(n)
        mu = piecewise_linear(hu, HU_KNOTS, MU_KNOTS)
        _PHANTOM_CACHE[key] = np.ascontiguousarray(mu.astype(np.float32))
    return _PHANTOM_CACHE[key]


def sphere_volume(n: int = 64, radius: float = 20.0, mu: float = 0.02, noise: float = 0.005,
                  seed: int = VOLUME_SEED_BASE + 1) -> np.ndarray:
    """Centred uniform sphere (voxel-centre inside test) plus U[0, noise) on every voxel."""
    c = voxel_centres(n, 1.0)
    z, y, x = np.meshgrid(c, c, c, indexing="ij")
    vol = np.where(x * x + y * y + z * z <= radius * radius, mu, 0.0)
    if noise > 0.0:
        rng = np.random.default_rng(seed)
        vol = vol + rng.uniform(0.0, noise, size=vol.shape)
    return np.ascontiguousarray(vol.astype(np.float32))


def helical_poses(n_views: int = 360, sid: float = 320.0, z_range: float = 40.0,
                  n_turns: float = 1.0) -> np.ndarray:
    """Helical source orbit around the z axis.  Angles cover [0, 2 pi n_turns)
    half-open; the source climbs linearly through z_range centred on z = 0.  The
    camera looks from the source towards the axis, image x along the tangent,
    image y along -z (rows grow downwards)."""
    poses = np.zeros((n_views, 3, 4), dtype=np.float32)
    for k in range(n_views):
        th = 2.0 * math.pi * n_turns * k / n_views
        c, s = math.cos(th), math.sin(th)
        src = np.array([sid * c, sid * s, z_range * (k / n_views - 0.5)])
        R = np.array([[-s, c, 0.0], [0.0, 0.0, -1.0], [-c, -s, 0.0]])
        poses[k] = pose_from_rotation_and_centre(R, src)
    return poses


def random_poses(n_views: int, distance: float, rot_deg: float, trans_sigma: float,
                 seed: int) -> np.ndarray:
    """Camera-to-world rotation Rz(g) Ry(b) Rx(a) with a, b, g ~ U[-rot, rot] deg;
    camera centre at R_c (0, 0, -distance) + N(0, sigma^2 I)."""
    rng = np.random.default_rng(seed)
    poses = np.zeros((n_views, 3, 4), dtype=np.float32)
    for v in range(n_views):
        a, b, g = np.deg2rad(rng.uniform(-rot_deg, rot_deg, size=3))
        Rc = _rot_z(g) @ _rot_y(b) @ _rot_x(a)
        C = Rc @ np.array([0.0, 0.0, -distance]) + rng.normal(0.0, trans_sigma, size=3)
        poses[v] = pose_from_rotation_and_centre(Rc.T, C)
    return poses


# --------------------------------------------------------------------------- workloads

WORKLOAD_NAMES = {
    1: "tiny-64^3-64x64-128spp-BL",
    2: "nanodrr-batch-256^3-16x200x200-256spp-BL",
    3: "flashdrr-train-256^3-1024x1024-512spp-BL-fwd+bwd",
    4: "hires-eval-256^3-2048x2048-256spp-BL",
    5: "cbct-helix-128^3-360x256x384-256spp-RAW-fwd+bwd",
}


def make_workload(i: int, with_bf16: bool = False) -> Workload:
    """Build workload ``i`` (1..5) deterministically from its seeds."""
    geo_rng = np.random.default_rng(GEOMETRY_SEED_BASE + i)
    sp = np.array([1.0, 1.0, 1.0], dtype=np.float32)
    if i == 1:
        vol = sphere_volume()
        K = intrinsics(1000.0 / 2.0, 32.0, 32.0)
        poses = pose_from_rotation_and_centre(np.eye(3), [0.0, 0.0, -500.0])[None]
        w = Workload(WORKLOAD_NAMES[1], vol, sp, K, poses, 64, 64, 128, BEER_LAMBERT)
    elif i == 2:
        vol = mu_phantom(256)
        K = intrinsics(1020.0 / 2.0, 100.0, 100.0)
        poses = random_poses(16, 510.0, 30.0, 10.0, seed=GEOMETRY_SEED_BASE + i)
        w = Workload(WORKLOAD_NAMES[2], vol, sp, K, poses, 200, 200, 256, BEER_LAMBERT)
    elif i in (3, 4):
        n_det, n_samp = (1024, 512) if i == 3 else (2048, 256)
        vol = mu_phantom(256)
        f = (n_det / 2.0) / math.tan(math.radians(10.0))
        K = intrinsics(f, n_det / 2.0, n_det / 2.0)
        poses = pose_from_rotation_and_centre(np.eye(3), [0.0, 0.0, -1000.0])[None]
        w = Workload(WORKLOAD_NAMES[i], vol, sp, K, poses, n_det, n_det, n_samp, BEER_LAMBERT)
        if i == 3:
            w.grad_out = geo_rng.uniform(-1.0, 1.0, size=(1, n_det, n_det)).astype(np.float32)
    elif i == 5:
        vrng = np.random.default_rng(VOLUME_SEED_BASE + i)
        vol = np.ascontiguousarray(vrng.uniform(0.0, 1.0, size=(128, 128, 128)).astype(np.float32))
        K = intrinsics(512.0 / 0.8, 192.0, 128.0)
        poses = helical_poses(360, 320.0, 40.0, 1.0)
        w = Workload(WORKLOAD_NAMES[5], vol, sp, K, poses, 256, 384, 256, LINE_INTEGRAL)
        w.grad_out = geo_rng.uniform(0.0, 1.0, size=(360, 256, 384)).astype(np.float32)
    else:
        raise ValueError(f"unknown workload {i}")
    if with_bf16:
        w.volume_bf16 = round_to_bf16_bits(w.volume)
    return w


def make_random_small(seed: int, shape=(7, 9, 11), n_views=2, det=(13, 17), n_samples=37,
                      mode=BEER_LAMBERT, spacing=(1.0, 1.25, 0.8), distance=60.0,
                      rot_deg=40.0) -> Workload:
    """Small random workload with ragged sizes and anisotropic spacing, for
    parity cases that span several pixel tiles plus a ragged tail."""
    rng = np.random.default_rng(seed)
    nz, ny, nx = shape
    vol = np.ascontiguousarray(rng.uniform(0.0, 1.0, size=shape).astype(np.float32))
    sp = np.asarray(spacing, dtype=np.float32)
    H, W = det
    ext = max(nx * sp[0], ny * sp[1], nz * sp[2])
    f = 1.2 * max(H, W) * distance / ext
    K = intrinsics(f, W / 2.0 + 0.3, H / 2.0 - 0.2)
    poses = random_poses(n_views, distance, rot_deg, 0.05 * ext, seed=seed + 7)
    g = rng.uniform(-1.0, 1.0, size=(n_views, H, W)).astype(np.float32)
    return Workload(f"random-{seed}", vol, sp, K, poses, H, W, n_samples, mode, grad_out=g)
