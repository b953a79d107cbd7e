"""Pins for the oracle's flashdrr front end (``oracle.render`` and
``oracle.render_adjoint``): volume and channel batching, the density factor,
front-to-back alpha compositing, the per-channel transfer function and the
per-view near/far clipping mode with zero padding.

Passages (source pages): flashdrr API, VolumeRaycaster.forward -- (B, C, D, H, W)
volumes, N = B * views_per_vol views, output (N, C, H, W); VolumeRaycaster.__init__
-- density_factor, use_beer_lambert = False selects front-to-back alpha
compositing (the over operator); compute_clipping_distances -- per-view near/far
from the closest / farthest volume point plus a margin; Transfer functions,
piecewise_linear_channelwise -- per-channel piecewise-linear map extending its end
segments.

Each pin fixes the result by something other than the oracle's own code: closed
forms (a constant box under Beer-Lambert, line integral and compositing; near/far
distances of a box), the over operator written out on a voxel column, numpy.interp
for zero padding and for the transfer function, finite differences and the adjoint
identity for the gradients.  A slip in the batching index, in the order of the
compositing, in where the density factor enters, in the padding, in the near/far
geometry or in the transfer function's slope fails at least one of them.
"""
import math

import numpy as np
import pytest

import oracle
import workloads as W

BL, RAW, ALPHA = oracle.BEER_LAMBERT, oracle.LINE_INTEGRAL, oracle.ALPHA_COMPOSITE
BOX, NEAR_FAR = oracle.CLIP_BOX, oracle.CLIP_NEAR_FAR

# camera axis along +z or -z (third row = camera forward in world coordinates)
FORWARD_Z = {"+z": np.eye(3), "-z": np.diag([1.0, -1.0, -1.0])}


def centre(pose):
    P = np.asarray(pose, dtype=np.float32).astype(np.float64)
    return -P[:, :3].T @ P[:, 3]


def direction(K, pose, r, c):
    K = np.asarray(K, dtype=np.float32).astype(np.float64)
    R = np.asarray(pose, dtype=np.float32).astype(np.float64)[:, :3]
    d = R.T @ np.linalg.solve(K, np.array([c + 0.5, r + 0.5, 1.0]))
    return d / np.linalg.norm(d)


def chord_by_faces(C, d, E):
    """Length of {C + t d : t >= 0} inside the box [-E/2, E/2] from the face-plane
    intersections (not the oracle's slab test)."""
    ts = []
    for a in range(3):
        if d[a] == 0.0:
            continue
        for sgn in (-1.0, 1.0):
            t = (sgn * E[a] / 2 - C[a]) / d[a]
            p = C + t * d
            if all(abs(p[b]) <= E[b] / 2 * (1 + 1e-12) for b in range(3) if b != a):
                ts.append(t)
    if len(ts) < 2:
        return 0.0
    return max(max(ts) - max(min(ts), 0.0), 0.0)


def column_camera(axis, cx, cy, dist, m=5):
    """m x m detector whose central pixel looks along the z axis (``axis``) from
    (cx, cy, -+dist) through the voxel column at (cx, cy)."""
    sign = 1.0 if axis == "+z" else -1.0
    K = W.intrinsics(50.0, m / 2.0, m / 2.0)
    pose = W.pose_from_rotation_and_centre(FORWARD_Z[axis], np.array([cx, cy, -sign * dist]))
    return K, pose[None], m


def over(vals, f, dz):
    """The front-to-back over operator written out: each slab of thickness dz
    has opacity 1 - exp(-f v dz) and emits v."""
    I, T = 0.0, 1.0
    for v in vals:
        a = 1.0 - math.exp(-f * v * dz)
        I += T * a * v
        T *= 1.0 - a
    return I


def pwl_numpy(x, xp, yp):
    """Piecewise-linear map with both end segments extended: numpy.interp inside,
    the end segments' lines outside."""
    x = np.asarray(x, dtype=np.float64)
    y = np.interp(x, xp, yp)
    lo, hi = x < xp[0], x > xp[-1]
    y[lo] = yp[0] + (x[lo] - xp[0]) * (yp[1] - yp[0]) / (xp[1] - xp[0])
    y[hi] = yp[-1] + (x[hi] - xp[-1]) * (yp[-1] - yp[-2]) / (xp[-1] - xp[-2])
    return y


def _problem(seed, B=2, C=2, views_per_vol=2, shape=(5, 4, 6), det=(3, 4), N=7):
    rng = np.random.default_rng(seed)
    vol = rng.uniform(0.05, 1.0, size=(B, C) + shape).astype(np.float32)
    spacing = np.array([1.0, 1.2, 0.9], dtype=np.float32)
    K = W.intrinsics(12.0, det[1] / 2 + 0.1, det[0] / 2 - 0.2)
    poses = W.random_poses(B * views_per_vol, 12.0, 60.0, 0.3, seed=seed + 100)
    return rng, vol, spacing, K, poses, det[0], det[1], N


# ----------------------------------------------------------------- closed forms

@pytest.mark.parametrize("mode", [BL, RAW, ALPHA])
def test_constant_box_closed_forms_with_density_factor(mode):
    """A constant mu box: tau = f mu L for every N; Beer-Lambert 1 - exp(-f mu L);
    compositing sum_k T_k alpha_k mu telescopes to mu (1 - exp(-f mu L))."""
    shape = (6, 5, 7)
    spacing = np.array([1.1, 0.9, 1.3], dtype=np.float32)
    sp = spacing.astype(np.float64)
    E = np.array([shape[2] * sp[0], shape[1] * sp[1], shape[0] * sp[2]])
    mu = float(np.float32(0.23))
    vol = np.full(shape, mu, dtype=np.float32)
    K = W.intrinsics(30.0, 6.3, 5.1)
    poses = W.random_poses(2, 40.0, 60.0, 1.0, seed=5)
    H, Wd = 11, 13
    hits = 0
    for f in (1.0, 0.37, 4.5):
        for N in (1, 3, 64):
            img, tau = oracle.render(vol, spacing, K, poses, H, Wd, N, mode, density_factor=f)
            for v in range(2):
                Cc = centre(poses[v])
                for r in range(H):
                    for c in range(Wd):
                        L = chord_by_faces(Cc, direction(K, poses[v], r, c), E)
                        hits += L > 0
                        want = {BL: -math.expm1(-f * mu * L), RAW: f * mu * L,
                                ALPHA: mu * -math.expm1(-f * mu * L)}[mode]
                        assert tau[v, 0, r, c] == pytest.approx(f * mu * L, rel=1e-11, abs=1e-12)
                        assert img[v, 0, r, c] == pytest.approx(want, rel=1e-11, abs=1e-13)
    assert hits > 200


def test_batching_index_by_constant_channel_volumes():
    """B volumes of C channels, each channel-volume a distinct constant: the line
    integral of view v, channel c is mu[v // views_per_vol, c] times the chord."""
    B, Cn, vpv = 2, 3, 2
    shape = (4, 5, 6)
    spacing = np.array([1.0, 1.1, 0.8], dtype=np.float32)
    sp = spacing.astype(np.float64)
    E = np.array([shape[2] * sp[0], shape[1] * sp[1], shape[0] * sp[2]])
    mus = np.array([[0.1, 0.2, 0.3], [0.5, 0.7, 1.1]], dtype=np.float32)
    vol = np.broadcast_to(mus[:, :, None, None, None], (B, Cn) + shape).astype(np.float32)
    K = W.intrinsics(20.0, 4.5, 3.5)
    poses = W.random_poses(B * vpv, 30.0, 60.0, 1.0, seed=9)
    H, Wd = 7, 9
    img, _ = oracle.render(vol, spacing, K, poses, H, Wd, 5, RAW)
    assert img.shape == (B * vpv, Cn, H, Wd)
    for v in range(B * vpv):
        Cc = centre(poses[v])
        for r in range(H):
            for c in range(Wd):
                L = chord_by_faces(Cc, direction(K, poses[v], r, c), E)
                for ch in range(Cn):
                    assert img[v, ch, r, c] == pytest.approx(float(mus[v // vpv, ch]) * L,
                                                             rel=1e-11, abs=1e-12)


@pytest.mark.parametrize("axis", ["+z", "-z"])
@pytest.mark.parametrize("f", [1.0, 2.5])
def test_alpha_compositing_is_the_over_operator_on_a_voxel_column(axis, f):
    """A ray along z through voxel centres with N = nz samples lands every sample
    on a voxel centre, so compositing reduces to the over operator applied to
    the column front to back (reversed when looking along -z); Beer-Lambert and
    the line integral reduce to the column sum."""
    rng = np.random.default_rng(11)
    shape = (9, 4, 5)
    spacing = np.array([1.0, 1.0, 1.0], dtype=np.float32)
    vol = rng.uniform(0.0, 0.8, size=shape).astype(np.float32)
    i, j = 2, 1
    cx, cy = W.voxel_centres(shape[2], 1.0)[i], W.voxel_centres(shape[1], 1.0)[j]
    K, poses, m = column_camera(axis, cx, cy, 50.0)
    col = vol[:, j, i].astype(np.float64)
    if axis == "-z":
        col = col[::-1]
    dz = 1.0
    img, tau = oracle.render(vol, spacing, K, poses, m, m, shape[0], ALPHA, density_factor=f)
    assert img[0, 0, m // 2, m // 2] == pytest.approx(over(col, f, dz), rel=1e-12)
    assert over(col, f, dz) != pytest.approx(over(col[::-1], f, dz), rel=1e-6)  # order matters
    assert tau[0, 0, m // 2, m // 2] == pytest.approx(f * dz * col.sum(), rel=1e-12)
    img_bl, _ = oracle.render(vol, spacing, K, poses, m, m, shape[0], BL, density_factor=f)
    assert img_bl[0, 0, m // 2, m // 2] == pytest.approx(-math.expm1(-f * dz * col.sum()),
                                                         rel=1e-12)


def test_near_far_distances_closed_form():
    """Closest box point and farthest corner: on the axis, off to the side, and
    from inside the box (near clamps at 0)."""
    E = np.array([10.0, 12.0, 8.0])
    h = E / 2
    for Cc, dn in [(np.array([0.0, 0.0, -50.0]), 50.0 - h[2]),
                   (np.array([h[0] + 3.0, h[1] + 4.0, 1.0]), 5.0),
                   (np.array([1.0, -2.0, 0.5]), 0.0)]:
        pose = W.pose_from_rotation_and_centre(np.eye(3), Cc)
        dfar = math.sqrt(sum((abs(Cc[a]) + h[a]) ** 2 for a in range(3)))
        for margin in (0.0, 2.0, 30.0):
            near, far = oracle.view_range(E, pose, margin)
            assert near == pytest.approx(max(dn - margin, 0.0), abs=1e-12)
            assert far == pytest.approx(dfar + margin, rel=1e-14)


@pytest.mark.parametrize("axis", ["+z", "-z"])
@pytest.mark.parametrize("N", [4, 37, 256])
def test_near_far_samples_are_zero_padded_numpy_interp(axis, N):
    """In the near/far mode every ray samples the midpoints of [near, far]; a
    column ray sees the linear interpolation of its voxel column with a zero
    voxel beyond each end (grid_sample's zero padding), 0 further out."""
    rng = np.random.default_rng(3)
    shape = (8, 3, 4)
    spacing = np.array([1.0, 1.0, 1.25], dtype=np.float32)
    base = rng.uniform(0.1, 1.0, size=shape[0]).astype(np.float32)
    vol = np.broadcast_to(base[:, None, None], shape).astype(np.float32)
    cx, cy = W.voxel_centres(shape[2], 1.0)[1], W.voxel_centres(shape[1], 1.0)[2]
    dist, margin, f = 30.0, 7.5, 1.7
    K, poses, m = column_camera(axis, cx, cy, dist)
    Ez = shape[0] * 1.25
    E = np.array([shape[2] * 1.0, shape[1] * 1.0, Ez])
    near = dist - Ez / 2 - margin
    far = math.sqrt((E[0] / 2 + abs(cx)) ** 2 + (E[1] / 2 + abs(cy)) ** 2 + (dist + Ez / 2) ** 2) \
        + margin
    dz = (far - near) / N
    t = near + (np.arange(N) + 0.5) * dz
    sign = 1.0 if axis == "+z" else -1.0
    z = -sign * dist + sign * t
    q = (z + Ez / 2) / 1.25 - 0.5
    col = np.concatenate([[0.0], base.astype(np.float64), [0.0]])
    vals = np.interp(q, np.arange(-1, shape[0] + 1), col, left=0.0, right=0.0)
    for mode in (RAW, ALPHA):
        img, tau = oracle.render(vol, spacing, K, poses, m, m, N, mode, density_factor=f,
                                 clip=NEAR_FAR, margin=margin)
        assert tau[0, 0, m // 2, m // 2] == pytest.approx(f * dz * vals.sum(), rel=1e-12,
                                                          abs=1e-14)
        if mode == ALPHA:
            assert img[0, 0, m // 2, m // 2] == pytest.approx(over(vals, f, dz), rel=1e-12,
                                                              abs=1e-14)


def test_near_far_constant_box_outside_rays_and_far_before_near():
    """Zero padding: a ray that passes beside the box renders exactly 0 (it would
    see the clamped edge value otherwise); a negative margin that puts far
    before near renders 0 everywhere."""
    shape = (4, 4, 4)
    spacing = np.ones(3, dtype=np.float32)
    vol = np.full(shape, 0.5, dtype=np.float32)
    K = W.intrinsics(10.0, 10.0, 10.0)
    pose = W.pose_from_rotation_and_centre(np.eye(3), np.array([0.0, 0.0, -30.0]))[None]
    img, _ = oracle.render(vol, spacing, K, pose, 20, 20, 64, RAW, clip=NEAR_FAR, margin=5.0)
    assert img[0, 0, 0, 0] == 0.0 and img[0, 0, 10, 10] > 0.0
    img_box, _ = oracle.render(vol, spacing, K, pose, 20, 20, 64, RAW)
    assert img_box[0, 0, 0, 0] == 0.0
    img2, _ = oracle.render(vol, spacing, K, pose, 20, 20, 8, RAW, clip=NEAR_FAR, margin=-40.0)
    assert np.all(img2 == 0.0)


def test_transfer_function_acts_on_voxels_before_sampling():
    """Per-channel knots: rendering x through the transfer function equals
    rendering the volume mapped voxel by voxel with numpy.interp (ends extended),
    in every mode and both clip modes.  The mapped volume passes the fp32
    interface, so the comparison allows fp32 rounding of each voxel."""
    rng, vol, spacing, K, poses, H, Wd, N = _problem(21)
    vol = rng.uniform(-1200.0, 1800.0, size=vol.shape).astype(np.float32)
    xp = np.array([[-1000.0, 0.0, 1500.0], [-500.0, 200.0, 900.0]])
    yp = np.array([[0.0, 0.02, 0.05], [0.01, 0.0, 0.03]])
    mapped = np.stack([pwl_numpy(vol[:, c], xp[c], yp[c]) for c in range(2)], axis=1)
    assert mapped.min() < 0.0 and mapped.max() > 0.05   # both end segments are exercised
    for mode in (BL, RAW, ALPHA):
        for clip in (BOX, NEAR_FAR):
            kw = dict(density_factor=3.0, clip=clip, margin=2.0)
            a, ta = oracle.render(vol, spacing, K, poses, H, Wd, N, mode, transfer=(xp, yp), **kw)
            b, tb = oracle.render(mapped.astype(np.float32), spacing, K, poses, H, Wd, N, mode,
                                  **kw)
            assert np.abs(a).max() > 0
            assert np.allclose(a, b, rtol=1e-6, atol=1e-6 * np.abs(a).max())
            assert np.allclose(ta, tb, rtol=1e-6, atol=1e-6 * np.abs(ta).max())


# ----------------------------------------------------------------- gradients

def _loss(vol, g, args, kw):
    img, _ = oracle.render(vol, *args, **kw)
    return float((img * g).sum())


@pytest.mark.parametrize("mode", [BL, RAW, ALPHA])
@pytest.mark.parametrize("clip", [BOX, NEAR_FAR])
@pytest.mark.parametrize("tf", [False, True])
def test_gradient_matches_central_differences(mode, clip, tf):
    """Directional and per-entry central differences of sum(g * render) against
    render_adjoint, with batching, a density factor and (optionally) a transfer
    function; fp64 volumes are perturbed through an exact route (the fp32
    interface), so h is chosen on the fp32 grid."""
    rng, vol, spacing, K, poses, H, Wd, N = _problem(30 + mode + 3 * clip)
    xp = np.array([[0.0, 0.4, 1.1], [0.1, 0.5, 0.9]])
    yp = np.array([[0.0, 0.5, 0.6], [0.2, 0.0, 0.7]])
    kw = dict(density_factor=1.7, clip=clip, margin=1.5, transfer=(xp, yp) if tf else None)
    args = (spacing, K, poses, H, Wd, N, mode)
    V, C = poses.shape[0], vol.shape[1]
    g = rng.normal(size=(V, C, H, Wd))
    grad = oracle.render_adjoint(vol, spacing, K, poses, H, Wd, N, mode, g, **kw)
    assert np.abs(grad).max() > 0
    # per-entry central differences on a sample of voxels (h on the fp32 grid)
    flat = vol.reshape(-1)
    # voxels not within 1e-3 of a knot, so that +-h stays on one segment
    away = np.min(np.abs(flat[:, None] - xp.reshape(1, -1)), axis=1) > 1e-3
    idx = rng.choice(np.flatnonzero(away), size=24, replace=False)
    for i in idx:
        h = float(np.float32(2.0 ** -12))
        vp, vm = flat.copy(), flat.copy()
        vp[i] += h
        vm[i] -= h
        fd = (_loss(vp.reshape(vol.shape), g, args, kw) -
              _loss(vm.reshape(vol.shape), g, args, kw)) / (float(vp[i]) - float(vm[i]))
        assert fd == pytest.approx(grad.reshape(-1)[i], rel=1e-5, abs=1e-7 * np.abs(grad).max())


def test_adjoint_identity_with_batching_density_factor_and_near_far():
    """Line-integral mode is linear in the volume: <A x, y> = <x, A^T y> to fp64
    round-off, per clip mode, with B = 2, C = 2 and f = 2.5."""
    for clip in (BOX, NEAR_FAR):
        rng, vol, spacing, K, poses, H, Wd, N = _problem(50 + clip)
        y = rng.normal(size=(poses.shape[0], vol.shape[1], H, Wd))
        ax, _ = oracle.render(vol, spacing, K, poses, H, Wd, N, RAW, density_factor=2.5,
                              clip=clip, margin=3.0)
        aty = oracle.render_adjoint(vol, spacing, K, poses, H, Wd, N, RAW, y,
                                    density_factor=2.5, clip=clip, margin=3.0)
        lhs = float((ax * y).sum())
        rhs = float((vol.astype(np.float64) * aty).sum())
        assert lhs == pytest.approx(rhs, rel=1e-12)


def test_reduces_to_the_single_volume_forward_and_adjoint():
    """B = C = 1, f = 1, box clip, no transfer function: the same operator as
    oracle.forward / oracle.adjoint (pinned separately by closed forms)."""
    w = W.make_random_small(7)
    for mode in (BL, RAW):
        a, s = oracle.forward(w.volume, w.spacing, w.K, w.poses, w.det_h, w.det_w, w.n_samples,
                              mode)
        b, tau = oracle.render(w.volume, w.spacing, w.K, w.poses, w.det_h, w.det_w, w.n_samples,
                               mode)
        assert np.array_equal(a, b[:, 0]) and np.array_equal(s, tau[:, 0])
        g = np.random.default_rng(8).normal(size=a.shape)
        ga, _ = oracle.adjoint(w.volume, w.volume.shape, w.spacing, w.K, w.poses, w.det_h,
                               w.det_w, w.n_samples, mode, g)
        gb = oracle.render_adjoint(w.volume, w.spacing, w.K, w.poses, w.det_h, w.det_w,
                                   w.n_samples, mode, g[:, None])
        assert np.allclose(ga, gb, rtol=1e-12, atol=1e-14 * np.abs(ga).max())


def test_invalid_arguments_are_rejected():
    rng, vol, spacing, K, poses, H, Wd, N = _problem(60)
    with pytest.raises(ValueError):     # 4 views cannot split over 3 volumes
        oracle.render(np.concatenate([vol, vol[:1]]), spacing, K, poses, H, Wd, N, RAW)
    with pytest.raises(ValueError):     # knots not increasing
        oracle.render(vol, spacing, K, poses, H, Wd, N, RAW,
                      transfer=(np.array([[0.0, 0.0], [0.0, 1.0]]), np.ones((2, 2))))
    with pytest.raises(ValueError):     # unknown mode
        oracle.render(vol, spacing, K, poses, H, Wd, N, 7)


@pytest.mark.parametrize("mode", [BL, RAW, ALPHA])
@pytest.mark.parametrize("clip", [BOX, NEAR_FAR])
@pytest.mark.parametrize("tf", [False, True])
def test_render_pose_gradient_matches_central_differences(mode, clip, tf):
    """The batched pose gradient (per view, summed over its channels, density
    factor and transfer function included) equals central differences of
    oracle.render with respect to each pose entry (fp64 poses pass through), in
    every mode and both clips."""
    rng, vol, spacing, K, poses, H, Wd, N = _problem(70 + mode + 3 * clip + 6 * tf)
    xp = np.array([[0.0, 0.4, 1.1], [0.1, 0.5, 0.9]], dtype=np.float32)
    yp = np.array([[0.0, 0.5, 0.6], [0.2, 0.0, 0.7]], dtype=np.float32)
    transfer = (xp, yp) if tf else None
    f = 0.8 if mode != ALPHA else 1.7
    margin = 2.5
    g = rng.normal(size=(poses.shape[0], vol.shape[1], H, Wd))
    gp = oracle.render_pose_gradient(vol, spacing, K, poses, H, Wd, N, mode, g,
                                     density_factor=f, transfer=transfer, clip=clip,
                                     margin=margin)
    P = np.asarray(poses, dtype=np.float32).astype(np.float64)
    h = 1e-6
    for v in (0, 3):
        for e in range(12):
            Pp, Pm = P.copy(), P.copy()
            Pp[v].reshape(-1)[e] += h
            Pm[v].reshape(-1)[e] -= h
            lp = float((oracle.render(vol, spacing, K, Pp, H, Wd, N, mode, density_factor=f,
                                      clip=clip, margin=margin, transfer=transfer)[0] * g).sum())
            lm = float((oracle.render(vol, spacing, K, Pm, H, Wd, N, mode, density_factor=f,
                                      clip=clip, margin=margin, transfer=transfer)[0] * g).sum())
            fd = (lp - lm) / (2 * h)
            assert fd == pytest.approx(gp[v].reshape(-1)[e], rel=1e-4,
                                       abs=1e-5 * np.abs(gp[v]).max())
    assert np.abs(gp[[0, 3]]).max() > 1e-3


def _transfer_numpy(x, xp, yp):
    """The per-channel piecewise-linear map written out in numpy: linear between
    knots, the first and last segments extended beyond them."""
    x = np.asarray(x, dtype=np.float64)
    xp = np.asarray(xp, dtype=np.float64)
    yp = np.asarray(yp, dtype=np.float64)
    seg = np.clip(np.searchsorted(xp, x, side="right") - 1, 0, len(xp) - 2)
    m = (yp[seg + 1] - yp[seg]) / (xp[seg + 1] - xp[seg])
    return yp[seg] + m * (x - xp[seg])


@pytest.mark.parametrize("mode", [BL, RAW])
def test_render_pose_gradient_is_the_plain_pose_gradient_per_channel(mode):
    """Beer-Lambert and the line integral with the box clip: render(x) with
    factor f and map tf is the plain forward of f * tf(x), so the render pose
    gradient equals oracle.pose_gradient (a separately pinned routine, a
    different code path) on each channel-volume f * tf(x) (rounded to fp32 for
    its interface), summed over a view's channels."""
    rng, vol, spacing, K, poses, H, Wd, N = _problem(90 + mode)
    xp = np.array([[0.0, 0.4, 1.1], [0.1, 0.5, 0.9]], dtype=np.float32)
    yp = np.array([[0.0, 0.5, 0.6], [0.2, 0.0, 0.7]], dtype=np.float32)
    f = 0.8
    B, C = vol.shape[:2]
    P = np.asarray(poses, dtype=np.float64).reshape(-1, 3, 4)
    V = P.shape[0]
    vpv = V // B
    g = rng.normal(size=(V, C, H, Wd))
    gp = oracle.render_pose_gradient(vol, spacing, K, poses, H, Wd, N, mode, g,
                                     density_factor=f, transfer=(xp, yp))
    ref = np.zeros((V, 3, 4))
    for b in range(B):
        for c in range(C):
            m = (f * _transfer_numpy(vol[b, c], xp[c], yp[c])).astype(np.float32)
            views = slice(b * vpv, (b + 1) * vpv)
            ref[views] += oracle.pose_gradient(m, spacing, K, P[views], H, Wd, N, mode,
                                               g[views, c])
    assert np.abs(gp - ref).max() <= 1e-6 * np.abs(ref).max()


def test_compositing_pose_gradient_of_constant_box_is_the_chord_derivative():
    """For a constant mu_c volume and the box clip, every sample reads mu_c and
    the over operator sums a geometric series: I = mu_c (1 - exp(-f mu_c L))
    with L the chord.  So dL/dP of sum g I is g f mu_c^2 exp(-f mu_c L) dL/dP,
    the chord from face intersections and its derivative by central
    differences of that chord (no voxels, no compositing loop)."""
    mu_c = float(np.float32(0.07))
    f = 1.3
    shape = (8, 10, 12)
    vol = np.full(shape, mu_c, dtype=np.float32)
    spacing = np.ones(3, dtype=np.float32)
    E = np.array([12.0, 10.0, 8.0])
    K = W.intrinsics(12.0, 2.5, 2.5)
    poses = W.random_poses(1, 30.0, 35.0, 1.0, seed=52).astype(np.float64)
    g = np.random.default_rng(53).normal(size=(1, 1, 5, 5))
    grad = oracle.render_pose_gradient(vol, spacing, K, poses, 5, 5, 17, ALPHA, g,
                                       density_factor=f)

    def chords(P):
        Rm, t = P[:, :3], P[:, 3]
        C = -Rm.T @ t
        out = np.zeros((5, 5))
        for r in range(5):
            for c in range(5):
                u = np.linalg.solve(K.astype(np.float64), [c + 0.5, r + 0.5, 1.0])
                d = Rm.T @ u
                out[r, c] = chord_by_faces(C, d / np.linalg.norm(d), E)
        return out

    L0 = chords(poses[0])
    ref = np.zeros((3, 4))
    h = 1e-6
    for r in range(3):
        for c in range(4):
            up, dn = poses[0].copy(), poses[0].copy()
            up[r, c] += h
            dn[r, c] -= h
            dL = (chords(up) - chords(dn)) / (2 * h)
            ref[r, c] = float((g[0, 0] * f * mu_c ** 2 * np.exp(-f * mu_c * L0) * dL).sum())
    assert (L0 > 0).sum() > 10
    assert np.abs(grad[0] - ref).max() <= 1e-6 * np.abs(ref).max()
