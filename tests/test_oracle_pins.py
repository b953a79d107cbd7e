"""Pins for the CPU oracle (``oracle/``), checked against what the pages and the
mathematics fix rather than against the oracle itself.

Passages the method follows (source pages):
  * nanodrr page, introduction -- Hartley-Zisserman pinhole camera P = K [R | t].
  * flashdrr API, VolumeRaycaster.__init__ -- ``ray_samples`` samples per ray;
    ``use_beer_lambert`` returns 1 - exp(-int mu dz).
  * flashdrr API, VolumeRaycaster.set_fov -- per-pixel directions normalised.
  * diffct 2.1.0, Quickstart -- project() = line integrals, backproject() = A^T,
    x.grad = A^T (A x - y) for 0.5 ||A x - y||^2.
  * torchtomo, "Discrete Adjoint and Learned Primal-Dual" -- <A x, y> = <x, A^T y>;
    prefer float64 and aggregate residuals for adjoint diagnostics.

Each pin is chosen so that a plausible slip in the oracle fails it: a wrong
clip or sample count (constant box, chord from face intersections), a dropped
normalisation (chord in mm), a transposed rotation (off-centre ball seen from a
random pose), a missing pixel half-offset (flip symmetry), a wrong index origin
or axis order (numpy.interp along each axis; affine field), left- instead of
midpoint sampling (reversal symmetry, affine exactness), a wrong adjoint
(dense brute force, finite differences).
"""
import math

import numpy as np
import pytest

import oracle
import workloads as W

BL, RAW = oracle.BEER_LAMBERT, oracle.LINE_INTEGRAL


# ----------------------------------------------------------------- independent helpers

def direction(K, pose, r, c):
    """Unit ray direction computed with numpy.linalg (not the oracle's code)."""
    K = np.asarray(K, dtype=np.float32).astype(np.float64)
    R = np.asarray(pose, dtype=np.float32).astype(np.float64)[:, :3]
    dc = np.linalg.solve(K, np.array([c + 0.5, r + 0.5, 1.0]))
    d = R.T @ dc
    return d / np.linalg.norm(d)


def centre(pose):
    P = np.asarray(pose, dtype=np.float32).astype(np.float64)
    return -P[:, :3].T @ P[:, 3]


def chord_by_faces(C, d, E):
    """Length of {C + t d : t >= 0} inside the box [-E/2, E/2], found by
    intersecting the six face planes and keeping points inside the face
    rectangles (a different route from the oracle's slab test)."""
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


def rotation_with_forward(u):
    """A proper rotation (world->camera rows) whose third row is the unit vector u."""
    u = np.asarray(u, dtype=np.float64)
    u = u / np.linalg.norm(u)
    helper = np.array([0.0, 1.0, 0.0]) if abs(u[1]) < 0.9 else np.array([1.0, 0.0, 0.0])
    x = np.cross(helper, u)
    x /= np.linalg.norm(x)
    y = np.cross(u, x)
    R = np.stack([x, y, u])
    assert abs(np.linalg.det(R) - 1.0) < 1e-12
    return R


def central_pixel_camera(R, C, f=50.0, n=5):
    """Odd n x n detector whose central pixel's ray is exactly the camera axis."""
    K = W.intrinsics(f, n / 2.0, n / 2.0)
    pose = W.pose_from_rotation_and_centre(R, C)
    return K, pose, n


def fwd(vol, spacing, K, poses, H, Wd, N, mode):
    poses = np.asarray(poses, dtype=np.float32).reshape(-1, 3, 4)
    return oracle.forward(vol, spacing, K, poses, H, Wd, N, mode, n_threads=4)


# ----------------------------------------------------------------- clip, dz, sample count

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_constant_box_equals_mu_times_chord_for_every_N(seed):
    """A constant mu_c volume integrates to mu_c * chord exactly, whatever N,
    and the Beer-Lambert image is 1 - exp(-mu_c * chord)."""
    rng = np.random.default_rng(seed)
    shape = tuple(int(x) for x in rng.integers(3, 12, size=3))
    spacing = rng.uniform(0.5, 2.0, size=3).astype(np.float32)
    mu_c = float(np.float32(0.037))
    vol = np.full(shape, mu_c, dtype=np.float32)
    sp64 = spacing.astype(np.float64)
    E = np.array([shape[2] * sp64[0], shape[1] * sp64[1], shape[0] * sp64[2]])
    ext = float(E.max())
    K = W.intrinsics(40.0, 9.5, 7.3)
    poses = W.random_poses(3, 4.0 * ext, 60.0, 0.1 * ext, seed=seed + 10)
    H, Wd = 15, 19
    hits = 0
    for N in (1, 2, 7, 64, 301):
        img, s = fwd(vol, spacing, K, poses, H, Wd, N, BL)
        for v in range(3):
            C = centre(poses[v])
            for r in range(H):
                for c in range(Wd):
                    L = chord_by_faces(C, direction(K, poses[v], r, c), E)
                    hits += L > 0
                    assert s[v, r, c] == pytest.approx(mu_c * L, rel=1e-11, abs=1e-11 * ext)
                    assert img[v, r, c] == pytest.approx(-math.expm1(-mu_c * L), rel=1e-11,
                                                         abs=1e-13)
        ch = oracle.chords(E, K, poses, H, Wd)
        for v in range(3):
            C = centre(poses[v])
            for r in range(H):
                for c in range(Wd):
                    L = chord_by_faces(C, direction(K, poses[v], r, c), E)
                    assert ch[v, r, c] == pytest.approx(L, rel=1e-11, abs=1e-11 * ext)
    assert hits > 100  # the geometry really exercises the box


def test_constant_box_central_axis_and_oblique_closed_forms():
    """Chord of the camera axis through the box centre: Ez on axis, and
    min(Ez / |cos th|, Ex / |sin th|) for an axis tilted by th in the x-z plane."""
    shape = (40, 30, 50)           # nz, ny, nx
    spacing = np.array([1.0, 1.0, 1.0], dtype=np.float32)
    Ex, Ez = 50.0, 40.0
    mu_c = float(np.float32(0.02))
    vol = np.full(shape, mu_c, dtype=np.float32)
    for th_deg in (0.0, 10.0, 38.0, 51.34, 75.0, 90.0):
        th = math.radians(th_deg)
        u = np.array([math.sin(th), 0.0, math.cos(th)])
        R = rotation_with_forward(u)
        K, pose, n = central_pixel_camera(R, -300.0 * u)
        d = direction(K, pose, n // 2, n // 2)
        L_closed = min(Ez / abs(math.cos(th)) if math.cos(th) > 1e-12 else np.inf,
                       Ex / abs(math.sin(th)) if math.sin(th) > 1e-12 else np.inf)
        img, s = fwd(vol, spacing, K, pose, n, n, 33, RAW)
        # the pose is stored in fp32, so the axis is u up to fp32 rounding
        assert np.allclose(d, u, atol=1e-6)
        assert s[0, n // 2, n // 2] == pytest.approx(mu_c * L_closed, rel=2e-5)


# ----------------------------------------------------------------- ray generation

def test_pixel_directions_and_camera_centre():
    """Identity pose: d(r, c) is ((c + 1/2 - cx) / f, (r + 1/2 - cy) / f, 1)
    normalised and C = -R^T t; for a rotated pose d is R^T of that."""
    K = W.intrinsics(500.0, 32.0, 32.0)
    pose = W.pose_from_rotation_and_centre(np.eye(3), [0.0, 0.0, -500.0])
    for (r, c) in [(0, 0), (31, 32), (63, 5), (10, 60)]:
        hit, C, d, t0, t1 = oracle.ray(K, pose, [64.0, 64.0, 64.0], r, c)
        ref = np.array([(c + 0.5 - 32.0) / 500.0, (r + 0.5 - 32.0) / 500.0, 1.0])
        assert np.allclose(d, ref / np.linalg.norm(ref), rtol=0, atol=1e-15)
        assert np.allclose(C, [0.0, 0.0, -500.0])
        assert hit
        # entering through the z = -32 face; the exit is wherever the box ends
        assert t0 == pytest.approx(468.0 / d[2], rel=1e-14)
        E = np.array([64.0, 64.0, 64.0])
        assert t1 - t0 == pytest.approx(chord_by_faces(C, ref / np.linalg.norm(ref), E),
                                        rel=1e-12)
    Rr = W._rot_z(0.3) @ W._rot_x(-0.4)
    pose = W.pose_from_rotation_and_centre(Rr, [5.0, -7.0, -300.0])
    R32 = pose[:, :3].astype(np.float64)
    for (r, c) in [(3, 4), (50, 20)]:
        hit, C, d, t0, t1 = oracle.ray(K, pose, [64.0, 64.0, 64.0], r, c)
        dc = np.array([(c + 0.5 - 32.0) / 500.0, (r + 0.5 - 32.0) / 500.0, 1.0])
        ref = R32.T @ dc
        assert np.allclose(d, ref / np.linalg.norm(ref), atol=1e-14)
        assert np.allclose(C, -R32.T @ pose[:, 3].astype(np.float64), atol=1e-12)


def test_image_axes_follow_hartley_zisserman():
    """x to the right (columns), y down (rows): a ball at +x lights up columns
    right of cx, a ball at +y rows below cy."""
    K = W.intrinsics(500.0, 32.0, 32.0)
    pose = W.pose_from_rotation_and_centre(np.eye(3), [0.0, 0.0, -500.0])
    E = [64.0, 64.0, 64.0]
    img = oracle.forward_spheres([[15.0, 0.0, 0.0, 6.0, 0.02]], E, K, pose, 64, 64, 256, RAW)[0]
    r, c = np.unravel_index(np.argmax(img), img.shape)
    assert c > 40 and 28 <= r <= 35
    img = oracle.forward_spheres([[0.0, 15.0, 0.0, 6.0, 0.02]], E, K, pose, 64, 64, 256, RAW)[0]
    r, c = np.unravel_index(np.argmax(img), img.shape)
    assert r > 40 and 28 <= c <= 35


def test_noise_free_sphere_image_symmetries():
    """The noise-free tiny workload (centred sphere, cx = cy = W/2) images to a
    picture symmetric under row flips, column flips and transposition -- which
    holds only with pixel centres at (c + 1/2, r + 1/2)."""
    vol = W.sphere_volume(noise=0.0)
    w = W.make_workload(1)
    img, s = fwd(vol, w.spacing, w.K, w.poses, 64, 64, 128, BL)
    img = img[0]
    scale = img.max()
    assert np.abs(img - img[::-1, :]).max() <= 1e-12 * scale
    assert np.abs(img - img[:, ::-1]).max() <= 1e-12 * scale
    assert np.abs(img - img.T).max() <= 1e-12 * scale
    # and without the half-pixel offset the picture would be off-centre:
    K_shift = W.intrinsics(500.0, 32.5, 32.5)
    img2 = fwd(vol, w.spacing, K_shift, w.poses, 64, 64, 128, BL)[0][0]
    assert np.abs(img2 - img2[::-1, :]).max() > 1e-3 * scale


# ----------------------------------------------------------------- analytic sphere chords

@pytest.mark.parametrize("mode", [RAW, BL])
def test_ball_field_matches_2_mu_sqrt_r2_minus_d2(mode):
    """With an analytic ball density the sampled line integral tends to the
    chord 2 mu sqrt(r^2 - d^2); the midpoint rule on an indicator is off by at
    most mu dz.  An off-centre ball seen from a random rotated pose pins the
    direction of the rotation (R^T, not R)."""
    E = np.array([64.0, 64.0, 64.0])
    balls = [(0.0, 0.0, 0.0, 20.0, 0.02), (9.0, -13.0, 6.0, 11.0, 0.03)]
    K = W.intrinsics(300.0, 20.0, 16.0)
    poses = np.concatenate([
        W.pose_from_rotation_and_centre(np.eye(3), [0.0, 0.0, -400.0])[None],
        W.random_poses(2, 400.0, 35.0, 5.0, seed=5)])
    N = 4096
    for b in balls:
        out = oracle.forward_spheres([b], E, K, poses, 32, 40, N, mode)
        worst = 0.0
        for v in range(poses.shape[0]):
            C = centre(poses[v])
            for r in range(32):
                for c in range(40):
                    d = direction(K, poses[v], r, c)
                    rel = np.array(b[:3]) - C
                    dist2 = max(rel @ rel - (rel @ d) ** 2, 0.0)
                    L = 2.0 * math.sqrt(max(b[3] ** 2 - dist2, 0.0))
                    s_exact = b[4] * L
                    dz = chord_by_faces(C, d, E) / N
                    got = out[v, r, c] if mode == RAW else -math.log1p(-out[v, r, c])
                    assert abs(got - s_exact) <= b[4] * dz * (1 + 1e-9) + 1e-12
                    worst = max(worst, s_exact)
        assert worst > 0.5 * b[4] * 2 * b[3]  # the ball was really hit near its centre


def test_voxelised_sphere_close_to_chord():
    """The voxelised (noise-free) tiny-workload sphere integrates close to the
    analytic chord for rays well inside it (partial-volume tolerance of about
    one voxel of mu at each crossing)."""
    w = W.make_workload(1)
    vol = W.sphere_volume(noise=0.0)
    _, s = fwd(vol, w.spacing, w.K, w.poses, 64, 64, 512, RAW)
    C = centre(w.poses[0])
    n_checked = 0
    for r in range(0, 64, 3):
        for c in range(0, 64, 3):
            d = direction(w.K, w.poses[0], r, c)
            dist2 = max(C @ C - (C @ d) ** 2, 0.0)
            if dist2 <= (0.8 * 20.0) ** 2:
                L = 2.0 * math.sqrt(400.0 - dist2)
                assert abs(s[0, r, c] - 0.02 * L) <= 0.02 * 1.5
                n_checked += 1
    assert n_checked > 50


# ----------------------------------------------------------------- trilinear + clamp + index map

AXIS_ROTATIONS = {
    # third row = camera forward in world coordinates
    "+z": np.eye(3),
    "-z": np.diag([1.0, -1.0, -1.0]),
    "+x": np.array([[0.0, 1.0, 0.0], [0.0, 0.0, 1.0], [1.0, 0.0, 0.0]]),
    "+y": np.array([[0.0, 0.0, 1.0], [1.0, 0.0, 0.0], [0.0, 1.0, 0.0]]),
}


@pytest.mark.parametrize("axis", list(AXIS_ROTATIONS))
@pytest.mark.parametrize("N", [1, 5, 64, 333])
def test_axis_aligned_ray_is_numpy_interp_with_midpoints(axis, N):
    """A ray along a volume axis through voxel centres sees the clamped 1-D
    linear interpolation of that voxel column (numpy.interp clamps to the end
    values), sampled at the N midpoints of the chord."""
    rng = np.random.default_rng(42)
    shape = (9, 7, 11)                       # nz, ny, nx
    spacing = np.array([1.1, 1.3, 0.8], dtype=np.float32)   # sx, sy, sz
    vol = rng.uniform(0.0, 1.0, size=shape).astype(np.float32)
    n = {"x": shape[2], "y": shape[1], "z": shape[0]}
    sp = {"x": float(spacing[0]), "y": float(spacing[1]), "z": float(spacing[2])}
    cx = W.voxel_centres(shape[2], sp["x"])
    cy = W.voxel_centres(shape[1], sp["y"])
    cz = W.voxel_centres(shape[0], sp["z"])
    i, j, k = 3, 5, 2
    R = AXIS_ROTATIONS[axis]
    ax = axis[1]
    sign = -1.0 if axis[0] == "-" else 1.0
    if ax == "z":
        C = np.array([cx[i], cy[j], -sign * 100.0])
        col = vol[:, j, i]
    elif ax == "x":
        C = np.array([-100.0, cy[j], cz[k]])
        col = vol[k, j, :]
    else:
        C = np.array([cx[i], -100.0, cz[k]])
        col = vol[k, :, i]
    K, pose, m = central_pixel_camera(R, C)
    _, s = fwd(vol, spacing, K, pose, m, m, N, RAW)
    L = n[ax] * sp[ax]
    dz = L / N
    # sample positions along the axis, measured from the entry face
    u = (np.arange(N) + 0.5) * dz
    pos = u if sign > 0 else L - u
    q = pos / sp[ax] - 0.5
    expected = dz * np.interp(q, np.arange(n[ax]), col.astype(np.float64)).sum()
    assert s[0, m // 2, m // 2] == pytest.approx(expected, rel=1e-13)


def test_affine_field_is_integrated_exactly():
    """Trilinear interpolation reproduces an affine field between the outermost
    voxel centres and the midpoint rule integrates an affine function exactly,
    so a field a + b x + c y (constant in z) along rays that stay inside that
    region integrates to chord * field(chord midpoint) for every N."""
    shape = (20, 24, 28)
    # dyadic spacings and coefficients: the stored fp32 voxel values are then
    # exactly affine in the voxel centres
    spacing = np.array([1.0, 0.75, 1.25], dtype=np.float32)
    xs = W.voxel_centres(shape[2], 1.0)
    ys = W.voxel_centres(shape[1], 0.75)
    a, b, c = 0.5, 2.0 ** -6, -(2.0 ** -5)
    field = a + b * xs[None, None, :] + c * ys[None, :, None] + np.zeros(shape)
    vol = field.astype(np.float32)
    assert np.array_equal(vol.astype(np.float64), field)
    vol64 = field
    E = np.array([28.0, 24 * 0.75, 20 * 1.25])
    K = W.intrinsics(200.0, 8.0, 8.0)
    pose = W.pose_from_rotation_and_centre(W._rot_z(0.2), [1.0, -0.5, -300.0])
    checked = 0
    for N in (1, 3, 50):
        _, s = fwd(vol, spacing, K, pose, 16, 16, N, RAW)
        _C = centre(pose)
        for r in range(16):
            for cc in range(16):
                d = direction(K, pose, r, cc)
                t_in = (-E[2] / 2 - _C[2]) / d[2]
                t_out = (E[2] / 2 - _C[2]) / d[2]
                p_in, p_out = _C + t_in * d, _C + t_out * d
                if max(abs(p_in[0]), abs(p_out[0])) > xs[-1] or \
                        max(abs(p_in[1]), abs(p_out[1])) > ys[-1]:
                    continue
                pm = 0.5 * (p_in + p_out)
                # bilinear interpolation of the stored values at the midpoint
                qx = (pm[0] - xs[0]) / 1.0
                qy = (pm[1] - ys[0]) / 0.75
                i0, j0 = int(math.floor(qx)), int(math.floor(qy))
                fx, fy = qx - i0, qy - j0
                v = ((1 - fx) * (1 - fy) * vol64[0, j0, i0] + fx * (1 - fy) * vol64[0, j0, i0 + 1]
                     + (1 - fx) * fy * vol64[0, j0 + 1, i0] + fx * fy * vol64[0, j0 + 1, i0 + 1])
                assert s[0, r, cc] == pytest.approx((t_out - t_in) * v, rel=1e-11)
                checked += 1
    assert checked > 60


def test_single_voxel_volume_clamps_to_its_value():
    mu_c = float(np.float32(0.7))
    vol = np.full((1, 1, 1), mu_c, dtype=np.float32)
    spacing = np.array([3.0, 2.0, 5.0], dtype=np.float32)
    E = np.array([3.0, 2.0, 5.0])
    K = W.intrinsics(30.0, 4.5, 4.5)
    pose = W.random_poses(1, 40.0, 30.0, 0.3, seed=3)
    _, s = fwd(vol, spacing, K, pose, 9, 9, 17, RAW)
    C = centre(pose[0])
    for r in range(9):
        for c in range(9):
            L = chord_by_faces(C, direction(K, pose[0], r, c), E)
            assert s[0, r, c] == pytest.approx(mu_c * L, rel=1e-12, abs=1e-12)


# ----------------------------------------------------------------- quadrature

def test_ray_reversal_symmetry():
    """Midpoint samples are symmetric under reversing the ray: the same chord
    traversed from the other side gives the same sum (left-Riemann would not)."""
    rng = np.random.default_rng(7)
    vol = rng.uniform(0.0, 1.0, size=(10, 12, 14)).astype(np.float32)
    spacing = np.array([1.0, 1.1, 0.9], dtype=np.float32)
    for trial in range(5):
        u = rng.normal(size=3)
        u /= np.linalg.norm(u)
        p0 = rng.uniform(-3, 3, size=3)
        for N in (4, 37):
            KA, poseA, m = central_pixel_camera(rotation_with_forward(u), p0 - 200.0 * u)
            KB, poseB, _ = central_pixel_camera(rotation_with_forward(-u), p0 + 200.0 * u)
            sA = fwd(vol, spacing, KA, poseA, m, m, N, RAW)[1][0, m // 2, m // 2]
            sB = fwd(vol, spacing, KB, poseB, m, m, N, RAW)[1][0, m // 2, m // 2]
            assert sA > 0
            # fp32 storage of the two poses perturbs the line by ~1e-7 mm
            assert sA == pytest.approx(sB, rel=2e-5)


def test_exact_integral_pins_and_second_order_convergence():
    """The piecewise-cubic exact integral reproduces the constant-box and affine
    closed forms, and the sampled sums converge to it at second order in N."""
    rng = np.random.default_rng(11)
    shape = (12, 14, 16)
    spacing = np.array([1.0, 1.2, 0.9], dtype=np.float32)
    sp64 = spacing.astype(np.float64)
    E = np.array([16 * sp64[0], 14 * sp64[1], 12 * sp64[2]])
    K = W.intrinsics(60.0, 6.0, 5.0)
    poses = W.random_poses(2, 80.0, 50.0, 1.0, seed=12)
    # constant field
    mu_c = float(np.float32(0.3))
    c0 = np.full(shape, mu_c, dtype=np.float32)
    ex = oracle.exact_line_integral(c0, spacing, K, poses, 10, 12)
    for v in range(2):
        C = centre(poses[v])
        for r in range(10):
            for c in range(12):
                L = chord_by_faces(C, direction(K, poses[v], r, c), E)
                assert ex[v, r, c] == pytest.approx(mu_c * L, rel=1e-11, abs=1e-12)
    # random field: sampled -> exact at order ~2
    vol = rng.uniform(0.0, 1.0, size=shape).astype(np.float32)
    ex = oracle.exact_line_integral(vol, spacing, K, poses, 10, 12)
    errs = []
    Ns = [256, 512, 1024, 2048, 4096]
    for N in Ns:
        _, s = fwd(vol, spacing, K, poses, 10, 12, N, RAW)
        errs.append(np.abs(s - ex).max() / np.abs(ex).max())
    orders = [math.log2(errs[i] / errs[i + 1]) for i in range(len(errs) - 1)]
    assert errs[-1] < 1e-6
    assert np.mean(orders) > 1.7, (errs, orders)


# ----------------------------------------------------------------- output stage

def test_beer_lambert_uses_expm1_for_small_s():
    """1 - exp(-s) must keep full relative precision for tiny s (computed as
    -expm1(-s)); compared with the Taylor series, which is exact to double
    precision at these s, with no absolute slack."""
    spacing = np.ones(3, dtype=np.float32)
    K, pose, m = central_pixel_camera(np.eye(3), [0.0, 0.0, -50.0])
    for mu in (1e-12, 3e-11, 7e-10, 2.5e-9):
        mu32 = float(np.float32(mu))
        vol = np.full((4, 4, 4), mu32, dtype=np.float32)
        img, s = fwd(vol, spacing, K, pose, m, m, 8, BL)
        s_exact = mu32 * 4.0
        assert s[0, m // 2, m // 2] == pytest.approx(s_exact, rel=1e-14, abs=0)
        taylor = s_exact - s_exact ** 2 / 2 + s_exact ** 3 / 6
        assert img[0, m // 2, m // 2] == pytest.approx(taylor, rel=1e-14, abs=0)


def test_source_inside_box_starts_at_zero():
    mu_c = float(np.float32(0.05))
    vol = np.full((10, 10, 10), mu_c, dtype=np.float32)
    spacing = np.ones(3, dtype=np.float32)
    K, pose, m = central_pixel_camera(np.eye(3), [0.0, 0.0, 0.0])
    hit, C, d, t0, t1 = oracle.ray(K, pose, [10.0, 10.0, 10.0], m // 2, m // 2)
    assert hit and t0 == 0.0 and t1 == pytest.approx(5.0)
    _, s = fwd(vol, spacing, K, pose, m, m, 16, RAW)
    assert s[0, m // 2, m // 2] == pytest.approx(mu_c * 5.0, rel=1e-12)


def test_rays_that_miss_give_zero_and_no_gradient():
    vol = np.full((6, 6, 6), 1.0, dtype=np.float32)
    spacing = np.ones(3, dtype=np.float32)
    K = W.intrinsics(100.0, 4.0, 4.0)
    away = W.pose_from_rotation_and_centre(AXIS_ROTATIONS["-z"], [0.0, 0.0, -50.0])
    img, s = fwd(vol, spacing, K, away, 8, 8, 10, BL)
    assert not img.any() and not s.any()
    g, _ = oracle.adjoint(vol, vol.shape, spacing, K, away[None], 8, 8, 10, BL,
                          np.ones((1, 8, 8)))
    assert not g.any()
    # grazing an edge of the box: entry == exit, both readings give 0
    u = np.array([1.0, 0.0, -1.0]) / math.sqrt(2.0)
    Kc, pose, m = central_pixel_camera(rotation_with_forward(u), np.array([3.0, 0.0, 3.0]) - 100 * u)
    _, s = fwd(vol, spacing, Kc, pose, m, m, 10, RAW)
    assert abs(s[0, m // 2, m // 2]) < 1e-5


# ----------------------------------------------------------------- adjoint / backward

def _tiny_problem(seed, mode=RAW):
    rng = np.random.default_rng(seed)
    shape = (4, 4, 4)
    spacing = np.array([1.0, 1.2, 0.9], dtype=np.float32)
    K = W.intrinsics(12.0, 2.1, 1.4)
    poses = W.random_poses(2, 12.0, 60.0, 0.3, seed=seed + 100)
    return rng, shape, spacing, K, poses, 3, 4, 7


def test_dense_matrix_brute_force():
    """Build A column by column from unit volumes (line-integral mode); the
    oracle's adjoint must equal the dense transpose, and its Beer-Lambert
    gradient must equal A^T diag(exp(-A mu)) g."""
    rng, shape, spacing, K, poses, H, Wd, N = _tiny_problem(3)
    n_vox = int(np.prod(shape))
    A = np.zeros((2 * H * Wd, n_vox))
    for vidx in range(n_vox):
        e = np.zeros(n_vox, dtype=np.float32)
        e[vidx] = 1.0
        A[:, vidx] = fwd(e.reshape(shape), spacing, K, poses, H, Wd, N, RAW)[1].ravel()
    assert np.count_nonzero(A) > 50
    x = rng.uniform(0, 1, size=shape).astype(np.float32)
    assert np.allclose(A @ x.ravel().astype(np.float64),
                       fwd(x, spacing, K, poses, H, Wd, N, RAW)[1].ravel(), rtol=1e-13, atol=1e-15)
    y = rng.normal(size=(2, H, Wd))
    aty, _ = oracle.adjoint(None, shape, spacing, K, poses, H, Wd, N, RAW, y)
    assert np.allclose(aty.ravel(), A.T @ y.ravel(), rtol=1e-13, atol=1e-15)
    g_bl, _ = oracle.adjoint(x, shape, spacing, K, poses, H, Wd, N, BL, y)
    s = A @ x.ravel().astype(np.float64)
    assert np.allclose(g_bl.ravel(), A.T @ (np.exp(-s) * y.ravel()), rtol=1e-13, atol=1e-15)


def test_adjoint_identity_aggregate_residual():
    """<A x, y> = <x, A^T y> over many random pairs and geometries, reported as
    an aggregate residual in float64."""
    num = den = 0.0
    for pair in range(40):
        rng = np.random.default_rng(500 + pair)
        shape = tuple(int(v) for v in rng.integers(2, 9, size=3))
        spacing = rng.uniform(0.6, 1.6, size=3).astype(np.float32)
        ext = max(shape[2] * spacing[0], shape[1] * spacing[1], shape[0] * spacing[2])
        K = W.intrinsics(float(rng.uniform(8, 20)), 3.3, 2.7)
        poses = W.random_poses(2, 3.0 * ext, 70.0, 0.2 * ext, seed=900 + pair)
        N = int(rng.integers(1, 40))
        x = rng.normal(size=shape).astype(np.float32)
        y = rng.normal(size=(2, 6, 7))
        ax = fwd(x, spacing, K, poses, 6, 7, N, RAW)[1]
        aty, _ = oracle.adjoint(None, shape, spacing, K, poses, 6, 7, N, RAW, y, n_threads=2)
        lhs = float((ax * y).sum())
        rhs = float((x.astype(np.float64) * aty).sum())
        num += abs(lhs - rhs)
        den += abs(lhs)
    assert num / den < 1e-13


def test_threaded_adjoint_matches_single_thread():
    w = W.make_random_small(5, shape=(12, 10, 14), n_views=3, det=(21, 19), n_samples=50)
    g1, t1 = oracle.adjoint_workload(w, n_threads=1)
    g4, t4 = oracle.adjoint_workload(w, n_threads=4)
    assert t1 == 1 and t4 == 4
    assert np.allclose(g1, g4, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("mode", [BL, RAW])
def test_gradient_matches_central_finite_differences(mode):
    """dL/dmu for L = sum g * I(mu) (Beer-Lambert) and for the diffct least-squares
    loss 0.5 ||A mu - y||^2, whose gradient is A^T (A mu - y)."""
    rng, shape, spacing, K, poses, H, Wd, N = _tiny_problem(9)
    mu = rng.uniform(0.1, 0.6, size=shape)
    h = 1e-4
    if mode == BL:
        g = rng.normal(size=(2, H, Wd))

        def loss(m):
            return float((g * fwd(m.astype(np.float32), spacing, K, poses, H, Wd, N, BL)[0]).sum())

        mu32 = mu.astype(np.float32)
        grad, _ = oracle.adjoint(mu32, shape, spacing, K, poses, H, Wd, N, BL, g)
    else:
        y = rng.normal(size=(2, H, Wd))
        mu32 = mu.astype(np.float32)
        r = fwd(mu32, spacing, K, poses, H, Wd, N, RAW)[1] - y

        def loss(m):
            return 0.5 * float(((fwd(m.astype(np.float32), spacing, K, poses, H, Wd, N, RAW)[1]
                                 - y) ** 2).sum())

        grad, _ = oracle.adjoint(None, shape, spacing, K, poses, H, Wd, N, RAW, r)
    base = mu32.astype(np.float64)
    for flat in rng.choice(int(np.prod(shape)), size=12, replace=False):
        idx = np.unravel_index(flat, shape)
        # choose h so that base +- h are exactly representable in fp32
        hp = float(np.float32(base[idx] + h)) - base[idx]
        hm = base[idx] - float(np.float32(base[idx] - h))
        up = base.copy()
        dn = base.copy()
        up[idx] += hp
        dn[idx] -= hm
        fd = (loss(up) - loss(dn)) / (hp + hm)
        assert fd == pytest.approx(grad[idx], rel=1e-5, abs=1e-9)


# ----------------------------------------------------------------- pose gradient

def _pose_problem(seed, mode):
    rng = np.random.default_rng(seed)
    shape = (9, 10, 11)
    spacing = np.array([1.0, 1.1, 0.9], dtype=np.float32)
    vol = rng.uniform(0.0, 0.3, size=shape).astype(np.float32)
    K = W.intrinsics(14.0, 3.1, 2.6)
    poses = W.random_poses(2, 25.0, 40.0, 1.0, seed=seed + 1).astype(np.float64)
    g = rng.normal(size=(2, 6, 7))
    return vol, spacing, K, poses, g


@pytest.mark.parametrize("mode", [BL, RAW])
@pytest.mark.parametrize("seed", [40, 41])
def test_pose_gradient_matches_central_differences(mode, seed):
    """dL/dP of L = sum g I(P) against central differences of the oracle forward
    in fp64 (h = 1e-7 moves samples ~1e-6 voxel, so no sample crosses a voxel
    plane and the difference quotient sees one smooth piece)."""
    vol, spacing, K, poses, g = _pose_problem(seed, mode)
    N = 23
    grad = oracle.pose_gradient(vol, spacing, K, poses, 6, 7, N, mode, g)
    h = 1e-7
    fd = np.zeros_like(grad)
    for v in range(2):
        for r in range(3):
            for c in range(4):
                up, dn = poses.copy(), poses.copy()
                up[v, r, c] += h
                dn[v, r, c] -= h
                Lp = float((g * oracle.forward(vol, spacing, K, up, 6, 7, N, mode)[0]).sum())
                Lm = float((g * oracle.forward(vol, spacing, K, dn, 6, 7, N, mode)[0]).sum())
                fd[v, r, c] = (Lp - Lm) / (2 * h)
    scale = np.abs(fd).max()
    assert scale > 1e-3
    assert np.abs(grad - fd).max() <= 1e-6 * scale, (grad, fd)


def test_pose_gradient_of_constant_box_is_the_chord_derivative():
    """For a constant mu_c volume I = 1 - exp(-mu_c L(P)): the pose gradient is
    g exp(-mu_c L) mu_c dL/dP with the chord L from face intersections and its
    derivative by central differences of that independent chord (no voxels)."""
    mu_c = float(np.float32(0.05))
    shape = (8, 10, 12)
    vol = np.full(shape, mu_c, dtype=np.float32)
    spacing = np.ones(3, dtype=np.float32)
    E = np.array([12.0, 10.0, 8.0])
    K = W.intrinsics(12.0, 2.5, 2.5)
    poses = W.random_poses(1, 30.0, 35.0, 1.0, seed=50).astype(np.float64)
    rng = np.random.default_rng(51)
    g = rng.normal(size=(1, 5, 5))
    grad = oracle.pose_gradient(vol, spacing, K, poses, 5, 5, 17, BL, g)

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
            ref[r, c] = float((g[0] * np.exp(-mu_c * L0) * mu_c * dL).sum())
    assert (L0 > 0).sum() > 10
    assert np.abs(grad[0] - ref).max() <= 1e-6 * np.abs(ref).max()
