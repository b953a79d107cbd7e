"""The C-ABI library loads, exports every symbol include/drr.h declares, and
rejects invalid calls on the host before anything touches a GPU.  Runs without
a GPU: every call here returns from host validation."""
import ctypes
import os
import re

import numpy as np
import pytest

import ct_forward_projection_amd as drr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "drr.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(drr_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = drr.library()
    names = declared_functions()
    assert {"drr_forward", "drr_backward_volume", "drr_workspace_bytes", "drr_status_string",
            "drr_last_error", "drr_abi_version"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.drr_abi_version() == 1


def test_status_strings():
    lib = drr.library()
    for code, text in [(0, b"ok"), (1, b"invalid argument"), (3, b"workspace too small"),
                       (4, b"HIP runtime error"), (99, b"unknown status")]:
        assert lib.drr_status_string(code) == text


def _f(*v):
    return (ctypes.c_float * len(v))(*v)


SP = _f(1.0, 1.0, 1.0)
K = _f(500.0, 0.0, 32.0, 0.0, 500.0, 32.0, 0.0, 0.0, 1.0)
DUMMY = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


def fwd(reuse=False, **kw):
    args = dict(volume=DUMMY, dtype=0, nz=8, ny=8, nx=8, spacing=SP, K=K, poses=DUMMY,
                n_views=1, det_h=4, det_w=4, n_samples=8, mode=0, out=DUMMY, s=None,
                ws=None, ws_bytes=0, stream=None)
    args.update(kw)
    lib = drr.library()
    fn = lib.drr_forward_reuse if reuse else lib.drr_forward
    return fn(args["volume"], args["dtype"], args["nz"], args["ny"], args["nx"],
                           args["spacing"], args["K"], args["poses"], args["n_views"],
                           args["det_h"], args["det_w"], args["n_samples"], args["mode"],
                           args["out"], args["s"], args["ws"], args["ws_bytes"], args["stream"])


def bwd(**kw):
    args = dict(nz=8, ny=8, nx=8, spacing=SP, K=K, poses=DUMMY, n_views=1, det_h=4, det_w=4,
                n_samples=8, mode=0, g=DUMMY, s=DUMMY, grad=DUMMY, ws=None, ws_bytes=0,
                stream=None)
    args.update(kw)
    lib = drr.library()
    return lib.drr_backward_volume(args["nz"], args["ny"], args["nx"], args["spacing"], args["K"],
                                   args["poses"], args["n_views"], args["det_h"], args["det_w"],
                                   args["n_samples"], args["mode"], args["g"], args["s"],
                                   args["grad"], args["ws"], args["ws_bytes"], args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(nz=0), 1), (dict(ny=-3), 1), (dict(nx=20000), 2),
    (dict(nz=2048, ny=2048, nx=1024), 2),
    (dict(n_views=-1), 1), (dict(det_h=-1), 1),
    (dict(n_samples=0), 1), (dict(n_samples=(1 << 24) + 1), 2),
    (dict(mode=2), 1), (dict(dtype=3), 1),
    (dict(volume=None), 1), (dict(poses=None), 1), (dict(out=None), 1),
    (dict(spacing=None), 1), (dict(K=None), 1),
    (dict(spacing=_f(1.0, 0.0, 1.0)), 1), (dict(spacing=_f(1.0, -2.0, 1.0)), 1),
    (dict(spacing=_f(1.0, float("nan"), 1.0)), 1),
    (dict(K=_f(1, 2, 3, 2, 4, 6, 0, 0, 1)), 1),            # singular
    (dict(K=_f(500, 0, 32, 0, float("inf"), 32, 0, 0, 1)), 1),
    (dict(n_views=65536, det_h=256, det_w=256), 2),          # > 2^31 rays
])
def test_forward_rejects_invalid_arguments(kw, status):
    assert fwd(**kw) == status
    assert drr.library().drr_last_error() != b""


@pytest.mark.parametrize("kw,status", [
    (dict(nz=0), 1), (dict(n_samples=0), 1), (dict(mode=-1), 1),
    (dict(grad=None), 1), (dict(g=None), 1), (dict(s=None), 1),  # BL needs line integrals
    (dict(poses=None), 1), (dict(spacing=_f(0.0, 1.0, 1.0)), 1),
])
def test_backward_rejects_invalid_arguments(kw, status):
    assert bwd(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(nz=0), 1), (dict(n_samples=0), 1), (dict(mode=2), 1), (dict(dtype=3), 1),
    (dict(volume=None), 1), (dict(poses=None), 1), (dict(out=None), 1),
    (dict(spacing=_f(1.0, 0.0, 1.0)), 1), (dict(nz=2048, ny=2048, nx=1024), 2),
    (dict(n_views=64, det_h=16, det_w=16), 3),               # the copy's workspace is missing
])
def test_reuse_forward_validates_like_the_forward(kw, status):
    """drr_forward_reuse checks its arguments as drr_forward does (the same
    status for the same call) before anything is enqueued."""
    assert fwd(reuse=True, **kw) == status == fwd(**kw)
    assert drr.library().drr_last_error() != b""
    assert fwd(reuse=True, n_views=0, poses=None, out=None) == 0


def test_reuse_pose_backward_validates_like_the_pose_backward():
    lib = drr.library()
    for fn in (lib.drr_backward_pose, lib.drr_backward_pose_reuse):
        # no workspace, then grad_out NULL, then an unknown dtype
        assert fn(DUMMY, 0, 8, 8, 8, SP, K, DUMMY, 1, 4, 4, 8, 0, DUMMY, DUMMY, None, 0,
                  None) == 3
        assert fn(DUMMY, 0, 8, 8, 8, SP, K, DUMMY, 1, 4, 4, 8, 0, None, DUMMY, DUMMY, 4096,
                  None) == 1
        assert fn(DUMMY, 5, 8, 8, 8, SP, K, DUMMY, 1, 4, 4, 8, 0, DUMMY, DUMMY, DUMMY, 4096,
                  None) == 1


def test_empty_forward_is_a_valid_no_op():
    # nothing to render: returns OK without touching the device
    assert fwd(n_views=0, poses=None, out=None) == 0
    assert fwd(det_h=0) == 0
    assert drr.library().drr_last_error() == b""


def test_workspace_query_is_consistent():
    for args in [(64, 64, 64, 0, 1, 64, 64, 128, 0), (256, 256, 256, 1, 16, 200, 200, 256, 0),
                 (128, 128, 128, 0, 360, 256, 384, 256, 1)]:
        n = drr.drr_workspace_bytes(*args)
        assert n >= 0 and n % 256 == 0


def test_binding_refuses_host_tensors():
    import torch
    with pytest.raises(ValueError):
        drr.drr_forward(torch.zeros(4, 4, 4), [1, 1, 1], torch.eye(3), torch.zeros(1, 3, 4),
                        4, 4, 8)


def test_workspace_too_small_is_rejected_on_the_host():
    # many views that together reuse cells plan the corner-cell relayout, which
    # needs a workspace
    need = drr.drr_workspace_bytes(8, 8, 8, 0, 64, 16, 16, 8, 0)
    assert need >= 9 * 9 * 9 * 32
    assert fwd(n_views=64, det_h=16, det_w=16, n_samples=8, ws=None, ws_bytes=0) == 3
    assert b"workspace" in drr.library().drr_last_error()
    # misaligned workspace
    assert fwd(n_views=64, det_h=16, det_w=16, n_samples=8, ws=ctypes.c_void_p(0x1004),
               ws_bytes=need) == 1
    # one dense view stages its boxes in LDS and needs none; neither does the backward
    assert drr.drr_workspace_bytes(8, 8, 8, 0, 1, 256, 256, 64, 0) == 0
    assert drr.drr_workspace_bytes(8, 8, 8, 0, 1, 256, 256, 64, 1) == 0


def fwd_siddon(**kw):
    args = dict(volume=DUMMY, dtype=0, nz=8, ny=8, nx=8, spacing=SP, K=K, poses=DUMMY,
                n_views=1, det_h=4, det_w=4, mode=0, out=DUMMY, s=None, stream=None)
    args.update(kw)
    return drr.library().drr_forward_siddon(
        args["volume"], args["dtype"], args["nz"], args["ny"], args["nx"], args["spacing"],
        args["K"], args["poses"], args["n_views"], args["det_h"], args["det_w"], args["mode"],
        args["out"], args["s"], args["stream"])


def bwd_siddon(**kw):
    args = dict(nz=8, ny=8, nx=8, spacing=SP, K=K, poses=DUMMY, n_views=1, det_h=4, det_w=4,
                mode=0, g=DUMMY, s=DUMMY, grad=DUMMY, stream=None)
    args.update(kw)
    return drr.library().drr_backward_volume_siddon(
        args["nz"], args["ny"], args["nx"], args["spacing"], args["K"], args["poses"],
        args["n_views"], args["det_h"], args["det_w"], args["mode"], args["g"], args["s"],
        args["grad"], args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(nz=0), 1), (dict(nx=20000), 2), (dict(n_views=-1), 1), (dict(mode=2), 1),
    (dict(dtype=3), 1), (dict(volume=None), 1), (dict(poses=None), 1), (dict(out=None), 1),
    (dict(spacing=_f(1.0, 0.0, 1.0)), 1), (dict(K=_f(1, 2, 3, 2, 4, 6, 0, 0, 1)), 1),
    (dict(n_views=65536, det_h=256, det_w=256), 2),
])
def test_siddon_forward_rejects_invalid_arguments(kw, status):
    assert fwd_siddon(**kw) == status
    assert drr.library().drr_last_error() != b""


@pytest.mark.parametrize("kw,status", [
    (dict(nz=0), 1), (dict(mode=-1), 1), (dict(grad=None), 1), (dict(g=None), 1),
    (dict(s=None), 1), (dict(poses=None), 1), (dict(K=None), 1),
])
def test_siddon_backward_rejects_invalid_arguments(kw, status):
    assert bwd_siddon(**kw) == status
    assert drr.library().drr_last_error() != b""


def test_siddon_empty_calls_are_valid_no_ops():
    assert fwd_siddon(n_views=0, poses=None, out=None) == 0
    assert fwd_siddon(det_w=0) == 0
    assert drr.library().drr_last_error() == b""


# ----------------------------------------------------------------- drr_render

def render_call(**kw):
    args = dict(volume=DUMMY, dtype=0, B=1, C=1, nz=8, ny=8, nx=8, spacing=SP, K=K, poses=DUMMY,
                n_views=2, det_h=4, det_w=4, n_samples=8, mode=0, f=1.0, clip=0, margin=30.0,
                xp=None, yp=None, knots=0, out=DUMMY, aux=None, ws=None, ws_bytes=0, stream=None)
    args.update(kw)
    a = args
    return drr.library().drr_render(a["volume"], a["dtype"], a["B"], a["C"], a["nz"], a["ny"],
                                    a["nx"], a["spacing"], a["K"], a["poses"], a["n_views"],
                                    a["det_h"], a["det_w"], a["n_samples"], a["mode"], a["f"],
                                    a["clip"], a["margin"], a["xp"], a["yp"], a["knots"],
                                    a["out"], a["aux"], a["ws"], a["ws_bytes"], a["stream"])


def render_bwd_call(**kw):
    args = dict(volume=DUMMY, dtype=0, B=1, C=1, nz=8, ny=8, nx=8, spacing=SP, K=K, poses=DUMMY,
                n_views=2, det_h=4, det_w=4, n_samples=8, mode=1, f=1.0, clip=0, margin=30.0,
                xp=None, yp=None, knots=0, g=DUMMY, out=DUMMY, aux=DUMMY, grad=DUMMY, ws=None,
                ws_bytes=0, stream=None)
    args.update(kw)
    a = args
    return drr.library().drr_render_backward_volume(
        a["volume"], a["dtype"], a["B"], a["C"], a["nz"], a["ny"], a["nx"], a["spacing"], a["K"],
        a["poses"], a["n_views"], a["det_h"], a["det_w"], a["n_samples"], a["mode"], a["f"],
        a["clip"], a["margin"], a["xp"], a["yp"], a["knots"], a["g"], a["out"], a["aux"],
        a["grad"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), 1), (dict(C=0), 1), (dict(B=3), 1), (dict(mode=3), 1), (dict(clip=2), 1),
    (dict(f=float("nan")), 1), (dict(margin=float("inf")), 1), (dict(dtype=2), 1),
    (dict(volume=None), 1), (dict(out=None), 1), (dict(poses=None), 1),
    (dict(xp=_f(0.0, 1.0), yp=None, knots=2), 1),
    (dict(xp=_f(0.0, 0.0), yp=_f(0.0, 1.0), knots=2), 1),
    (dict(xp=_f(0.0), yp=_f(0.0), knots=1), 1),
    (dict(xp=_f(0.0, float("nan")), yp=_f(0.0, 1.0), knots=2), 1),
    (dict(C=65, xp=_f(*range(130)), yp=_f(*range(130)), knots=2), 2),
    (dict(B=300, C=300, n_views=300), 2),
    (dict(clip=1), 3),                      # the near/far mode always needs a padded copy
])
def test_render_rejects_invalid_arguments(kw, status):
    assert render_call(**kw) == status
    assert drr.library().drr_last_error() != b""


@pytest.mark.parametrize("kw,status", [
    (dict(mode=0, aux=None), 1),            # Beer-Lambert needs the optical depth
    (dict(mode=2, out=None), 1),            # compositing needs the forward image
    (dict(mode=2, volume=None), 1),         # ... and the volume
    (dict(volume=None, xp=_f(0.0, 1.0), yp=_f(0.0, 2.0), knots=2), 1),
    (dict(grad=None), 1), (dict(g=None), 1), (dict(B=2, n_views=3), 1),
    (dict(mode=2, xp=_f(0.0, 1.0), yp=_f(0.0, 2.0), knots=2), 3),   # mapped fp32 copy
])
def test_render_backward_rejects_invalid_arguments(kw, status):
    assert render_bwd_call(**kw) == status


def test_render_empty_call_and_workspace_queries():
    assert render_call(n_views=0) == 0
    assert render_call(det_h=0, out=None) == 0
    lib = drr.library()
    q = lib.drr_render_workspace_bytes
    # near/far: a zero-padded copy of every channel-volume, 256-byte multiples --
    # z-pairs with a border of zeros ((nx + 2) x (ny + 2) x (nz + 1) pairs) ...
    zpad = ((10 * 10 * 9 * 2 * 4 + 255) // 256) * 256
    assert q(2, 3, 8, 8, 8, 0, 4, 4, 4, 8, 0, 1, 0, 0) == 6 * zpad
    # ... or, from 16 samples per cell, zero-padded corner cells
    cells = ((9 * 9 * 9 * 8 * 4 + 255) // 256) * 256
    assert q(1, 1, 8, 8, 8, 0, 1, 32, 32, 16, 0, 1, 0, 0) == cells
    # a transfer function and few samples per cell: the mapped fp32 volumes
    assert q(1, 2, 8, 8, 8, 1, 1, 4, 4, 8, 0, 0, 3, 0) == 2 * 2048
    # about one sample per cell or more, but under 16: z-pair copies of
    # (nz - 1) x ny x nx pairs, of the input dtype or mapped fp32
    assert q(1, 1, 8, 8, 8, 0, 4, 8, 8, 16, 0, 0, 0, 0) == 8 * 8 * 7 * 2 * 4
    assert q(1, 1, 8, 8, 8, 1, 4, 8, 8, 16, 0, 0, 0, 0) == 8 * 8 * 7 * 2 * 2
    assert q(2, 1, 8, 8, 8, 1, 8, 8, 8, 16, 0, 0, 3, 0) == 2 * 8 * 8 * 7 * 2 * 4
    # a volume one voxel deep has no z-pairs: the volume itself
    assert q(1, 1, 1, 8, 8, 0, 4, 8, 8, 4, 0, 0, 0, 0) == 0
    # compositing backward: under one sample per cell the mapped fp32 volumes with
    # a transfer function (else none); from one per cell a z-pair copy for its
    # coefficient passes, zero-padded in the near/far mode; other modes none.
    # After a copy, 8 bytes per channel-volume (in 256) for its largest value
    bound = 256
    assert q(1, 2, 8, 8, 8, 0, 1, 4, 4, 8, 2, 0, 3, 1) == 2 * 2048 + bound
    assert q(1, 2, 8, 8, 8, 0, 1, 4, 4, 8, 2, 0, 0, 1) == 0
    # Beer-Lambert / line integral with the box clip, views sparse against the
    # voxels (under 4 samples per cell from one view): the brick-owned backward's
    # ray records (64 bytes per ray of each (view, channel) pair), one float
    # per 256 rays and 48 bytes per view (its fp32 projection),
    # each rounded to 256 bytes; denser views and near/far: none
    rnd = lambda b: (b + 255) // 256 * 256
    assert q(1, 2, 8, 8, 8, 0, 1, 4, 4, 8, 0, 0, 3, 1) == rnd(2 * 16 * 64) + rnd(4) + rnd(48)
    assert q(2, 1, 8, 8, 8, 0, 6, 40, 40, 1, 1, 0, 0, 1) == rnd(6 * 1600 * 64) + rnd(38 * 4) + rnd(6 * 48)
    assert q(1, 1, 8, 8, 8, 0, 1, 32, 32, 16, 0, 0, 0, 1) == 0      # 22 samples per view-cell
    assert q(1, 1, 8, 8, 8, 0, 1, 4, 4, 8, 0, 1, 0, 1) == 0         # near/far
    assert drr.drr_workspace_bytes(8, 8, 8, 0, 3, 5, 7, 8, 1) == rnd(105 * 64) + rnd(4) + rnd(3 * 48)
    assert q(1, 1, 8, 8, 8, 0, 4, 8, 8, 16, 2, 0, 0, 1) == 8 * 8 * 7 * 2 * 4 + bound
    assert q(1, 1, 8, 8, 8, 1, 4, 8, 8, 16, 2, 0, 0, 1) == 8 * 8 * 7 * 2 * 2 + bound
    assert q(1, 1, 8, 8, 8, 1, 4, 8, 8, 16, 2, 0, 3, 1) == 8 * 8 * 7 * 2 * 4 + bound
    assert q(1, 1, 8, 8, 8, 0, 4, 8, 8, 16, 2, 1, 0, 1) == \
        ((10 * 10 * 9 * 2 * 4 + 255) // 256) * 256 + bound
    # 33 channel-volumes need 264 bytes of bounds: two 256-byte blocks
    assert q(1, 33, 8, 8, 8, 0, 4, 8, 8, 16, 2, 0, 0, 1) == 33 * 8 * 8 * 7 * 2 * 4 + 512
    assert q(1, 1, 8, 8, 8, 0, 4, 8, 8, 16, 0, 1, 0, 1) == 0
    assert q(2, 1, 8, 8, 8, 0, 3, 4, 4, 8, 0, 0, 0, 0) == 0     # views not a multiple
    # the single-volume call's plan is drr_forward's
    for args in [(64, 64, 64, 0, 1, 1024, 1024, 512), (64, 64, 64, 0, 1, 16, 16, 8)]:
        nz, ny, nx, dt, V, H, Wd, N = args
        assert q(1, 1, nz, ny, nx, dt, V, H, Wd, N, 0, 0, 0, 0) == \
            lib.drr_workspace_bytes(nz, ny, nx, dt, V, H, Wd, N, 0)


# ----------------------------------------------------------------- cameras

def test_intrinsics_from_fov_on_the_host():
    from oracle import camera
    for fov, H, Wd in [(20.0, 1024, 1024), (35.5, 200, 320)]:
        K = drr.drr_intrinsics_from_fov(fov, H, Wd).double().numpy()
        assert np.allclose(K, camera.intrinsics_from_fov(fov, H, Wd), rtol=1e-6)
    for bad in [(0.0, 10, 10), (180.0, 10, 10), (20.0, 0, 10), (float("nan"), 10, 10)]:
        with pytest.raises(drr.DRRError):
            drr.drr_intrinsics_from_fov(*bad)


RAS = _f(1.0, 0.0, 0.0, 3.0, 0.0, 0.0, 2.0, 1.0, 0.0, -0.5, 0.0, 2.0, 0.0, 0.0, 0.0, 1.0)


@pytest.mark.parametrize("ras,status", [
    (RAS, 0),
    (_f(1.0, 0.5, 0.0, 0.0, 0.0, 1.0, 0.0, 0.0, 0.0, 0.0, 1.0, 0.0, 0.0, 0.0, 0.0, 1.0), 1),
    (_f(1.0, 0.0, 0.0, 0.0, 0.0, 1.0, 0.0, 0.0, 0.0, 0.0, 1.0, 0.0, 0.0, 0.0, 1.0, 1.0), 1),
    (_f(0.0, 0.0, 0.0, 0.0, 0.0, 1.0, 0.0, 0.0, 0.0, 0.0, 1.0, 0.0, 0.0, 0.0, 0.0, 1.0), 1),
    (None, 1),
])
def test_view_matrix_conversion_validates_ras2ijk(ras, status):
    """A scaled rotation is accepted (empty call), skewed or projective affines
    are refused; the voxel sizes come out of the row norms."""
    lib = drr.library()
    sp = (ctypes.c_float * 3)()
    assert lib.drr_poses_from_view_matrices(None, 0, ras, 4, 5, 6, None, sp, None) == status
    if status == 0:
        assert list(sp) == pytest.approx([1.0, 0.5, 2.0])
    assert lib.drr_view_matrices_backward(None, 0, ras, 4, 5, 6, None, None, None) == status
    assert lib.drr_poses_from_view_matrices(None, 1, RAS, 4, 5, 6, None, None, None) == 1


def test_poisson_surrogate_validates_on_the_host():
    lib = drr.library()
    assert lib.drr_poisson_surrogate(None, None, 0, 100.0, None, None) == 0
    assert lib.drr_poisson_surrogate(None, None, -1, 100.0, None, None) == 1
    assert lib.drr_poisson_surrogate(DUMMY, DUMMY, 4, 0.0, DUMMY, None) == 1
    assert lib.drr_poisson_surrogate(DUMMY, DUMMY, 4, float("inf"), DUMMY, None) == 1
    assert lib.drr_poisson_surrogate(DUMMY, None, 4, 10.0, DUMMY, None) == 1
    assert lib.drr_poisson_surrogate_backward(DUMMY, DUMMY, 4, 10.0, None, DUMMY, None) == 1
    assert lib.drr_poisson_surrogate_backward(None, None, 0, 10.0, None, None, None) == 0


def fwd_no_alloc(**kw):
    args = dict(volume=DUMMY, dtype=0, nz=8, ny=8, nx=8, spacing=SP, K=K, poses=DUMMY,
                n_views=1, det_h=4, det_w=4, n_samples=8, mode=0, out=DUMMY, s=None,
                stream=None)
    args.update(kw)
    return drr.library().drr_forward_no_alloc(
        args["volume"], args["dtype"], args["nz"], args["ny"], args["nx"], args["spacing"],
        args["K"], args["poses"], args["n_views"], args["det_h"], args["det_w"],
        args["n_samples"], args["mode"], args["out"], args["s"], args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(nz=0), 1), (dict(n_samples=0), 1), (dict(mode=2), 1), (dict(dtype=3), 1),
    (dict(volume=None), 1), (dict(poses=None), 1), (dict(out=None), 1),
    (dict(spacing=_f(1.0, 0.0, 1.0)), 1), (dict(nz=2048, ny=2048, nx=1024), 2),
])
def test_no_alloc_forward_rejects_invalid_arguments(kw, status):
    assert fwd_no_alloc(**kw) == status
    assert drr.library().drr_last_error() != b""


def test_no_alloc_forward_rejects_plans_beyond_its_scratch_on_the_host():
    """A read plan whose copy exceeds the fixed scratch is refused before any
    HIP call (64 views of 256^2 x 256 samples put 8 samples per cell of a 512^3
    fp32 volume: the z-pair copy, about 1 GiB)."""
    need = drr.drr_workspace_bytes(512, 512, 512, 0, 64, 256, 256, 256, 0)
    assert need > drr.NO_ALLOC_SCRATCH_BYTES
    assert fwd_no_alloc(nz=512, ny=512, nx=512, n_views=64, det_h=256, det_w=256,
                        n_samples=256) == 2
    assert b"scratch" in drr.library().drr_last_error()
    # an empty call within the limit is a valid no-op without a device
    assert fwd_no_alloc(n_views=0, poses=None, out=None) == 0


def test_no_alloc_scratch_size_matches_the_header():
    text = open(HEADER).read()
    m = re.search(r"#define DRR_NO_ALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m is not None
    assert int(m.group(1)) << int(m.group(2)) == drr.NO_ALLOC_SCRATCH_BYTES
