"""CPU oracle for cone-beam DRR ray casting -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and its
Python binding) never imports, links or calls it, and this package never
imports the product: the two share only the seeded input arrays from
``workloads``.

The arithmetic lives in ``drr_oracle.c`` (plain C, scalar fp64, OpenMP over
rays); this module only builds it with gcc, loads it with ctypes and converts
arrays.  Inputs the HIP side receives in fp32 (spacing, K, poses) are widened
exactly to fp64 here; the volume stays fp32 and is widened per read.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "drr_oracle.c")
LIBRARY = os.path.join(HERE, "libdrr_oracle.so")

BEER_LAMBERT = 0
LINE_INTEGRAL = 1
ALPHA_COMPOSITE = 2
CLIP_BOX = 0
CLIP_NEAR_FAR = 1

_lib = None


def build(verbose: bool = False) -> str:
    """Compile the oracle with gcc: -O2, OpenMP, no fast-math, no FMA contraction."""
    cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-Wall", "-Wextra", "-o", LIBRARY + ".tmp", SOURCE, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIBRARY + ".tmp", LIBRARY)
    return LIBRARY


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIBRARY) or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE):
        build()
    lib = ctypes.CDLL(LIBRARY)
    P = ctypes.c_void_p
    I = ctypes.c_int
    lib.oracle_forward.argtypes = [P, I, I, I, P, P, P, I, I, I, I, I, P, P, I]
    lib.oracle_forward.restype = I
    lib.oracle_adjoint.argtypes = [P, I, I, I, P, P, P, I, I, I, I, I, P, P, I, ctypes.c_longlong]
    lib.oracle_adjoint.restype = I
    lib.oracle_ray.argtypes = [P, P, P, I, I, P]
    lib.oracle_ray.restype = I
    lib.oracle_forward_spheres.argtypes = [P, I, P, P, P, I, I, I, I, I, P, I]
    lib.oracle_forward_spheres.restype = I
    lib.oracle_exact_line_integral.argtypes = [P, I, I, I, P, P, P, I, I, I, P, I]
    lib.oracle_exact_line_integral.restype = I
    lib.oracle_chords.argtypes = [P, P, P, I, I, I, P, I]
    lib.oracle_chords.restype = I
    lib.oracle_pose_gradient.argtypes = [P, I, I, I, P, P, P, I, I, I, I, I, P, P, I]
    lib.oracle_pose_gradient.restype = I
    lib.oracle_siddon_forward.argtypes = [P, I, I, I, P, P, P, I, I, I, I, P, P, I]
    lib.oracle_siddon_forward.restype = I
    lib.oracle_siddon_adjoint.argtypes = [P, I, I, I, P, P, P, I, I, I, I, P, P, I,
                                          ctypes.c_longlong]
    lib.oracle_siddon_adjoint.restype = I
    D = ctypes.c_double
    lib.oracle_render.argtypes = [P, I, I, I, I, I, P, P, P, I, I, I, I, I, D, I, D, P, P, I, P,
                                  P, I]
    lib.oracle_render.restype = I
    lib.oracle_render_adjoint.argtypes = [P, I, I, I, I, I, P, P, P, I, I, I, I, I, D, I, D, P,
                                          P, I, P, P, I, ctypes.c_longlong]
    lib.oracle_render_adjoint.restype = I
    lib.oracle_render_pose_gradient.argtypes = [P, I, I, I, I, I, P, P, P, I, I, I, I, I, D, I,
                                                D, P, P, I, P, P, I]
    lib.oracle_render_pose_gradient.restype = I
    lib.oracle_view_range.argtypes = [P, P, D, P]
    lib.oracle_view_range.restype = None
    lib.oracle_poisson_surrogate.argtypes = [P, P, ctypes.c_long, D, P, P, P]
    lib.oracle_poisson_surrogate.restype = None
    lib.oracle_max_threads.restype = I
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _f64(a) -> np.ndarray:
    """fp32 inputs (what the HIP side receives) widen exactly; fp64 arrays pass
    through unchanged (finite-difference pins perturb below fp32 resolution)."""
    a = np.asarray(a)
    if a.dtype == np.float64:
        return np.ascontiguousarray(a)
    return np.ascontiguousarray(a.astype(np.float32).astype(np.float64))


def _threads(n: Optional[int]) -> int:
    """Threads for a call: ``n``, else OMP_NUM_THREADS when set, else the CPUs
    this process may run on."""
    if n:
        return int(n)
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        return int(env)
    try:
        return len(os.sched_getaffinity(0)) or 1
    except (AttributeError, OSError):
        return os.cpu_count() or 1


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def forward(volume: np.ndarray, spacing, K, poses, det_h: int, det_w: int, n_samples: int,
            mode: int, n_threads: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Forward DRR.  Returns (image, line_integral), both float64 (V, H, W)."""
    lib = _load()
    vol = np.ascontiguousarray(volume, dtype=np.float32)
    nz, ny, nx = vol.shape
    sp, Kd, Pd = _f64(spacing), _f64(K), _f64(poses).reshape(-1, 12)
    V = Pd.shape[0]
    out = np.zeros((V, det_h, det_w), dtype=np.float64)
    s = np.zeros((V, det_h, det_w), dtype=np.float64)
    rc = lib.oracle_forward(_ptr(vol), nz, ny, nx, _ptr(sp), _ptr(Kd), _ptr(Pd), V, det_h, det_w,
                            n_samples, mode, _ptr(out), _ptr(s), _threads(n_threads))
    if rc != 0:
        raise ValueError("oracle_forward: invalid arguments")
    return out, s


def adjoint(volume: Optional[np.ndarray], shape, spacing, K, poses, det_h: int, det_w: int,
            n_samples: int, mode: int, grad_out: np.ndarray, n_threads: Optional[int] = None,
            max_buffer_bytes: int = 4 << 30) -> Tuple[np.ndarray, int]:
    """Volume gradient for upstream dL/dI = grad_out.  ``volume`` is required for
    Beer-Lambert (it fixes exp(-s)) and ignored for the line integral.
    Returns (grad float64 (nz, ny, nx), threads used)."""
    lib = _load()
    nz, ny, nx = (int(x) for x in shape)
    vol = None if volume is None else np.ascontiguousarray(volume, dtype=np.float32)
    sp, Kd, Pd = _f64(spacing), _f64(K), _f64(poses).reshape(-1, 12)
    V = Pd.shape[0]
    g = np.ascontiguousarray(grad_out, dtype=np.float64).reshape(V, det_h, det_w)
    grad = np.zeros((nz, ny, nx), dtype=np.float64)
    rc = lib.oracle_adjoint(None if vol is None else _ptr(vol), nz, ny, nx, _ptr(sp), _ptr(Kd),
                            _ptr(Pd), V, det_h, det_w, n_samples, mode, _ptr(g), _ptr(grad),
                            _threads(n_threads), int(max_buffer_bytes))
    if rc < 1:
        raise ValueError("oracle_adjoint: invalid arguments or out of memory")
    return grad, int(rc)


def ray(K, pose, extent, r: int, c: int):
    """(hit, C, d, t0, t1) of the ray through pixel (r, c)."""
    lib = _load()
    out = np.zeros(8, dtype=np.float64)
    hit = lib.oracle_ray(_ptr(_f64(K)), _ptr(_f64(pose).reshape(12)),
                         _ptr(np.ascontiguousarray(extent, dtype=np.float64)), r, c, _ptr(out))
    if hit < 0:
        raise ValueError("singular K")
    return bool(hit), out[0:3].copy(), out[3:6].copy(), float(out[6]), float(out[7])


def chords(extent, K, poses, det_h: int, det_w: int, n_threads: Optional[int] = None):
    """Clipped chord length t1 - t0 of every ray, 0 where the ray misses the box."""
    lib = _load()
    Kd, Pd = _f64(K), _f64(poses).reshape(-1, 12)
    V = Pd.shape[0]
    out = np.zeros((V, det_h, det_w), dtype=np.float64)
    rc = lib.oracle_chords(_ptr(np.ascontiguousarray(extent, dtype=np.float64)), _ptr(Kd),
                           _ptr(Pd), V, det_h, det_w, _ptr(out), _threads(n_threads))
    if rc != 0:
        raise ValueError("oracle_chords: invalid arguments")
    return out


def chords_workload(w, n_threads: Optional[int] = None):
    sp = np.asarray(w.spacing, dtype=np.float32).astype(np.float64)
    nz, ny, nx = w.volume.shape
    extent = np.array([nx * sp[0], ny * sp[1], nz * sp[2]])
    return chords(extent, w.K, w.poses, w.det_h, w.det_w, n_threads)


def forward_spheres(spheres, extent, K, poses, det_h: int, det_w: int, n_samples: int,
                    mode: int, n_threads: Optional[int] = None) -> np.ndarray:
    """Forward through an analytic density: a sum of uniform balls given as rows
    (cx, cy, cz, radius, mu); the box ``extent`` (centred at 0) still clips."""
    lib = _load()
    sph = np.ascontiguousarray(np.asarray(spheres, dtype=np.float64).reshape(-1, 5))
    Kd, Pd = _f64(K), _f64(poses).reshape(-1, 12)
    V = Pd.shape[0]
    out = np.zeros((V, det_h, det_w), dtype=np.float64)
    rc = lib.oracle_forward_spheres(_ptr(sph), sph.shape[0],
                                    _ptr(np.ascontiguousarray(extent, dtype=np.float64)),
                                    _ptr(Kd), _ptr(Pd), V, det_h, det_w, n_samples, mode,
                                    _ptr(out), _threads(n_threads))
    if rc != 0:
        raise ValueError("oracle_forward_spheres: invalid arguments")
    return out


def exact_line_integral(volume: np.ndarray, spacing, K, poses, det_h: int, det_w: int,
                        n_threads: Optional[int] = None) -> np.ndarray:
    """Exact integral of the clamped trilinear field along each clipped ray."""
    lib = _load()
    vol = np.ascontiguousarray(volume, dtype=np.float32)
    nz, ny, nx = vol.shape
    sp, Kd, Pd = _f64(spacing), _f64(K), _f64(poses).reshape(-1, 12)
    V = Pd.shape[0]
    s = np.zeros((V, det_h, det_w), dtype=np.float64)
    rc = lib.oracle_exact_line_integral(_ptr(vol), nz, ny, nx, _ptr(sp), _ptr(Kd), _ptr(Pd), V,
                                        det_h, det_w, _ptr(s), _threads(n_threads))
    if rc != 0:
        raise ValueError("oracle_exact_line_integral: invalid arguments")
    return s


def pose_gradient(volume: np.ndarray, spacing, K, poses, det_h: int, det_w: int, n_samples: int,
                  mode: int, grad_out: np.ndarray, n_threads: Optional[int] = None) -> np.ndarray:
    """dL/dP for L = sum g I, per view: float64 (V, 3, 4) over the [R | t] entries."""
    lib = _load()
    vol = np.ascontiguousarray(volume, dtype=np.float32)
    nz, ny, nx = vol.shape
    sp, Kd, Pd = _f64(spacing), _f64(K), _f64(poses).reshape(-1, 12)
    V = Pd.shape[0]
    g = np.ascontiguousarray(grad_out, dtype=np.float64).reshape(V, det_h, det_w)
    out = np.zeros((V, 12), dtype=np.float64)
    rc = lib.oracle_pose_gradient(_ptr(vol), nz, ny, nx, _ptr(sp), _ptr(Kd), _ptr(Pd), V, det_h,
                                  det_w, n_samples, mode, _ptr(g), _ptr(out), _threads(n_threads))
    if rc != 0:
        raise ValueError("oracle_pose_gradient: invalid arguments")
    return out.reshape(V, 3, 4)


def siddon_forward(volume: np.ndarray, spacing, K, poses, det_h: int, det_w: int, mode: int,
                   n_threads: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Forward DRR in the cell-constant (Siddon) model: s = sum_v mu_v l_v.
    Returns (image, line_integral), both float64 (V, H, W)."""
    lib = _load()
    vol = np.ascontiguousarray(volume, dtype=np.float32)
    nz, ny, nx = vol.shape
    sp, Kd, Pd = _f64(spacing), _f64(K), _f64(poses).reshape(-1, 12)
    V = Pd.shape[0]
    out = np.zeros((V, det_h, det_w), dtype=np.float64)
    s = np.zeros((V, det_h, det_w), dtype=np.float64)
    rc = lib.oracle_siddon_forward(_ptr(vol), nz, ny, nx, _ptr(sp), _ptr(Kd), _ptr(Pd), V,
                                   det_h, det_w, mode, _ptr(out), _ptr(s), _threads(n_threads))
    if rc != 0:
        raise ValueError("oracle_siddon_forward: invalid arguments or out of memory")
    return out, s


def siddon_adjoint(volume: Optional[np.ndarray], shape, spacing, K, poses, det_h: int,
                   det_w: int, mode: int, grad_out: np.ndarray, n_threads: Optional[int] = None,
                   max_buffer_bytes: int = 4 << 30) -> Tuple[np.ndarray, int]:
    """Matched adjoint of ``siddon_forward`` (volume gradient for dL/dI =
    grad_out).  Returns (grad float64 (nz, ny, nx), threads used)."""
    lib = _load()
    nz, ny, nx = (int(x) for x in shape)
    vol = None if volume is None else np.ascontiguousarray(volume, dtype=np.float32)
    sp, Kd, Pd = _f64(spacing), _f64(K), _f64(poses).reshape(-1, 12)
    V = Pd.shape[0]
    g = np.ascontiguousarray(grad_out, dtype=np.float64).reshape(V, det_h, det_w)
    grad = np.zeros((nz, ny, nx), dtype=np.float64)
    rc = lib.oracle_siddon_adjoint(None if vol is None else _ptr(vol), nz, ny, nx, _ptr(sp),
                                   _ptr(Kd), _ptr(Pd), V, det_h, det_w, mode, _ptr(g),
                                   _ptr(grad), _threads(n_threads), int(max_buffer_bytes))
    if rc < 1:
        raise ValueError("oracle_siddon_adjoint: invalid arguments or out of memory")
    return grad, int(rc)


def siddon_forward_workload(w, n_threads: Optional[int] = None, use_bf16: bool = False):
    """Convenience: cell-constant forward of a ``workloads.Workload``."""
    vol = w.volume_bf16_as_f32() if use_bf16 else w.volume
    return siddon_forward(vol, w.spacing, w.K, w.poses, w.det_h, w.det_w, w.mode, n_threads)


def siddon_adjoint_workload(w, grad_out=None, n_threads: Optional[int] = None,
                            max_buffer_bytes: int = 4 << 30):
    """Convenience: cell-constant volume gradient of a ``workloads.Workload``."""
    g = w.grad_out if grad_out is None else grad_out
    return siddon_adjoint(w.volume, w.volume.shape, w.spacing, w.K, w.poses, w.det_h, w.det_w,
                          w.mode, g, n_threads, max_buffer_bytes)


def forward_workload(w, n_threads: Optional[int] = None, use_bf16: bool = False):
    """Convenience: forward of a ``workloads.Workload``."""
    vol = w.volume_bf16_as_f32() if use_bf16 else w.volume
    return forward(vol, w.spacing, w.K, w.poses, w.det_h, w.det_w, w.n_samples, w.mode, n_threads)


def adjoint_workload(w, grad_out=None, n_threads: Optional[int] = None,
                     max_buffer_bytes: int = 4 << 30):
    """Convenience: volume gradient of a ``workloads.Workload``."""
    g = w.grad_out if grad_out is None else grad_out
    return adjoint(w.volume, w.volume.shape, w.spacing, w.K, w.poses, w.det_h, w.det_w,
                   w.n_samples, w.mode, g, n_threads, max_buffer_bytes)


def _render_args(volume, poses, transfer):
    vol = np.ascontiguousarray(volume, dtype=np.float32)
    if vol.ndim == 3:
        vol = vol[None, None]
    if vol.ndim != 5:
        raise ValueError("volume must be (nz, ny, nx) or (B, C, nz, ny, nx)")
    Pd = _f64(poses).reshape(-1, 12)
    if transfer is None:
        return vol, Pd, None, None, 0
    xp = np.ascontiguousarray(np.asarray(transfer[0], dtype=np.float64).reshape(vol.shape[1], -1))
    yp = np.ascontiguousarray(np.asarray(transfer[1], dtype=np.float64).reshape(xp.shape))
    return vol, Pd, xp, yp, xp.shape[1]


def render(volume: np.ndarray, spacing, K, poses, det_h: int, det_w: int, n_samples: int,
           mode: int, density_factor: float = 1.0, clip: int = CLIP_BOX, margin: float = 30.0,
           transfer=None, n_threads: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """flashdrr-style render of ``volume`` (B, C, nz, ny, nx) (or (nz, ny, nx)):
    view v of ``poses`` (V = B * views_per_vol) renders volume v // views_per_vol.
    ``transfer`` = (xp, yp), each (C, K): a per-channel piecewise-linear map
    applied to the voxels first.  Returns (image, optical depth), float64
    (V, C, H, W)."""
    lib = _load()
    vol, Pd, xp, yp, nk = _render_args(volume, poses, transfer)
    B, C, nz, ny, nx = vol.shape
    V = Pd.shape[0]
    out = np.zeros((V, C, det_h, det_w), dtype=np.float64)
    tau = np.zeros_like(out)
    rc = lib.oracle_render(_ptr(vol), B, C, nz, ny, nx, _ptr(_f64(spacing)), _ptr(_f64(K)),
                           _ptr(Pd), V, det_h, det_w, n_samples, mode, float(density_factor),
                           clip, float(margin), None if xp is None else _ptr(xp),
                           None if yp is None else _ptr(yp), nk, _ptr(out), _ptr(tau),
                           _threads(n_threads))
    if rc != 0:
        raise ValueError("oracle_render: invalid arguments or out of memory")
    return out, tau


def render_adjoint(volume: np.ndarray, spacing, K, poses, det_h: int, det_w: int,
                   n_samples: int, mode: int, grad_out: np.ndarray, density_factor: float = 1.0,
                   clip: int = CLIP_BOX, margin: float = 30.0, transfer=None,
                   n_threads: Optional[int] = None, max_buffer_bytes: int = 4 << 30) -> np.ndarray:
    """Gradient of sum(grad_out * render(volume)) with respect to ``volume``:
    float64 of the volume's shape (B, C, nz, ny, nx) (or (nz, ny, nx))."""
    lib = _load()
    vol, Pd, xp, yp, nk = _render_args(volume, poses, transfer)
    B, C, nz, ny, nx = vol.shape
    V = Pd.shape[0]
    g = np.ascontiguousarray(grad_out, dtype=np.float64).reshape(V, C, det_h, det_w)
    grad = np.zeros(vol.shape, dtype=np.float64)
    rc = lib.oracle_render_adjoint(_ptr(vol), B, C, nz, ny, nx, _ptr(_f64(spacing)),
                                   _ptr(_f64(K)), _ptr(Pd), V, det_h, det_w, n_samples, mode,
                                   float(density_factor), clip, float(margin),
                                   None if xp is None else _ptr(xp),
                                   None if yp is None else _ptr(yp), nk, _ptr(g), _ptr(grad),
                                   _threads(n_threads), int(max_buffer_bytes))
    if rc < 1:
        raise ValueError("oracle_render_adjoint: invalid arguments or out of memory")
    return grad.reshape(np.shape(volume))


def view_range(extent, pose, margin: float):
    """(near, far) of the near/far clipping mode for one view."""
    out = np.zeros(2, dtype=np.float64)
    _load().oracle_view_range(_ptr(np.ascontiguousarray(extent, dtype=np.float64)),
                              _ptr(_f64(pose).reshape(12)), float(margin), _ptr(out))
    return float(out[0]), float(out[1])


def poisson_surrogate(transmission, noise, i0: float, grad_out=None):
    """flashdrr apply_poisson with the standard-normal draws given: returns the
    noisy, clamped transmission (float64), and with ``grad_out`` also the
    gradient with respect to the transmission."""
    lib = _load()
    T = _f64(transmission)
    z = _f64(noise)
    out = np.zeros(T.shape, dtype=np.float64)
    g = None if grad_out is None else _f64(grad_out)
    grad = None if grad_out is None else np.zeros(T.shape, dtype=np.float64)
    lib.oracle_poisson_surrogate(_ptr(T), _ptr(z), T.size, float(i0), _ptr(out),
                                 None if g is None else _ptr(g),
                                 None if grad is None else _ptr(grad))
    return out if grad is None else (out, grad)


def render_pose_gradient(volume, spacing, K, poses, det_h: int, det_w: int, n_samples: int,
                         mode: int, grad_out, density_factor: float = 1.0, transfer=None,
                         clip: int = CLIP_BOX, margin: float = 30.0,
                         n_threads: Optional[int] = None) -> np.ndarray:
    """dL/dP (V, 3, 4) for L = sum(grad_out * render(...)) in any mode
    (Beer-Lambert, line integral, alpha compositing) and either clip: forward-mode
    differentiation of ``render`` per pose entry (``oracle_render_pose_gradient``),
    each view's channels summed."""
    lib = _load()
    vol, Pd, xp, yp, nk = _render_args(volume, poses, transfer)
    B, C, nz, ny, nx = vol.shape
    V = Pd.shape[0]
    g = np.ascontiguousarray(grad_out, dtype=np.float64).reshape(V, C, det_h, det_w)
    out = np.zeros((V, 12), dtype=np.float64)
    rc = lib.oracle_render_pose_gradient(_ptr(vol), B, C, nz, ny, nx, _ptr(_f64(spacing)),
                                         _ptr(_f64(K)), _ptr(Pd), V, det_h, det_w, n_samples,
                                         mode, float(density_factor), clip, float(margin),
                                         None if xp is None else _ptr(xp),
                                         None if yp is None else _ptr(yp), nk, _ptr(g),
                                         _ptr(out), _threads(n_threads))
    if rc != 0:
        raise ValueError("oracle_render_pose_gradient: invalid arguments or out of memory")
    return out.reshape(V, 3, 4)
