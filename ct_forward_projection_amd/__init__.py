"""Differentiable cone-beam DRR ray casting on AMD Instinct MI355X (gfx950).

A thin Python binding over the C ABI of ``libdrr.so`` (``include/drr.h``): it
only marshals arguments -- torch tensors provide device memory and the current
HIP stream -- and every step of the path runs in the library's HIP kernels.
There is no CPU or PyTorch fallback: if the library is not built, or a tensor
is not on a GPU, the call raises.

Functions carry the C names (``drr_forward``, ``drr_forward_no_alloc``,
``drr_backward_volume``,
``drr_backward_pose``, ``drr_forward_siddon``, ``drr_backward_volume_siddon``,
``drr_render``, ``drr_render_backward_volume``, ``drr_workspace_bytes``,
``drr_render_workspace_bytes``, ``drr_intrinsics_from_fov``,
``drr_poses_from_view_matrices``, ``drr_view_matrices_backward``);
``render_view_matrices`` renders from flashdrr's VTK view matrices, ras2ijk and
fov with gradients to the volume and the view matrices; ``raycast`` wraps the flashdrr front end
(volume and channel batches, density factor, alpha compositing, transfer
function, near/far clipping) with autograd to the volume; ``render`` wraps the trilinear model as a
``torch.autograd.Function`` (flashdrr ``VolumeRaycaster`` style: gradients flow
to the volume and to the view poses), ``render_siddon`` the cell-constant model,
and ``project`` / ``backproject`` (``project_siddon`` / ``backproject_siddon``)
give diffct's A and A^T in line-integral mode.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import torch

from .build import LIBRARY

F32, BF16 = 0, 1
BEER_LAMBERT, LINE_INTEGRAL, ALPHA_COMPOSITE = 0, 1, 2
CLIP_BOX, CLIP_NEAR_FAR = 0, 1
NO_ALLOC_SCRATCH_BYTES = 256 << 20       # DRR_NO_ALLOC_SCRATCH_BYTES of include/drr.h
STATUS = {0: "DRR_OK", 1: "DRR_ERR_INVALID_ARGUMENT", 2: "DRR_ERR_UNSUPPORTED",
          3: "DRR_ERR_WORKSPACE_TOO_SMALL", 4: "DRR_ERR_HIP"}

_lib = None


class DRRError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status


def library() -> ctypes.CDLL:
    """Load the in-tree libdrr.so (built by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY):
            raise RuntimeError(f"{LIBRARY} is not built; run `python -c 'import __graft_entry__ as "
                               "g; g.build()'` (hipcc, gfx950)")
        lib = ctypes.CDLL(LIBRARY)
        P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        lib.drr_workspace_bytes.argtypes = [I, I, I, I, I, I, I, I, I]
        lib.drr_workspace_bytes.restype = Z
        lib.drr_forward.argtypes = [P, I, I, I, I, P, P, P, I, I, I, I, I, P, P, P, Z, P]
        lib.drr_forward.restype = I
        lib.drr_forward_reuse.argtypes = lib.drr_forward.argtypes
        lib.drr_forward_reuse.restype = I
        lib.drr_forward_no_alloc.argtypes = [P, I, I, I, I, P, P, P, I, I, I, I, I, P, P, P]
        lib.drr_forward_no_alloc.restype = I
        lib.drr_backward_volume.argtypes = [I, I, I, P, P, P, I, I, I, I, I, P, P, P, P, Z, P]
        lib.drr_backward_volume.restype = I
        lib.drr_backward_pose.argtypes = [P, I, I, I, I, P, P, P, I, I, I, I, I, P, P, P, Z, P]
        lib.drr_backward_pose.restype = I
        lib.drr_backward_pose_reuse.argtypes = lib.drr_backward_pose.argtypes
        lib.drr_backward_pose_reuse.restype = I
        lib.drr_forward_siddon.argtypes = [P, I, I, I, I, P, P, P, I, I, I, I, P, P, P]
        lib.drr_forward_siddon.restype = I
        lib.drr_backward_volume_siddon.argtypes = [I, I, I, P, P, P, I, I, I, I, P, P, P, P]
        lib.drr_backward_volume_siddon.restype = I
        F = ctypes.c_float
        lib.drr_render_workspace_bytes.argtypes = [I] * 14
        lib.drr_render_workspace_bytes.restype = Z
        lib.drr_render.argtypes = [P, I, I, I, I, I, I, P, P, P, I, I, I, I, I, F, I, F, P, P, I,
                                   P, P, P, Z, P]
        lib.drr_render.restype = I
        lib.drr_render_reuse.argtypes = lib.drr_render.argtypes
        lib.drr_render_reuse.restype = I
        lib.drr_render_backward_volume.argtypes = [P, I, I, I, I, I, I, P, P, P, I, I, I, I, I, F,
                                                   I, F, P, P, I, P, P, P, P, P, Z, P]
        lib.drr_render_backward_volume.restype = I
        lib.drr_render_backward_pose.argtypes = [P, I, I, I, I, I, I, P, P, P, I, I, I, I, I, F, I,
                                                 F, P, P, I, P, P, P, Z, P]
        lib.drr_render_backward_pose.restype = I
        lib.drr_render_backward_pose_reuse.argtypes = lib.drr_render_backward_pose.argtypes
        lib.drr_render_backward_pose_reuse.restype = I
        lib.drr_intrinsics_from_fov.argtypes = [F, I, I, P]
        lib.drr_intrinsics_from_fov.restype = I
        lib.drr_poses_from_view_matrices.argtypes = [P, I, P, I, I, I, P, P, P]
        lib.drr_poses_from_view_matrices.restype = I
        lib.drr_view_matrices_backward.argtypes = [P, I, P, I, I, I, P, P, P]
        lib.drr_view_matrices_backward.restype = I
        L = ctypes.c_longlong
        lib.drr_poisson_surrogate.argtypes = [P, P, L, F, P, P]
        lib.drr_poisson_surrogate.restype = I
        lib.drr_poisson_surrogate_backward.argtypes = [P, P, L, F, P, P, P]
        lib.drr_poisson_surrogate_backward.restype = I
        lib.drr_status_string.argtypes = [I]
        lib.drr_status_string.restype = ctypes.c_char_p
        lib.drr_last_error.restype = ctypes.c_char_p
        lib.drr_abi_version.restype = I
        _lib = lib
    return _lib


def _check(status: int):
    if status != 0:
        raise DRRError(status, library().drr_last_error().decode())


def _host_floats(x, n: int):
    vals = torch.as_tensor(x, dtype=torch.float32).detach().cpu().reshape(-1)
    if vals.numel() != n:
        raise ValueError(f"expected {n} values, got {vals.numel()}")
    return (ctypes.c_float * n)(*[float(v) for v in vals])


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _device_tensor(t: torch.Tensor, name: str, dtype=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _volume_dtype(volume: torch.Tensor) -> int:
    if volume.dtype == torch.float32:
        return F32
    if volume.dtype == torch.bfloat16:
        return BF16
    raise ValueError(f"volume must be float32 or bfloat16, got {volume.dtype}")


def drr_workspace_bytes(nz: int, ny: int, nx: int, dtype: int, n_views: int, det_h: int,
                        det_w: int, n_samples: int, for_backward: int) -> int:
    return int(library().drr_workspace_bytes(nz, ny, nx, dtype, n_views, det_h, det_w,
                                             n_samples, for_backward))


def _workspace(nbytes: int, device) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def drr_forward(volume: torch.Tensor, spacing: Sequence[float], K, poses: torch.Tensor,
                det_h: int, det_w: int, n_samples: int, mode: int = BEER_LAMBERT,
                out: Optional[torch.Tensor] = None, line_integral=True,
                workspace: Optional[torch.Tensor] = None,
                stream=None, reuse_copy: bool = False) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Forward DRR of ``volume`` (nz, ny, nx) for ``poses`` (V, 3, 4) world-to-camera.
    Returns (image (V, det_h, det_w) fp32, line integrals or None).  With
    ``reuse_copy`` the call skips the relayout (``drr_forward_reuse``):
    ``workspace`` must hold the read copy an earlier call made of the same
    volume for the same n_views, det_h, det_w and n_samples."""
    volume = _device_tensor(volume, "volume")
    dtype = _volume_dtype(volume)
    poses = _device_tensor(poses, "poses", torch.float32)
    if volume.dim() != 3 or poses.dim() != 3 or tuple(poses.shape[1:]) != (3, 4):
        raise ValueError("volume must be (nz, ny, nx) and poses (V, 3, 4)")
    nz, ny, nx = (int(s) for s in volume.shape)
    V = int(poses.shape[0])
    dev = volume.device
    if out is None:
        out = torch.empty((V, det_h, det_w), dtype=torch.float32, device=dev)
    out = _device_tensor(out, "out", torch.float32)
    if out.numel() != V * det_h * det_w:
        raise ValueError("out has the wrong size")
    if line_integral is True:
        line_integral = torch.empty_like(out)
    elif line_integral is False:
        line_integral = None
    if line_integral is not None:
        line_integral = _device_tensor(line_integral, "line_integral", torch.float32)
        if line_integral.numel() != out.numel():
            raise ValueError("line_integral has the wrong size")
    need = drr_workspace_bytes(nz, ny, nx, dtype, V, det_h, det_w, n_samples, 0)
    if reuse_copy and need and workspace is None:
        raise ValueError("reuse_copy needs the workspace that holds the read copy")
    if workspace is None:
        workspace = _workspace(need, dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    fn = library().drr_forward_reuse if reuse_copy else library().drr_forward
    _check(fn(
        _ptr(volume), dtype, nz, ny, nx, _host_floats(spacing, 3), _host_floats(K, 9),
        _ptr(poses), V, det_h, det_w, n_samples, mode, _ptr(out), _ptr(line_integral),
        _ptr(workspace), ws_bytes, _stream(stream)))
    return out, line_integral


def drr_forward_no_alloc(volume: torch.Tensor, spacing: Sequence[float], K,
                         poses: torch.Tensor, det_h: int, det_w: int, n_samples: int,
                         mode: int = BEER_LAMBERT, out: Optional[torch.Tensor] = None,
                         line_integral=True, stream=None):
    """``drr_forward`` without a workspace: the library's fixed device scratch
    (``NO_ALLOC_SCRATCH_BYTES`` per GPU) holds the volume copy the read plan
    marches.  Passing ``out`` (and ``line_integral``, or ``False``) makes the call
    allocate nothing, e.g. under graph capture.  Calls that overlap on one GPU
    share the scratch and race."""
    volume = _device_tensor(volume, "volume")
    dtype = _volume_dtype(volume)
    poses = _device_tensor(poses, "poses", torch.float32)
    if volume.dim() != 3 or poses.dim() != 3 or tuple(poses.shape[1:]) != (3, 4):
        raise ValueError("volume must be (nz, ny, nx) and poses (V, 3, 4)")
    nz, ny, nx = (int(s) for s in volume.shape)
    V = int(poses.shape[0])
    if out is None:
        out = torch.empty((V, det_h, det_w), dtype=torch.float32, device=volume.device)
    out = _device_tensor(out, "out", torch.float32)
    if out.numel() != V * det_h * det_w:
        raise ValueError("out has the wrong size")
    if line_integral is True:
        line_integral = torch.empty_like(out)
    elif line_integral is False:
        line_integral = None
    if line_integral is not None:
        line_integral = _device_tensor(line_integral, "line_integral", torch.float32)
        if line_integral.numel() != out.numel():
            raise ValueError("line_integral has the wrong size")
    _check(library().drr_forward_no_alloc(
        _ptr(volume), dtype, nz, ny, nx, _host_floats(spacing, 3), _host_floats(K, 9),
        _ptr(poses), V, det_h, det_w, n_samples, mode, _ptr(out), _ptr(line_integral),
        _stream(stream)))
    return out, line_integral


def drr_backward_volume(shape: Sequence[int], spacing: Sequence[float], K, poses: torch.Tensor,
                        det_h: int, det_w: int, n_samples: int, mode: int,
                        grad_out: torch.Tensor, line_integral: Optional[torch.Tensor],
                        grad_volume: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Volume gradient for upstream ``grad_out`` (V, det_h, det_w); ``line_integral``
    (the forward's s) is required for Beer-Lambert.  Returns (nz, ny, nx) fp32."""
    nz, ny, nx = (int(s) for s in shape)
    poses = _device_tensor(poses, "poses", torch.float32)
    grad_out = _device_tensor(grad_out, "grad_out", torch.float32)
    V = int(poses.shape[0])
    if grad_out.numel() != V * det_h * det_w:
        raise ValueError("grad_out has the wrong size")
    if line_integral is not None:
        line_integral = _device_tensor(line_integral, "line_integral", torch.float32)
    dev = grad_out.device
    if grad_volume is None:
        grad_volume = torch.empty((nz, ny, nx), dtype=torch.float32, device=dev)
    grad_volume = _device_tensor(grad_volume, "grad_volume", torch.float32)
    if grad_volume.numel() != nz * ny * nx:
        raise ValueError("grad_volume has the wrong size")
    need = drr_workspace_bytes(nz, ny, nx, F32, V, det_h, det_w, n_samples, 1)
    if workspace is None:
        workspace = _workspace(need, dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(library().drr_backward_volume(
        nz, ny, nx, _host_floats(spacing, 3), _host_floats(K, 9), _ptr(poses), V, det_h, det_w,
        n_samples, mode, _ptr(grad_out), _ptr(line_integral), _ptr(grad_volume),
        _ptr(workspace), ws_bytes, _stream(stream)))
    return grad_volume


def drr_backward_pose(volume: torch.Tensor, spacing: Sequence[float], K, poses: torch.Tensor,
                      det_h: int, det_w: int, n_samples: int, mode: int, grad_out: torch.Tensor,
                      grad_poses: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None, stream=None,
                      reuse_copy: bool = False) -> torch.Tensor:
    """dL/dP for L = sum(grad_out * I): (V, 3, 4) fp32 over each view's [R | t].
    With ``reuse_copy`` the call skips the relayout (``drr_backward_pose_reuse``):
    ``workspace`` must hold the read copy an earlier pose call made of the same
    volume for the same n_views, det_h, det_w and n_samples."""
    volume = _device_tensor(volume, "volume")
    dtype = _volume_dtype(volume)
    poses = _device_tensor(poses, "poses", torch.float32)
    grad_out = _device_tensor(grad_out, "grad_out", torch.float32)
    nz, ny, nx = (int(s) for s in volume.shape)
    V = int(poses.shape[0])
    if grad_out.numel() != V * det_h * det_w:
        raise ValueError("grad_out has the wrong size")
    if grad_poses is None:
        grad_poses = torch.empty((V, 3, 4), dtype=torch.float32, device=volume.device)
    grad_poses = _device_tensor(grad_poses, "grad_poses", torch.float32)
    need = drr_workspace_bytes(nz, ny, nx, dtype, V, det_h, det_w, n_samples, 2)
    if reuse_copy and workspace is None:
        raise ValueError("reuse_copy needs the workspace that holds the read copy")
    if workspace is None:
        workspace = _workspace(need, volume.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    fn = library().drr_backward_pose_reuse if reuse_copy else library().drr_backward_pose
    _check(fn(
        _ptr(volume), dtype, nz, ny, nx, _host_floats(spacing, 3), _host_floats(K, 9),
        _ptr(poses), V, det_h, det_w, n_samples, mode, _ptr(grad_out), _ptr(grad_poses),
        _ptr(workspace), ws_bytes, _stream(stream)))
    return grad_poses


def drr_forward_siddon(volume: torch.Tensor, spacing: Sequence[float], K, poses: torch.Tensor,
                       det_h: int, det_w: int, mode: int = BEER_LAMBERT,
                       out: Optional[torch.Tensor] = None, line_integral=True,
                       stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Forward DRR in the cell-constant (Siddon) model: s = sum_v mu_v l_v.
    Returns (image (V, det_h, det_w) fp32, line integrals or None)."""
    volume = _device_tensor(volume, "volume")
    dtype = _volume_dtype(volume)
    poses = _device_tensor(poses, "poses", torch.float32)
    if volume.dim() != 3 or poses.dim() != 3 or tuple(poses.shape[1:]) != (3, 4):
        raise ValueError("volume must be (nz, ny, nx) and poses (V, 3, 4)")
    nz, ny, nx = (int(s) for s in volume.shape)
    V = int(poses.shape[0])
    if out is None:
        out = torch.empty((V, det_h, det_w), dtype=torch.float32, device=volume.device)
    out = _device_tensor(out, "out", torch.float32)
    if out.numel() != V * det_h * det_w:
        raise ValueError("out has the wrong size")
    if line_integral is True:
        line_integral = torch.empty_like(out)
    elif line_integral is False:
        line_integral = None
    if line_integral is not None:
        line_integral = _device_tensor(line_integral, "line_integral", torch.float32)
        if line_integral.numel() != out.numel():
            raise ValueError("line_integral has the wrong size")
    _check(library().drr_forward_siddon(
        _ptr(volume), dtype, nz, ny, nx, _host_floats(spacing, 3), _host_floats(K, 9),
        _ptr(poses), V, det_h, det_w, mode, _ptr(out), _ptr(line_integral), _stream(stream)))
    return out, line_integral


def drr_backward_volume_siddon(shape: Sequence[int], spacing: Sequence[float], K,
                               poses: torch.Tensor, det_h: int, det_w: int, mode: int,
                               grad_out: torch.Tensor, line_integral: Optional[torch.Tensor],
                               grad_volume: Optional[torch.Tensor] = None,
                               stream=None) -> torch.Tensor:
    """Matched adjoint of ``drr_forward_siddon`` (its volume gradient)."""
    nz, ny, nx = (int(s) for s in shape)
    poses = _device_tensor(poses, "poses", torch.float32)
    grad_out = _device_tensor(grad_out, "grad_out", torch.float32)
    V = int(poses.shape[0])
    if grad_out.numel() != V * det_h * det_w:
        raise ValueError("grad_out has the wrong size")
    if line_integral is not None:
        line_integral = _device_tensor(line_integral, "line_integral", torch.float32)
    if grad_volume is None:
        grad_volume = torch.empty((nz, ny, nx), dtype=torch.float32, device=grad_out.device)
    grad_volume = _device_tensor(grad_volume, "grad_volume", torch.float32)
    if grad_volume.numel() != nz * ny * nx:
        raise ValueError("grad_volume has the wrong size")
    _check(library().drr_backward_volume_siddon(
        nz, ny, nx, _host_floats(spacing, 3), _host_floats(K, 9), _ptr(poses), V, det_h, det_w,
        mode, _ptr(grad_out), _ptr(line_integral), _ptr(grad_volume), _stream(stream)))
    return grad_volume


class _Render(torch.autograd.Function):
    @staticmethod
    def forward(ctx, volume, spacing, K, poses, det_h, det_w, n_samples, mode):
        img, s = drr_forward(volume.detach(), spacing, K, poses.detach(), det_h, det_w,
                             n_samples, mode)
        ctx.save_for_backward(volume.detach(), poses.detach(), s)
        ctx.geom = (spacing, K, det_h, det_w, n_samples, mode)
        return img

    @staticmethod
    def backward(ctx, grad_img):
        volume, poses, s = ctx.saved_tensors
        spacing, K, det_h, det_w, n_samples, mode = ctx.geom
        g_img = grad_img.contiguous().float()
        g_vol = g_pose = None
        if ctx.needs_input_grad[0]:
            g_vol = drr_backward_volume(tuple(volume.shape), spacing, K, poses, det_h, det_w,
                                        n_samples, mode, g_img, s).to(volume.dtype)
        if ctx.needs_input_grad[3]:
            g_pose = drr_backward_pose(volume, spacing, K, poses, det_h, det_w, n_samples, mode,
                                       g_img)
        return g_vol, None, None, g_pose, None, None, None, None


def render(volume: torch.Tensor, spacing, K, poses: torch.Tensor, det_h: int, det_w: int,
           n_samples: int, mode: int = BEER_LAMBERT) -> torch.Tensor:
    """Differentiable DRR: image (V, det_h, det_w); gradients flow to ``volume``
    and to ``poses`` (each view's [R | t] entries)."""
    return _Render.apply(volume, spacing, K, poses, det_h, det_w, n_samples, mode)


class _RenderSiddon(torch.autograd.Function):
    @staticmethod
    def forward(ctx, volume, spacing, K, poses, det_h, det_w, mode):
        img, s = drr_forward_siddon(volume.detach(), spacing, K, poses.detach(), det_h, det_w,
                                    mode)
        ctx.save_for_backward(poses.detach(), s)
        ctx.geom = (tuple(volume.shape), volume.dtype, spacing, K, det_h, det_w, mode)
        return img

    @staticmethod
    def backward(ctx, grad_img):
        poses, s = ctx.saved_tensors
        shape, dtype, spacing, K, det_h, det_w, mode = ctx.geom
        g_vol = None
        if ctx.needs_input_grad[0]:
            g_vol = drr_backward_volume_siddon(shape, spacing, K, poses, det_h, det_w, mode,
                                               grad_img.contiguous().float(), s).to(dtype)
        return g_vol, None, None, None, None, None, None


def render_siddon(volume: torch.Tensor, spacing, K, poses: torch.Tensor, det_h: int, det_w: int,
                  mode: int = BEER_LAMBERT) -> torch.Tensor:
    """Differentiable cell-constant DRR: image (V, det_h, det_w); the gradient
    flows to ``volume`` (the poses are treated as constants here)."""
    return _RenderSiddon.apply(volume, spacing, K, poses, det_h, det_w, mode)


def project_siddon(volume, spacing, K, poses, det_h, det_w) -> torch.Tensor:
    """A x in the cell-constant model (diffct ``project``)."""
    return drr_forward_siddon(volume, spacing, K, poses, det_h, det_w, LINE_INTEGRAL,
                              line_integral=False)[0]


def backproject_siddon(y, shape, spacing, K, poses, det_h, det_w) -> torch.Tensor:
    """A^T y, the matched adjoint of ``project_siddon`` (diffct ``backproject``)."""
    return drr_backward_volume_siddon(shape, spacing, K, poses, det_h, det_w, LINE_INTEGRAL,
                                      y.contiguous(), None)


def project(volume, spacing, K, poses, det_h, det_w, n_samples) -> torch.Tensor:
    """A x: raw line integrals (diffct ``project``)."""
    return drr_forward(volume, spacing, K, poses, det_h, det_w, n_samples, LINE_INTEGRAL,
                       line_integral=False)[0]


def backproject(y, shape, spacing, K, poses, det_h, det_w, n_samples) -> torch.Tensor:
    """A^T y: the matched adjoint of ``project`` (diffct ``backproject``)."""
    return drr_backward_volume(shape, spacing, K, poses, det_h, det_w, n_samples, LINE_INTEGRAL,
                               y.contiguous(), None)


# ---------------------------------------------------------------- flashdrr front end

def _transfer(transfer, C: int):
    """(xp, yp), each (C, K) -> two host float arrays and K (or Nones and 0)."""
    if transfer is None:
        return None, None, 0
    xp = torch.as_tensor(transfer[0], dtype=torch.float32).detach().cpu().reshape(C, -1)
    yp = torch.as_tensor(transfer[1], dtype=torch.float32).detach().cpu().reshape(C, -1)
    if xp.shape != yp.shape:
        raise ValueError("transfer xp and yp must have the same shape (C, K)")
    k = int(xp.shape[1])
    return _host_floats(xp, C * k), _host_floats(yp, C * k), k


def _batched_volume(volume: torch.Tensor):
    if volume.dim() == 3:
        return 1, 1, tuple(int(x) for x in volume.shape)
    if volume.dim() == 5:
        B, C, nz, ny, nx = (int(x) for x in volume.shape)
        return B, C, (nz, ny, nx)
    raise ValueError("volume must be (nz, ny, nx) or (B, C, nz, ny, nx)")


def drr_render_workspace_bytes(n_volumes: int, n_channels: int, nz: int, ny: int, nx: int,
                               dtype: int, n_views: int, det_h: int, det_w: int, n_samples: int,
                               mode: int, clip: int, tf_knots: int, for_backward: int) -> int:
    return int(library().drr_render_workspace_bytes(n_volumes, n_channels, nz, ny, nx, dtype,
                                                    n_views, det_h, det_w, n_samples, mode, clip,
                                                    tf_knots, for_backward))


def drr_render(volume: torch.Tensor, spacing, K, poses: torch.Tensor, det_h: int, det_w: int,
               n_samples: int, mode: int = BEER_LAMBERT, density_factor: float = 1.0,
               clip: int = CLIP_BOX, margin: float = 30.0, transfer=None,
               out: Optional[torch.Tensor] = None, aux=True,
               workspace: Optional[torch.Tensor] = None,
               stream=None, reuse_copy: bool = False) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Render ``volume`` (B, C, nz, ny, nx) (or (nz, ny, nx)) for ``poses``
    (V, 3, 4), V a multiple of B (view v renders volume v // (V // B)).
    Returns (image (V, C, det_h, det_w) fp32, optical depth or None).  With
    ``reuse_copy`` the call skips the relayout (``drr_render_reuse``):
    ``workspace`` must hold the read copy an earlier render made of the same
    volume, transfer function and clip for the same launch shape."""
    volume = _device_tensor(volume, "volume")
    dtype = _volume_dtype(volume)
    poses = _device_tensor(poses, "poses", torch.float32)
    if poses.dim() != 3 or tuple(poses.shape[1:]) != (3, 4):
        raise ValueError("poses must be (V, 3, 4)")
    B, C, (nz, ny, nx) = _batched_volume(volume)
    V = int(poses.shape[0])
    xp, yp, nk = _transfer(transfer, C)
    dev = volume.device
    if out is None:
        out = torch.empty((V, C, det_h, det_w), dtype=torch.float32, device=dev)
    out = _device_tensor(out, "out", torch.float32)
    if out.numel() != V * C * det_h * det_w:
        raise ValueError("out has the wrong size")
    if aux is True:
        aux = torch.empty_like(out)
    elif aux is False:
        aux = None
    if aux is not None:
        aux = _device_tensor(aux, "aux", torch.float32)
        if aux.numel() != out.numel():
            raise ValueError("aux has the wrong size")
    need = drr_render_workspace_bytes(B, C, nz, ny, nx, dtype, V, det_h, det_w, n_samples, mode,
                                      clip, nk, 0)
    if reuse_copy and need and workspace is None:
        raise ValueError("reuse_copy needs the workspace that holds the read copy")
    if workspace is None:
        workspace = _workspace(need, dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check((library().drr_render_reuse if reuse_copy else library().drr_render)(
        _ptr(volume), dtype, B, C, nz, ny, nx, _host_floats(spacing, 3), _host_floats(K, 9),
        _ptr(poses), V, det_h, det_w, n_samples, mode, float(density_factor), clip, float(margin),
        xp, yp, nk, _ptr(out), _ptr(aux), _ptr(workspace), ws_bytes, _stream(stream)))
    return out, aux


def drr_render_backward_volume(volume: Optional[torch.Tensor], shape, dtype: int, spacing, K,
                               poses: torch.Tensor, det_h: int, det_w: int, n_samples: int,
                               mode: int, grad_out: torch.Tensor,
                               out: Optional[torch.Tensor], aux: Optional[torch.Tensor],
                               density_factor: float = 1.0, clip: int = CLIP_BOX,
                               margin: float = 30.0, transfer=None,
                               grad_volume: Optional[torch.Tensor] = None,
                               workspace: Optional[torch.Tensor] = None,
                               stream=None) -> torch.Tensor:
    """Gradient of sum(grad_out * image) with respect to the input volume of
    ``drr_render``; ``shape`` is the volume's (B, C, nz, ny, nx) or (nz, ny, nx).
    ``volume`` is needed for alpha compositing and with a transfer function,
    ``out`` for alpha compositing, ``aux`` for Beer-Lambert.  Returns fp32 of
    ``shape``."""
    shape = tuple(int(x) for x in shape)
    if len(shape) == 3:
        B, C, (nz, ny, nx) = 1, 1, shape
    elif len(shape) == 5:
        B, C, nz, ny, nx = shape
    else:
        raise ValueError("shape must be (nz, ny, nx) or (B, C, nz, ny, nx)")
    if volume is not None:
        volume = _device_tensor(volume, "volume")
        dtype = _volume_dtype(volume)
    poses = _device_tensor(poses, "poses", torch.float32)
    grad_out = _device_tensor(grad_out, "grad_out", torch.float32)
    V = int(poses.shape[0])
    if grad_out.numel() != V * C * det_h * det_w:
        raise ValueError("grad_out has the wrong size")
    if out is not None:
        out = _device_tensor(out, "out", torch.float32)
    if aux is not None:
        aux = _device_tensor(aux, "aux", torch.float32)
    xp, yp, nk = _transfer(transfer, C)
    dev = grad_out.device
    if grad_volume is None:
        grad_volume = torch.empty(shape, dtype=torch.float32, device=dev)
    grad_volume = _device_tensor(grad_volume, "grad_volume", torch.float32)
    if grad_volume.numel() != B * C * nz * ny * nx:
        raise ValueError("grad_volume has the wrong size")
    need = drr_render_workspace_bytes(B, C, nz, ny, nx, dtype, V, det_h, det_w, n_samples, mode,
                                      clip, nk, 1)
    if workspace is None:
        workspace = _workspace(need, dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(library().drr_render_backward_volume(
        _ptr(volume), dtype, B, C, nz, ny, nx, _host_floats(spacing, 3), _host_floats(K, 9),
        _ptr(poses), V, det_h, det_w, n_samples, mode, float(density_factor), clip, float(margin),
        xp, yp, nk, _ptr(grad_out), _ptr(out), _ptr(aux), _ptr(grad_volume), _ptr(workspace),
        ws_bytes, _stream(stream)))
    return grad_volume


def drr_render_backward_pose(volume: torch.Tensor, spacing, K, poses: torch.Tensor, det_h: int,
                             det_w: int, n_samples: int, mode: int, grad_out: torch.Tensor,
                             density_factor: float = 1.0, clip: int = CLIP_BOX,
                             margin: float = 30.0, transfer=None,
                             grad_poses: Optional[torch.Tensor] = None,
                             workspace: Optional[torch.Tensor] = None,
                             stream=None, reuse_copy: bool = False) -> torch.Tensor:
    """dL/dP (V, 3, 4) for L = sum(grad_out * image) of ``drr_render`` (every
    mode, either clip), summed over each view's channels.  With ``reuse_copy``
    (``drr_render_backward_pose_reuse``) ``workspace`` must hold the read copy
    an earlier call made of the same volume for the same launch shape."""
    volume = _device_tensor(volume, "volume")
    dtype = _volume_dtype(volume)
    poses = _device_tensor(poses, "poses", torch.float32)
    grad_out = _device_tensor(grad_out, "grad_out", torch.float32)
    B, C, (nz, ny, nx) = _batched_volume(volume)
    V = int(poses.shape[0])
    if grad_out.numel() != V * C * det_h * det_w:
        raise ValueError("grad_out has the wrong size")
    xp, yp, nk = _transfer(transfer, C)
    if grad_poses is None:
        grad_poses = torch.empty((V, 3, 4), dtype=torch.float32, device=volume.device)
    grad_poses = _device_tensor(grad_poses, "grad_poses", torch.float32)
    need = drr_render_workspace_bytes(B, C, nz, ny, nx, dtype, V, det_h, det_w, n_samples, mode,
                                      clip, nk, 2)
    if reuse_copy and workspace is None:
        raise ValueError("reuse_copy needs the workspace that holds the read copy")
    if workspace is None:
        workspace = _workspace(need, volume.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check((library().drr_render_backward_pose_reuse if reuse_copy
            else library().drr_render_backward_pose)(
        _ptr(volume), dtype, B, C, nz, ny, nx, _host_floats(spacing, 3), _host_floats(K, 9),
        _ptr(poses), V, det_h, det_w, n_samples, mode, float(density_factor), clip, float(margin),
        xp, yp, nk, _ptr(grad_out), _ptr(grad_poses), _ptr(workspace), ws_bytes, _stream(stream)))
    return grad_poses


class _Raycast(torch.autograd.Function):
    @staticmethod
    def forward(ctx, volume, spacing, K, poses, det_h, det_w, n_samples, mode, density_factor,
                clip, margin, transfer):
        img, tau = drr_render(volume.detach(), spacing, K, poses.detach(), det_h, det_w,
                              n_samples, mode, density_factor, clip, margin, transfer)
        ctx.save_for_backward(volume.detach(), poses.detach(), img, tau)
        ctx.args = (spacing, K, det_h, det_w, n_samples, mode, density_factor, clip, margin,
                    transfer)
        return img

    @staticmethod
    def backward(ctx, grad_img):
        volume, poses, img, tau = ctx.saved_tensors
        spacing, K, det_h, det_w, n_samples, mode, f, clip, margin, transfer = ctx.args
        g_vol = g_pose = None
        g_img = grad_img.contiguous().float()
        if ctx.needs_input_grad[0]:
            g_vol = drr_render_backward_volume(
                volume, tuple(volume.shape), _volume_dtype(volume), spacing, K, poses, det_h,
                det_w, n_samples, mode, g_img, img, tau, f, clip, margin,
                transfer).to(volume.dtype)
        if ctx.needs_input_grad[3]:
            g_pose = drr_render_backward_pose(volume, spacing, K, poses, det_h, det_w, n_samples,
                                              mode, g_img, f, clip, margin, transfer)
        return (g_vol, None, None, g_pose) + (None,) * 8


def raycast(volume: torch.Tensor, spacing, K, poses: torch.Tensor, det_h: int, det_w: int,
            n_samples: int, mode: int = BEER_LAMBERT, density_factor: float = 1.0,
            clip: int = CLIP_BOX, margin: float = 30.0, transfer=None) -> torch.Tensor:
    """Differentiable flashdrr-style render: ``volume`` (B, C, nz, ny, nx) and
    ``poses`` (V, 3, 4) with V a multiple of B -- or one pose, used for every
    volume -- give images (V, C, det_h, det_w); gradients flow to the volume
    and to the poses."""
    if volume.dim() == 5 and poses.shape[0] == 1 and volume.shape[0] > 1:
        poses = poses.expand(volume.shape[0], 3, 4).contiguous()
    return _Raycast.apply(volume, spacing, K, poses, det_h, det_w, n_samples, mode,
                          density_factor, clip, margin, transfer)


# ---------------------------------------------------------------- flashdrr cameras

def drr_intrinsics_from_fov(fov_deg: float, det_h: int, det_w: int) -> torch.Tensor:
    """HZ intrinsics (3, 3) fp32 (host) for a vertical field of view in degrees."""
    K = (ctypes.c_float * 9)()
    _check(library().drr_intrinsics_from_fov(float(fov_deg), det_h, det_w, K))
    return torch.tensor(list(K), dtype=torch.float32).reshape(3, 3)


def drr_poses_from_view_matrices(view_mats: torch.Tensor, ras2ijk, shape,
                                 poses: Optional[torch.Tensor] = None,
                                 stream=None) -> Tuple[torch.Tensor, Tuple[float, float, float]]:
    """VTK camera-to-world view matrices (V, 4, 4) and a ras2ijk affine -> HZ
    world-to-camera poses (V, 3, 4) in the rendering frame of a volume of
    ``shape`` (nz, ny, nx), and its voxel sizes (sx, sy, sz)."""
    view_mats = _device_tensor(view_mats, "view_mats", torch.float32)
    if view_mats.dim() != 3 or tuple(view_mats.shape[1:]) != (4, 4):
        raise ValueError("view_mats must be (V, 4, 4)")
    nz, ny, nx = (int(x) for x in shape)
    V = int(view_mats.shape[0])
    if poses is None:
        poses = torch.empty((V, 3, 4), dtype=torch.float32, device=view_mats.device)
    poses = _device_tensor(poses, "poses", torch.float32)
    sp = (ctypes.c_float * 3)()
    _check(library().drr_poses_from_view_matrices(
        _ptr(view_mats), V, _host_floats(ras2ijk, 16), nz, ny, nx, _ptr(poses), sp,
        _stream(stream)))
    return poses, (sp[0], sp[1], sp[2])


def drr_view_matrices_backward(view_mats: torch.Tensor, ras2ijk, shape, grad_poses: torch.Tensor,
                               grad_view_mats: Optional[torch.Tensor] = None,
                               stream=None) -> torch.Tensor:
    """dL/d(view_mats) (V, 4, 4) from dL/d(poses) (V, 3, 4)."""
    view_mats = _device_tensor(view_mats, "view_mats", torch.float32)
    grad_poses = _device_tensor(grad_poses, "grad_poses", torch.float32)
    nz, ny, nx = (int(x) for x in shape)
    V = int(view_mats.shape[0])
    if grad_poses.numel() != V * 12:
        raise ValueError("grad_poses must be (V, 3, 4)")
    if grad_view_mats is None:
        grad_view_mats = torch.empty((V, 4, 4), dtype=torch.float32, device=view_mats.device)
    grad_view_mats = _device_tensor(grad_view_mats, "grad_view_mats", torch.float32)
    _check(library().drr_view_matrices_backward(
        _ptr(view_mats), V, _host_floats(ras2ijk, 16), nz, ny, nx, _ptr(grad_poses),
        _ptr(grad_view_mats), _stream(stream)))
    return grad_view_mats


class _ViewPoses(torch.autograd.Function):
    @staticmethod
    def forward(ctx, view_mats, ras2ijk, shape):
        poses, spacing = drr_poses_from_view_matrices(view_mats.detach(), ras2ijk, shape)
        ctx.save_for_backward(view_mats.detach())
        ctx.args = (ras2ijk, shape)
        ctx.spacing = spacing
        return poses

    @staticmethod
    def backward(ctx, grad_poses):
        (view_mats,) = ctx.saved_tensors
        ras2ijk, shape = ctx.args
        g = drr_view_matrices_backward(view_mats, ras2ijk, shape, grad_poses.contiguous().float())
        return g, None, None


def render_view_matrices(volume: torch.Tensor, view_mats: torch.Tensor, ras2ijk, fov_deg: float,
                         det_h: int, det_w: int, n_samples: int,
                         mode: int = BEER_LAMBERT) -> torch.Tensor:
    """flashdrr-style render of one volume (nz, ny, nx) in IJK voxel space from
    VTK camera-to-world ``view_mats`` (V, 4, 4), a ``ras2ijk`` affine and a
    vertical field of view: images (V, det_h, det_w), differentiable with
    respect to the volume and the view matrices."""
    shape = tuple(int(x) for x in volume.shape)
    _, spacing = drr_poses_from_view_matrices(view_mats.detach(), ras2ijk, shape)
    poses = _ViewPoses.apply(view_mats, ras2ijk, shape)
    K = drr_intrinsics_from_fov(fov_deg, det_h, det_w)
    return render(volume, spacing, K, poses, det_h, det_w, n_samples, mode)


# ---------------------------------------------------------------- noise surrogate

def drr_poisson_surrogate(transmission: torch.Tensor, noise: torch.Tensor, i0: float,
                          out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """flashdrr apply_poisson with the standard-normal draws ``noise`` given:
    clamp(T + noise * sqrt(T / i0), 0, 1), same shape as ``transmission``."""
    T = _device_tensor(transmission, "transmission", torch.float32)
    z = _device_tensor(noise, "noise", torch.float32)
    if z.numel() != T.numel():
        raise ValueError("noise must have as many elements as transmission")
    if out is None:
        out = torch.empty_like(T)
    out = _device_tensor(out, "out", torch.float32)
    _check(library().drr_poisson_surrogate(_ptr(T), _ptr(z), T.numel(), float(i0), _ptr(out),
                                           _stream(stream)))
    return out


def drr_poisson_surrogate_backward(transmission: torch.Tensor, noise: torch.Tensor, i0: float,
                                   grad_out: torch.Tensor,
                                   grad_transmission: Optional[torch.Tensor] = None,
                                   stream=None) -> torch.Tensor:
    T = _device_tensor(transmission, "transmission", torch.float32)
    z = _device_tensor(noise, "noise", torch.float32)
    g = _device_tensor(grad_out, "grad_out", torch.float32)
    if grad_transmission is None:
        grad_transmission = torch.empty_like(T)
    grad_transmission = _device_tensor(grad_transmission, "grad_transmission", torch.float32)
    _check(library().drr_poisson_surrogate_backward(_ptr(T), _ptr(z), T.numel(), float(i0),
                                                    _ptr(g), _ptr(grad_transmission),
                                                    _stream(stream)))
    return grad_transmission


class _Poisson(torch.autograd.Function):
    @staticmethod
    def forward(ctx, transmission, noise, i0):
        ctx.save_for_backward(transmission.detach(), noise.detach())
        ctx.i0 = i0
        return drr_poisson_surrogate(transmission.detach().contiguous(),
                                     noise.detach().contiguous(), i0)

    @staticmethod
    def backward(ctx, grad):
        T, z = ctx.saved_tensors
        g = drr_poisson_surrogate_backward(T.contiguous(), z.contiguous(), ctx.i0,
                                           grad.contiguous().float())
        return g, None, None


def poisson_noise(transmission: torch.Tensor, noise: torch.Tensor, i0: Optional[float]):
    """Differentiable Gaussian-Poisson surrogate; ``i0 = None`` returns the
    transmission unchanged (flashdrr's default: no noise model)."""
    if i0 is None:
        return transmission
    return _Poisson.apply(transmission, noise, float(i0))
