"""Shared test helpers: parity metrics and GPU plumbing (no method arithmetic)."""
import numpy as np


def forward_rel_err(gpu, ref):
    """Max relative error with a floor: max |g - o| / max(|o|, 1e-3 max|o|).
    Near-zero outputs would otherwise inflate per-pixel relative errors
    (torchtomo's adjoint-diagnostics advice: prefer aggregate residuals)."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    scale = np.abs(ref).max()
    if scale == 0.0:
        return float(np.abs(gpu).max())
    floor = 1e-3 * scale
    return float((np.abs(gpu - ref) / np.maximum(np.abs(ref), floor)).max())


def normwise_err(gpu, ref):
    """max |g - o| / max |o| (gradients: uniform upstream signs make single voxel
    sums cancel, so a per-voxel relative error is not meaningful)."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    scale = np.abs(ref).max()
    return float(np.abs(gpu - ref).max() / scale) if scale > 0 else float(np.abs(gpu).max())


def l2_err(gpu, ref):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(gpu - ref) / max(np.linalg.norm(ref), 1e-300))


def say(*a):
    print(*a, flush=True)


def check_forward(img_gpu, ref, bar, what, chord=None):
    """Floored max relative error within ``bar``; rays the oracle finds missing
    the box (chord 0) must be exactly 0 on the GPU as well."""
    g = img_gpu.cpu().double().numpy() if hasattr(img_gpu, "cpu") else np.asarray(img_gpu)
    err = forward_rel_err(g, ref)
    say(f"{what}: forward max rel err {err:.3e} (bar {bar:g}), "
        f"normwise {normwise_err(g, ref):.3e}")
    assert err <= bar
    if chord is not None:
        miss = chord == 0.0
        assert np.all(g[miss] == 0.0), f"{what}: misses must be exactly 0"
        say(f"{what}: {int(miss.sum())} misses, all exactly 0")
    return err
