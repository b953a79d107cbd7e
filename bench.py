#!/usr/bin/env python3
"""Throughput of the cone-beam DRR hot path on one MI355X.

A step is one FlashDRR-style train step on the 1024x1024 workload (256^3 fp32
phantom, one view, 512 samples per ray, Beer-Lambert): the forward DRR
(ray setup, box clip, march, epilogue) followed by the volume backward (fill,
scatter) -- every stage of the path, on inputs already resident in HBM.

Printed (one JSON line on stdout):
  value        rays x samples per second of the step (nominal: every pixel's
               ray counts N samples), in Gsamples/s
  fps          views per second of the step
  roofline     the dominant kernel against the 8 TB/s HBM peak, on
               algorithmic bytes (8 corners x element bytes per sample on rays
               that hit the volume, plus per-ray reads/writes), with its
               duration measured by HIP events on the launch stream
  cpu_baseline the CPU oracle on the same step, timed on the host cores
  front_end    flashdrr front-end variants (transfer function from HU, near/far
               clipping, alpha compositing, volume and channel batches),
               forward and volume backward, graph-timed like the workloads
  workloads    every workload (200x200 16-view batch in fp32 and bf16, the
               1024^2 step's kernels, 2048^2 eval, 360-view helix, 64^3 tiny)
               as context lines, with the pose gradient (registration) on the
               batch and the 1024^2 camera, each
               kernel timed per launch from a replayed HIP graph of
               back-to-back launches (GPU time, no host launch latency)

Options: --gpus N (only 1 is supported: this build runs on one GPU),
--steps K, --warmup W, --no-cpu, --no-workloads, and --pmc-pass
{forward,backward,copy} which runs a short fixed launch sequence for
rocprofv3 counter collection.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "DRR FPS and Gsamples/s (rays x samples) at 200^2 and 1024^2; % HBM roofline"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_revision() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "ct_forward_projection_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


class Resident:
    """A workload's arrays on the device plus preallocated outputs."""

    def __init__(self, w, dev, bf16=False):
        import torch
        self.w = w
        if bf16:
            self.vol = torch.from_numpy(w.volume_bf16.view(np.int16)).to(dev).view(torch.bfloat16)
        else:
            self.vol = torch.from_numpy(w.volume).to(dev)
        self.poses = torch.from_numpy(w.poses).to(dev)
        self.out = torch.empty((w.n_views, w.det_h, w.det_w), device=dev)
        self.s = torch.empty_like(self.out)
        self.g = None if w.grad_out is None else torch.from_numpy(w.grad_out).to(dev)
        self.grad = torch.empty(w.volume.shape, device=dev) if w.grad_out is not None else None
        self.elem_bytes = 2 if bf16 else 4
        import ct_forward_projection_amd as drr
        nz, ny, nx = w.volume.shape
        need = drr.drr_workspace_bytes(nz, ny, nx, drr.BF16 if bf16 else drr.F32, w.n_views,
                                       w.det_h, w.det_w, w.n_samples, 0)
        self.workspace = torch.empty(need, dtype=torch.uint8, device=dev) if need else None
        self.pose_ws = None

    def forward(self):
        import ct_forward_projection_amd as drr
        w = self.w
        drr.drr_forward(self.vol, w.spacing, w.K, self.poses, w.det_h, w.det_w, w.n_samples,
                        w.mode, out=self.out, line_integral=self.s, workspace=self.workspace)

    def backward(self):
        import ct_forward_projection_amd as drr
        w = self.w
        drr.drr_backward_volume(w.volume.shape, w.spacing, w.K, self.poses, w.det_h, w.det_w,
                                w.n_samples, w.mode, self.g, self.s, grad_volume=self.grad)

    def pose_backward(self):
        import ct_forward_projection_amd as drr
        w = self.w
        if self.pose_ws is None:
            import torch
            nz, ny, nx = w.volume.shape
            need = drr.drr_workspace_bytes(nz, ny, nx, drr.BF16 if self.elem_bytes == 2 else drr.F32,
                                           w.n_views, w.det_h, w.det_w, w.n_samples, 2)
            self.pose_ws = torch.empty(need, dtype=torch.uint8, device=self.out.device)
            self.pose_g = torch.ones_like(self.out) if self.g is None else self.g
            self.grad_poses = torch.empty((w.n_views, 3, 4), device=self.out.device)
        drr.drr_backward_pose(self.vol, w.spacing, w.K, self.poses, w.det_h, w.det_w, w.n_samples,
                              w.mode, self.pose_g, grad_poses=self.grad_poses,
                              workspace=self.pose_ws)

    def siddon_forward(self):
        import ct_forward_projection_amd as drr
        w = self.w
        drr.drr_forward_siddon(self.vol, w.spacing, w.K, self.poses, w.det_h, w.det_w, w.mode,
                               out=self.out, line_integral=self.s)

    def siddon_backward(self):
        import ct_forward_projection_amd as drr
        w = self.w
        drr.drr_backward_volume_siddon(w.volume.shape, w.spacing, w.K, self.poses, w.det_h,
                                       w.det_w, w.mode, self.g, self.s, grad_volume=self.grad)

    def hit_rays(self) -> int:
        """Rays that intersect the volume box, counted by the library itself: the
        line integral of a volume of ones is the chord, > 0 exactly on hits."""
        import torch

        import ct_forward_projection_amd as drr
        w = self.w
        ones = torch.ones(w.volume.shape, device=self.out.device)
        chord = drr.project(ones, w.spacing, w.K, self.poses, w.det_h, w.det_w, 1)
        return int((chord > 0).sum().item())


def time_events(fns, reps):
    """Per-function GPU time (ms, mean over reps) from events recorded on the
    current stream -- the stream the library launches on."""
    import torch
    st = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)] for _ in range(reps)]
    torch.cuda.synchronize()
    for r in range(reps):
        ev[r][0].record(st)
        for i, f in enumerate(fns):
            f()
            ev[r][i + 1].record(st)
    torch.cuda.synchronize()
    return [float(np.mean([ev[r][i].elapsed_time(ev[r][i + 1]) for r in range(reps)]))
            for i in range(len(fns))]


def time_graph(fns, min_ms=40.0):
    """Per-launch GPU time (ms) of each function, from a captured HIP graph of
    back-to-back launches replayed on the current stream: host launch latency
    is out of the measurement, as in a per-kernel GPU time."""
    import torch
    out = []
    for f in fns:
        f()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        f()
        e1.record()
        e1.synchronize()
        reps = int(max(1, min(200, min_ms / max(e0.elapsed_time(e1), 1e-3))))
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                f()
        g.replay()
        torch.cuda.synchronize()
        ts = []
        for _ in range(5):
            e0.record()
            g.replay()
            e1.record()
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) / reps)
        out.append(float(np.median(ts)))
        del g
    return out


def siddon_pieces(w) -> int:
    """Ray-voxel pieces of a workload (the cell-constant model's unit of work):
    a ray crossing the box from entry point p0 to exit point p1 visits
    1 + sum_a |floor index of p1 - floor index of p0| voxels.  Host-side
    geometry for the measurement only, vectorised over the rays of a view."""
    nz, ny, nx = w.volume.shape
    n = np.array([nx, ny, nz])
    s = np.asarray(w.spacing, dtype=np.float64)
    half = 0.5 * n * s
    K = np.asarray(w.K, dtype=np.float64)
    Ki = np.linalg.inv(K)
    cc, rr = np.meshgrid(np.arange(w.det_w) + 0.5, np.arange(w.det_h) + 0.5)
    m = np.stack([cc.ravel(), rr.ravel(), np.ones(cc.size)])
    total = 0
    for P in np.asarray(w.poses, dtype=np.float64):
        R, t = P[:, :3], P[:, 3]
        C = -R.T @ t
        d = R.T @ (Ki @ m)
        d /= np.linalg.norm(d, axis=0)
        with np.errstate(divide="ignore", invalid="ignore"):
            ta = (-half[:, None] - C[:, None]) / d
            tb = (half[:, None] - C[:, None]) / d
        inside = (np.abs(C) <= half)[:, None] | (d != 0)
        ta = np.where(d == 0, -np.inf, ta)
        tb = np.where(d == 0, np.inf, tb)
        t0 = np.maximum(np.max(np.minimum(ta, tb), axis=0), 0.0)
        t1 = np.min(np.maximum(ta, tb), axis=0)
        hit = (t1 > t0) & inside.all(axis=0)
        p0 = C[:, None] + t0 * d
        p1 = C[:, None] + t1 * d
        i0 = np.clip(np.floor((p0 + half[:, None]) / s[:, None]), 0, n[:, None] - 1)
        i1 = np.clip(np.floor((p1 + half[:, None]) / s[:, None]), 0, n[:, None] - 1)
        total += int(np.sum(np.where(hit, 1 + np.abs(i1 - i0).sum(axis=0), 0)))
    return total


def forward_bytes(res, hits):
    w = res.w
    return hits * w.n_samples * 8 * res.elem_bytes + w.n_rays * 8


def backward_bytes(res, hits):
    w = res.w
    return hits * w.n_samples * 8 * 4 + w.n_rays * 8


def roofline(name, alg_bytes, ms, traffic=None, valu_busy=None):
    """HBM roofline on algorithmic bytes.  Staged and cached kernels move far
    fewer bytes than the algorithm names (frac above 1): ``traffic`` gives the
    calibrated HBM bytes and ``valu_busy`` the share of VALU issue cycles, both
    from the committed counters of the current kernel sources (else None)."""
    achieved = alg_bytes / (ms * 1e-3) / 1e9
    return {"kernel": name, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
            "valu_busy": valu_busy}


def _committed_counters():
    """The committed counter summary, if it was taken on the current kernel
    sources; otherwise None."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    return d if d.get("kernel_revision") == kernel_revision() else None


def measured_valu_busy(kernel):
    """VALU busy of one kernel from the committed counters (None if stale)."""
    d = _committed_counters()
    k = None if d is None else d.get("kernels", {}).get(kernel)
    return None if k is None else k.get("valu_busy")


def measured_traffic(kernels):
    """HBM bytes per launch of a pass (the sum over its kernels) from the
    committed rocprofv3 counter summary, if it was taken on the current kernel
    sources and covers every kernel; otherwise None."""
    d = _committed_counters()
    if d is None:
        return None
    total = 0.0
    for name in kernels:
        k = d.get("kernels", {}).get(name)
        if k is None or k.get("hbm_bytes_per_launch") is None:
            return None
        total += k["hbm_bytes_per_launch"]
    return round(total)


def cpu_baseline(w):
    """The CPU oracle on the same train step (forward + volume gradient)."""
    import oracle
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or (os.cpu_count() or 1)
    t0 = time.perf_counter()
    oracle.forward_workload(w, n_threads=threads)
    _, used = oracle.adjoint_workload(w, n_threads=threads, max_buffer_bytes=8 << 30)
    dt = time.perf_counter() - t0
    return {"value": round(w.nominal_samples / dt / 1e9, 4), "unit": "Gsamples/s",
            "cores": int(min(threads, used) if used else threads), "kind": "oracle",
            "seconds": round(dt, 2),
            "sample": f"the whole step: {w.name} forward + volume gradient, fp64, "
                      f"{threads} threads forward / {used} threads scatter"}


def workload_lines(dev, reps):
    import workloads as W
    lines = {}
    for i, bf16 in [(1, False), (2, False), (2, True), (3, False), (4, False), (5, False)]:
        w = W.make_workload(i, with_bf16=bf16)
        res = Resident(w, dev, bf16=bf16)
        hits = res.hit_rays()
        fns = [res.forward] + ([res.backward] if w.grad_out is not None else [])
        with_pose = i in (2, 3)
        if with_pose:
            res.pose_backward()
            fns.append(res.pose_backward)
        t = time_graph(fns)
        fwd_ms = t[0]
        line = {"views": w.n_views, "detector": [w.det_h, w.det_w], "n_samples": w.n_samples,
                "dtype": "bf16" if bf16 else "f32",
                "forward_ms": round(fwd_ms, 4),
                "forward_fps": round(w.n_views / fwd_ms * 1e3, 1),
                "forward_gsamples_s": round(w.nominal_samples / fwd_ms / 1e6, 1),
                "forward_effective_gsamples_s": round(hits * w.n_samples / fwd_ms / 1e6, 1),
                "forward_hbm_frac": round(forward_bytes(res, hits) / (fwd_ms * 1e-3) / 1e9
                                          / HBM_PEAK_GBS, 4),
                "hit_rays": hits}
        if with_pose:
            pose_ms = t.pop()
            line["pose_backward_ms"] = round(pose_ms, 4)
            line["pose_backward_gsamples_s"] = round(w.nominal_samples / pose_ms / 1e6, 1)
            line["registration_step_fps"] = round(w.n_views / (fwd_ms + pose_ms) * 1e3, 1)
        if len(t) > 1:
            line["backward_ms"] = round(t[1], 4)
            line["backward_gsamples_s"] = round(w.nominal_samples / t[1] / 1e6, 1)
            line["backward_hbm_frac"] = round(backward_bytes(res, hits) / (t[1] * 1e-3) / 1e9
                                              / HBM_PEAK_GBS, 4)
        if i in (2, 3, 5):
            # cell-constant (Siddon) pair on the same inputs: algorithmic bytes are
            # one element read (forward) or one fp32 update (backward) per
            # ray-voxel piece, plus 8 B per ray
            pieces = siddon_pieces(w)
            sfns = [res.siddon_forward] + ([res.siddon_backward] if res.g is not None else [])
            ts = time_graph(sfns)
            line["siddon_pieces"] = pieces
            line["siddon_forward_ms"] = round(ts[0], 4)
            line["siddon_forward_fps"] = round(w.n_views / ts[0] * 1e3, 1)
            line["siddon_forward_gpieces_s"] = round(pieces / ts[0] / 1e6, 1)
            line["siddon_forward_hbm_frac"] = round(
                (pieces * res.elem_bytes + w.n_rays * 8) / (ts[0] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
            if len(ts) > 1:
                line["siddon_backward_ms"] = round(ts[1], 4)
                line["siddon_backward_hbm_frac"] = round(
                    (pieces * 4 + w.n_rays * 8) / (ts[1] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
        lines[w.name + ("-bf16" if bf16 else "")] = line
        log(f"workload {w.name}{' bf16' if bf16 else ''}: {line}")
        del res
    return lines


def read_plan(ws, B, C, nz, ny, nx, elem, V, H, Wd, N, clip, nk):
    """Name of the forward's read plan, told apart by its workspace size
    (corner cells, z-pairs and the mapped linear copy differ in size; no
    workspace is the LDS-staged boxes or the caller's volume)."""
    rnd = lambda b: (b + 255) // 256 * 256
    if ws == B * C * rnd((nx + 1) * (ny + 1) * (nz + 1) * 8 * elem):
        return "mapped corner cells" if nk else "corner cells"
    if clip == 1 and ws == B * C * rnd((nx + 2) * (ny + 2) * (nz + 1) * 2 * elem):
        return "mapped padded z-pairs" if nk else "padded z-pairs"
    if nz >= 2 and ws == B * C * rnd(nx * ny * (nz - 1) * 2 * elem):
        return "mapped z-pairs" if nk else "z-pairs"
    if ws > 0:
        return "mapped volume"
    staged = clip == 0 and V * C * H * Wd >= 65536 and \
        H * Wd * N / ((nx + 1) * (ny + 1) * (nz + 1)) >= 16
    return "LDS-staged boxes" if staged else "volume"


class RenderCase:
    """A drr_render configuration resident on the device, with preallocated
    outputs, workspaces and upstream gradient (so a captured graph allocates
    nothing)."""

    def __init__(self, vol, spacing, K, poses, H, Wd, N, mode, f=1.0, clip=0, margin=30.0,
                 transfer=None):
        import torch

        import ct_forward_projection_amd as drr
        self.args = (spacing, K, poses, H, Wd, N, mode, f, clip, margin, transfer)
        self.vol = vol
        B, C, nz, ny, nx = vol.shape
        V = poses.shape[0]
        dt = drr.BF16 if vol.dtype == torch.bfloat16 else drr.F32
        nk = 0 if transfer is None else len(transfer[0][0])
        dev = vol.device
        self.out = torch.empty((V, C, H, Wd), device=dev)
        self.aux = torch.empty_like(self.out)
        rng = np.random.default_rng(2100 + V)
        self.g = torch.from_numpy(rng.uniform(-1.0, 1.0, size=tuple(self.out.shape)).astype(
            np.float32)).to(dev)
        self.grad = torch.empty(vol.shape, device=dev)
        wf = drr.drr_render_workspace_bytes(B, C, nz, ny, nx, dt, V, H, Wd, N, mode, clip, nk, 0)
        wb = drr.drr_render_workspace_bytes(B, C, nz, ny, nx, dt, V, H, Wd, N, mode, clip, nk, 1)
        self.ws_f = torch.empty(wf, dtype=torch.uint8, device=dev) if wf else None
        self.ws_b = torch.empty(wb, dtype=torch.uint8, device=dev) if wb else None
        self.samples = V * C * H * Wd * N
        self.read_elem = 4 if (transfer is not None or dt == drr.F32) else 2
        self.plan = read_plan(wf, B, C, nz, ny, nx, self.read_elem, V, H, Wd, N, clip, nk)

    def forward(self):
        import ct_forward_projection_amd as drr
        sp, K, P, H, Wd, N, mode, f, clip, margin, tf = self.args
        drr.drr_render(self.vol, sp, K, P, H, Wd, N, mode, f, clip, margin, tf, out=self.out,
                       aux=self.aux, workspace=self.ws_f)

    def backward(self):
        import ct_forward_projection_amd as drr
        sp, K, P, H, Wd, N, mode, f, clip, margin, tf = self.args
        drr.drr_render_backward_volume(self.vol, tuple(self.vol.shape), 0, sp, K, P, H, Wd, N,
                                       mode, self.g, self.out, self.aux, f, clip, margin, tf,
                                       grad_volume=self.grad, workspace=self.ws_b)


def frontend_lines(dev):
    """The flashdrr front end (drr_render) at full size: the 16-view 200^2 batch
    rendered from the HU phantom through the transfer function (box clip with
    Beer-Lambert; near/far with a 30 mm margin and alpha compositing; fp32 and
    bf16 HU), four volumes of two channels, and the 1024^2 camera composited.
    Nominal samples count every ray's N samples (the near/far range marches
    its N samples whether or not they fall inside the volume); the HBM
    fraction prices 8 corner elements per nominal sample of the forward."""
    import torch

    import ct_forward_projection_amd as drr
    import workloads as W
    hu32 = W.hu_phantom().astype(np.float32)
    bits = W.round_to_bf16_bits(hu32)
    tf = (np.array([[-1000.0, 0.0, 1500.0]], dtype=np.float32),
          np.array([[0.0, 0.02, 0.05]], dtype=np.float32))
    w2, w3 = W.make_workload(2), W.make_workload(3)
    P2 = torch.from_numpy(w2.poses).to(dev)
    P3 = torch.from_numpy(w3.poses).to(dev)
    hu = torch.from_numpy(hu32).to(dev)[None, None]
    hub = torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)[None, None]
    mu = torch.from_numpy(w2.volume).to(dev)
    # four volumes of two channels: the mu phantom and a flipped copy, channel 2
    # a scaled copy; each volume seen by 4 of the 16 batch views
    mu4 = torch.stack([torch.stack([mu.flip(a % 3), 0.5 * mu.flip(a % 3)]) for a in range(4)])
    D = drr
    cases = [
        ("batch16x200-hu-transfer-box-BL", hu, P2, w2, D.BEER_LAMBERT, 0, tf),
        ("batch16x200-hu-transfer-nearfar30-alpha", hu, P2, w2, D.ALPHA_COMPOSITE, 1, tf),
        ("batch16x200-hu-bf16-transfer-nearfar30-alpha", hub, P2, w2, D.ALPHA_COMPOSITE, 1, tf),
        ("batch16x200-4vol-2ch-BL", mu4.contiguous(), P2, w2, D.BEER_LAMBERT, 0, None),
        ("train1024-alpha", mu[None, None], P3, w3, D.ALPHA_COMPOSITE, 0, None),
    ]
    lines = {}
    for name, vol, P, w, mode, clip, transfer in cases:
        c = RenderCase(vol, w.spacing, w.K, P, w.det_h, w.det_w, w.n_samples, mode, 1.0, clip,
                       30.0, transfer)
        c.forward()
        c.backward()
        torch.cuda.synchronize()
        f_ms, b_ms = time_graph([c.forward, c.backward])
        views = P.shape[0] * vol.shape[1]
        fwd_bytes = c.samples * 8 * c.read_elem + c.out.numel() * 8
        line = {"views_x_channels": views, "detector": [w.det_h, w.det_w],
                "n_samples": w.n_samples, "volumes": vol.shape[0], "channels": vol.shape[1],
                "dtype": "bf16" if vol.dtype == torch.bfloat16 else "f32",
                "mode": {0: "beer-lambert", 1: "line-integral", 2: "alpha"}[mode],
                "clip": "near-far-30mm" if clip else "box",
                "transfer": transfer is not None, "read": c.plan,
                "forward_ms": round(f_ms, 4), "forward_fps": round(views / f_ms * 1e3, 1),
                "forward_gsamples_s": round(c.samples / f_ms / 1e6, 1),
                "forward_hbm_frac": round(fwd_bytes / (f_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "backward_ms": round(b_ms, 4),
                "backward_gsamples_s": round(c.samples / b_ms / 1e6, 1)}
        lines[name] = line
        log(f"front end {name}: {line}")
        del c
    return lines


def pmc_pass(kind: str, dev):
    """A short fixed launch sequence for rocprofv3 counter runs: 3 launches of
    the chosen pass (forward, volume backward or pose backward) on the
    train-step workload, or a plain 1 GiB copy (the calibration kernel for the
    byte counters)."""
    import torch

    import workloads as W
    if kind == "copy":
        a = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        log("pmc copy: 3 x 1 GiB")
        return
    res = Resident(W.make_workload(3), dev)
    res.forward()
    torch.cuda.synchronize()
    run = {"forward": res.forward, "backward": res.backward, "pose": res.pose_backward}[kind]
    for _ in range(3):
        run()
    torch.cuda.synchronize()
    log(f"pmc pass: 3 x {kind}")


# ---------------------------------------------------------------- profile summaries

PROFILE_COMMANDS = {
    "trace": "rocprofv3 --kernel-trace --stats -d gpurun_out/prof/trace -o trace "
             "--output-format csv -- python3 bench.py --steps 20 --warmup 5 --no-cpu "
             "--no-workloads",
    "pmc": "rocprofv3 --pmc {counters} -d gpurun_out/prof/{kind}_{tag} -o pmc "
           "--output-format csv -- python3 bench.py --pmc-pass {kind}",
}
PMC_SETS = {
    "fetch": ["FETCH_SIZE"],
    "write": ["WRITE_SIZE", "TCC_HIT_sum", "TCC_MISS_sum"],
    "sq": ["SQ_WAVES", "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES", "SQ_INSTS_VALU", "SQ_INSTS_VMEM_RD",
           "SQ_INSTS_LDS", "SQ_ACTIVE_INST_VALU", "SQ_WAIT_INST_ANY", "GRBM_GUI_ACTIVE"],
    "ta": ["TA_TA_BUSY_sum", "TA_BUSY_avr", "TD_TD_BUSY_sum", "SQ_LDS_BANK_CONFLICT",
           "SQ_LDS_ADDR_CONFLICT"],
}
# kernels whose counters each pass reports (matched as substrings of the name)
KERNEL_KEYS = {"forward": ["drr_march_staged_kernel"],
               "backward": ["drr_fill_kernel", "drr_scatter_kernel"],
               "pose": ["drr_pose_staged_kernel"],
               "copy": ["copy"]}
PMC_KINDS = ("forward", "backward", "pose", "copy")


def _csv_rows(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _find(root, suffix):
    hits = []
    for d, _, files in os.walk(root):
        hits += [os.path.join(d, f) for f in files if f.endswith(suffix)]
    return sorted(hits)


def profile_summary(root: str):
    """Summarise rocprofv3 outputs under ``root`` (the layout PROFILE_COMMANDS
    writes) into profiles/*.md and profiles/pmc_traffic.json."""
    prof_dir = os.path.join(ROOT, "profiles")
    os.makedirs(prof_dir, exist_ok=True)
    rev = kernel_revision()
    # kernel trace statistics
    stats = _find(os.path.join(root, "trace"), "kernel_stats.csv")
    durations = {}     # kernel key -> average duration (ns) in the trace
    if stats:
        rows = _csv_rows(stats[0])
        for key in {k for keys in KERNEL_KEYS.values() for k in keys}:
            hits = [r for r in rows if key in r.get("Name", "")]
            if hits:
                best = max(hits, key=lambda r: int(r.get("Calls", 0)))
                durations[key] = float(best.get("AverageNs", 0))
        lines = ["# Kernel trace: train step on the 1024x1024 workload", "",
                 f"Command: `{PROFILE_COMMANDS['trace']}`", "",
                 f"Kernel sources revision: `{rev}`", "",
                 "| kernel | calls | average (us) | min (us) | max (us) | share |",
                 "|---|---|---|---|---|---|"]
        for r in rows:
            name = r.get("Name", r.get("KernelName", "?"))
            if len(name) > 90:
                name = name[:87] + "..."
            lines.append(f"| `{name}` | {r.get('Calls')} | {float(r.get('AverageNs', 0)) / 1e3:.2f} "
                         f"| {float(r.get('MinNs', 0)) / 1e3:.2f} | {float(r.get('MaxNs', 0)) / 1e3:.2f} "
                         f"| {float(r.get('Percentage', 0)):.1f}% |")
        path = os.path.join(prof_dir, "kernel_trace_train_step_1024.md")
        with open(path, "w") as f:
            f.write("\n".join(lines) + "\n")
        log("wrote", path)
    # counters
    values = {}   # (pass, kernel) -> counter -> per-dispatch values
    for kind in PMC_KINDS:
        for tag in PMC_SETS:
            for path in _find(os.path.join(root, f"{kind}_{tag}"), "counter_collection.csv"):
                per = {}
                for r in _csv_rows(path):
                    name = r.get("Kernel_Name", "")
                    key = next((k for k in KERNEL_KEYS[kind] if k in name), None)
                    if key is None:
                        continue
                    per_key = (key, r["Counter_Name"], r["Dispatch_Id"])
                    per[per_key] = per.get(per_key, 0.0) + float(r["Counter_Value"])
                for (key, cname, _), v in per.items():
                    values.setdefault((kind, key), {}).setdefault(cname, []).append(v)
    if not values:
        return
    med = {k: {c: float(np.median(v)) for c, v in d.items()} for k, d in values.items()}
    copy_bytes = float(1 << 30)
    fetch_factor = write_factor = None
    cm = med.get(("copy", "copy"), {})
    if cm.get("FETCH_SIZE"):
        fetch_factor = copy_bytes / (cm["FETCH_SIZE"] * 1024.0)
    if cm.get("WRITE_SIZE"):
        write_factor = copy_bytes / (cm["WRITE_SIZE"] * 1024.0)
    traffic = {"kernel_revision": rev, "fetch_calibration": fetch_factor,
               "write_calibration": write_factor, "kernels": {}}
    lines = ["# Hardware counters per dispatch (median), train-step workload 1024x1024", "",
             "Commands (one counter set per run):", ""]
    for tag, counters in PMC_SETS.items():
        lines.append("- `" + PROFILE_COMMANDS["pmc"].format(counters=" ".join(counters),
                                                            kind="<forward|backward|pose|copy>",
                                                            tag=tag) + "`")
    lines += ["", f"Kernel sources revision: `{rev}`", "",
              "Calibration: a plain 1 GiB device copy (`bench.py --pmc-pass copy`) reads "
              f"FETCH_SIZE x {fetch_factor} and WRITE_SIZE x {write_factor} of its known size "
              "(factors applied below).", ""]
    for kind in ("forward", "backward", "pose"):
        for name in KERNEL_KEYS[kind]:
            if (kind, name) not in med:
                continue
            _counter_table(lines, traffic, name, f"{kind} pass", med[(kind, name)],
                           fetch_factor, write_factor, durations.get(name))
    path = os.path.join(prof_dir, "counters_train_step_1024.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    with open(os.path.join(prof_dir, "pmc_traffic.json"), "w") as f:
        json.dump(traffic, f, indent=1)
    log("wrote", path)


MI355X_CUS, MI355X_SIMDS, MI355X_GHZ = 256, 1024, 2.4


def _counter_table(lines, traffic, name, where, m, fetch_factor, write_factor, dur_ns=None):
    """One kernel's median counters as a markdown table, plus its calibrated
    HBM bytes per launch into ``traffic``.  With the kernel's traced duration,
    VALU busy = wave instructions x 4 cycles (a wave64 instruction occupies a
    16-lane SIMD for 4 cycles) over 1024 SIMDs x the duration's cycles, and the
    LDS bank-conflict share = conflict cycles over 256 CUs x those cycles."""
    lines += [f"## {name} ({where})", "", "| counter | value |", "|---|---|"]
    for c in sorted(m):
        lines.append(f"| {c} | {m[c]:.6g} |")
    fb = m.get("FETCH_SIZE", 0.0) * 1024.0 * (fetch_factor or 1.0)
    wb = m.get("WRITE_SIZE", 0.0) * 1024.0 * (write_factor or 1.0)
    hit = m.get("TCC_HIT_sum"), m.get("TCC_MISS_sum")
    if all(h is not None for h in hit) and sum(hit) > 0:
        lines.append(f"| L2 hit rate | {hit[0] / (hit[0] + hit[1]):.4f} |")
    valu_busy = None
    if dur_ns:
        cycles = dur_ns * MI355X_GHZ
        lines.append(f"| traced duration (us) | {dur_ns / 1e3:.2f} |")
        if m.get("SQ_INSTS_VALU"):
            valu_busy = round(m["SQ_INSTS_VALU"] * 4 / (MI355X_SIMDS * cycles), 3)
            lines.append(f"| VALU busy | {valu_busy:.3f} |")
        if m.get("SQ_LDS_BANK_CONFLICT") is not None:
            lines.append(f"| LDS bank-conflict share | "
                         f"{m['SQ_LDS_BANK_CONFLICT'] / (MI355X_CUS * cycles):.3f} |")
    lines += ["", f"HBM-side traffic per launch (calibrated): read {fb / 1e6:.1f} MB, "
                  f"write {wb / 1e6:.1f} MB, total {(fb + wb) / 1e6:.1f} MB", ""]
    if fb or wb:
        traffic["kernels"][name] = {"hbm_bytes_per_launch": fb + wb, "read_bytes": fb,
                                    "write_bytes": wb, "valu_busy": valu_busy}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-workloads", action="store_true")
    ap.add_argument("--pmc-pass", choices=list(PMC_KINDS))
    ap.add_argument("--profile-summary", metavar="DIR",
                    help="summarise rocprofv3 outputs under DIR into profiles/ (CPU only)")
    args = ap.parse_args()
    if args.profile_summary:
        profile_summary(args.profile_summary)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on one GPU only; --gpus must be 1 "
              "(the multi-GPU sharding design is described in DESIGN.md)", file=sys.stderr)
        sys.exit(2)

    import torch

    import ct_forward_projection_amd as drr
    import workloads as W
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    drr.library()   # fail loudly if the HIP library is not built
    dev = torch.device("cuda:0")
    if args.pmc_pass:
        pmc_pass(args.pmc_pass, dev)
        return

    w = W.make_workload(3)
    res = Resident(w, dev)
    hits = res.hit_rays()
    log(f"bench: {w.name} on {torch.cuda.get_device_name(0)}; {hits} of {w.n_rays} rays hit")

    def step():
        res.forward()
        res.backward()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall / max(args.steps, 1) * 1e3

    # per-kernel GPU time of the same step, HIP events on the launch stream
    fwd_ms, bwd_ms = time_events([res.forward, res.backward], max(args.steps, 1))
    # each pass is one ABI call: the forward launches the corner-cell relayout
    # and the march, the backward the gradient fill and the scatter
    # the forward of this workload is one launch of the LDS-staged march
    rf = roofline("drr_march_staged_kernel", forward_bytes(res, hits), fwd_ms,
                  measured_traffic(KERNEL_KEYS["forward"]),
                  measured_valu_busy("drr_march_staged_kernel"))
    rb = roofline("drr_scatter_kernel (with gradient fill)", backward_bytes(res, hits), bwd_ms,
                  measured_traffic(KERNEL_KEYS["backward"]),
                  measured_valu_busy("drr_scatter_kernel"))
    dominant, other = (rb, rf) if bwd_ms >= fwd_ms else (rf, rb)

    out = {
        "metric": METRIC,
        "value": round(w.nominal_samples / (ms_per_step * 1e-3) / 1e9, 2),
        "unit": "Gsamples/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "volume": list(w.volume.shape), "voxel_mm": 1.0,
                   "views": w.n_views, "detector": [w.det_h, w.det_w], "n_samples": w.n_samples,
                   "output": "beer-lambert", "pass": "forward+volume-backward",
                   "parallelism": "single-gpu"},
        "fps": round(w.n_views / (ms_per_step * 1e-3), 2),
        "kernels_ms": {"forward": round(fwd_ms, 4), "backward": round(bwd_ms, 4)},
        "effective_gsamples_s": round(hits * w.n_samples / (ms_per_step * 1e-3) / 1e9, 2),
        "roofline": dominant,
        "roofline_other": other,
        "kernel_revision": kernel_revision(),
        "context": "pages' figures, other hardware: FlashDRR Triton train step 15.4 ms at "
                   "1024^2/512 (RTX 5070 Ti); nanodrr 12,600 FPS fused / 17,820 FPS bf16+compile "
                   "at 200^2 (RTX 6000 Ada); FlashDRR 9.16 ms at 2048^2/256 (RTX 5070 Ti)",
    }
    if not args.no_workloads:
        out["workloads"] = workload_lines(dev, reps=10)
        out["front_end"] = frontend_lines(dev)
    if not args.no_cpu:
        log("cpu baseline: oracle on the same step ...")
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
