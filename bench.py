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
  roofline     the dominant kernel's VALU roofline: the method's algorithmic
               VALU lane-operations per sample on rays that hit the volume
               (26 forward, 28 backward) over the pass's duration from HIP
               events on the launch stream, against MI355X's VALU issue peak
               without packed FP32 (1024 SIMDs x 16 lanes x 2.4 GHz); with the
               committed counters of the current kernel sources it also carries
               the kernel's HBM traffic, L2 hit rate, measured clock and VALU busy
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
--steps K, --warmup W, --no-cpu, --no-workloads; --profile-run CASE [--reps R]
runs one workload's passes as a short fixed launch sequence for rocprofv3
(kernel trace or counters), --profile-run CASE --meta-dir DIR records the
case's unit counts, and --profile-summary DIR turns rocprofv3's outputs into
profiles/*.md and profiles/pmc_traffic.json on the CPU.
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


def _code_only(src: str) -> str:
    """C/C++/HIP source without its comments, whitespace runs collapsed, so
    that the revision below changes with the code and not with its comments."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":                                   # string or char literal
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_revision() -> str:
    """Hash of the kernel sources' code (comments and layout excluded): the
    counters in profiles/ apply only while it is unchanged."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "ct_forward_projection_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update(name.encode() + _code_only(f.read()).encode())
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
        need_b = drr.drr_workspace_bytes(nz, ny, nx, drr.F32, w.n_views, w.det_h, w.det_w,
                                         w.n_samples, 1) if w.grad_out is not None else 0
        self.workspace_b = torch.empty(need_b, dtype=torch.uint8, device=dev) if need_b else None
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
                                w.n_samples, w.mode, self.g, self.s, grad_volume=self.grad,
                                workspace=self.workspace_b)

    def forward_reuse(self):
        """The forward reading the copy the last forward left in the workspace
        (drr_forward_reuse): a registration loop over this fixed volume."""
        import ct_forward_projection_amd as drr
        w = self.w
        drr.drr_forward(self.vol, w.spacing, w.K, self.poses, w.det_h, w.det_w, w.n_samples,
                        w.mode, out=self.out, line_integral=self.s, workspace=self.workspace,
                        reuse_copy=True)

    def pose_backward_reuse(self):
        """The pose gradient reading the copy the last pose gradient left in its
        workspace (drr_backward_pose_reuse)."""
        import ct_forward_projection_amd as drr
        w = self.w
        drr.drr_backward_pose(self.vol, w.spacing, w.K, self.poses, w.det_h, w.det_w,
                              w.n_samples, w.mode, self.pose_g, grad_poses=self.grad_poses,
                              workspace=self.pose_ws, reuse_copy=True)

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
    return hits * w.n_samples * 8 * 4 + w.n_rays * 8 + int(np.prod(w.volume.shape)) * 4


# VALU issue peak of MI355X without packed FP32 (the build switches packed-FP32
# instruction selection off): 256 CUs x 4 SIMDs, each issuing one wave64 VALU
# instruction over 4 cycles (16 lanes per cycle), at the 2.4 GHz peak engine
# clock -> 16384 lane-operations per cycle, 39.3 T lane-operations per second.
# (The published fp32 vector peak, 157.3 TFLOP/s, counts a packed FMA as four
# flops per lane and cycle.)
MI355X_CUS, MI355X_SIMDS, MI355X_GHZ, MI355X_XCDS = 256, 1024, 2.4, 8
ALU_PEAK_TOPS = MI355X_SIMDS * 16 * MI355X_GHZ * 1e9 / 1e12
# Algorithmic VALU lane-operations of one sample, the method's own work (an FMA
# counts once, a load or an atomic's memory-side add not at all):
#   forward trilinear sample: position step 3, floor 3, fractions 3, corner
#   address 2 (i + nx (j + ny k)), 7 lerps x 2 (subtract, fma), accumulate 1 = 26
#   backward sample: position 3, floor 3, fractions 3, corner address 2,
#   1 - f per axis 3, c (1 - fz) and c fz 2, four yz products 4, eight
#   x products fused with their accumulation 8 = 28
#   pose-gradient sample: the forward's 26, the trilinear gradient (three
#   bilinear differences: 3 lerps x 2 + 1 subtract each = 21), two running
#   vector sums (3 adds, 3 fmas) = 53
OPS_FORWARD_SAMPLE = 26
OPS_BACKWARD_SAMPLE = 28
OPS_POSE_SAMPLE = 53


def roofline_alu(name, ops, ms, counters=None):
    """VALU roofline of one kernel: algorithmic lane-operations (``ops`` per
    launch) over its launch duration against ALU_PEAK_TOPS.  ``counters``
    (measured at the current kernel sources, else None) add HBM traffic, L2 hit
    rate, measured VALU busy and issued/algorithmic operations."""
    achieved = ops / (ms * 1e-3) / 1e12
    r = {"kernel": name, "bound": "alu", "achieved": round(achieved, 3),
         "peak": round(ALU_PEAK_TOPS, 3), "unit": "TOP/s",
         "frac": round(achieved / ALU_PEAK_TOPS, 4),
         "ops_per_launch": int(ops), "traffic": None}
    if counters:
        r["traffic"] = counters.get("hbm_bytes_per_launch")
        for k in ("hbm_gbs", "hbm_frac", "l2_hit", "valu_busy", "valu_busy_rocprof",
                  "valu_lane_util", "clock_ghz", "issued_per_algorithmic", "lds_bank_conflict"):
            if counters.get(k) is not None:
                r[k] = counters[k]
    return r


def backward_kernel() -> str:
    """The kernel that carries the train step's volume backward."""
    return "drr_scatter_kernel"


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


def measured_counters(case, kernel):
    """Counter-derived figures of one kernel in one profile case from the
    committed summary (None if absent or taken on other kernel sources)."""
    d = _committed_counters()
    if d is None:
        return None
    return d.get("cases", {}).get(case, {}).get(kernel)


def cpu_model() -> str:
    """The host CPU as /proc/cpuinfo names it, with its family, model and
    stepping numbers (a virtual machine may report only the vendor's brand)."""
    fields = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if not line.strip():
                    break                        # the first processor's block is enough
                k, _, v = line.partition(":")
                fields.setdefault(k.strip(), v.strip())
    except OSError:
        return "unknown"
    name = fields.get("model name", "unknown")
    ids = [f"{k} {fields[k]}" for k in ("cpu family", "model", "stepping") if k in fields]
    return name + (f" ({', '.join(ids)})" if ids else "")


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
            "cpu_model": cpu_model(),
            "seconds": round(dt, 2),
            "sample": f"the whole step: {w.name} forward + volume gradient, fp64, "
                      f"{threads} threads forward / {used} threads scatter"}


def workload_lines(dev, reps):
    import workloads as W
    lines = {}
    for i, bf16 in [(1, False), (2, False), (2, True), (3, False), (4, False), (5, False)]:
        w = W.make_workload(i, with_bf16=bf16)
        if i == 2 and not bf16:
            # the batch's volume backward (views sparse against the voxels), for an
            # upstream gradient U[-1, 1) seeded as the profile case's
            w.grad_out = np.random.default_rng(2100 + w.n_views).uniform(
                -1.0, 1.0, size=(w.n_views, w.det_h, w.det_w)).astype(np.float32)
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
                "forward_alu_frac": round(hits * w.n_samples * OPS_FORWARD_SAMPLE /
                                          (fwd_ms * 1e-3) / 1e12 / ALU_PEAK_TOPS, 4),
                "hit_rays": hits}
        if with_pose:
            pose_ms = t.pop()
            line["pose_backward_ms"] = round(pose_ms, 4)
            line["pose_backward_gsamples_s"] = round(w.nominal_samples / pose_ms / 1e6, 1)
            line["pose_backward_alu_frac"] = round(hits * w.n_samples * OPS_POSE_SAMPLE /
                                                   (pose_ms * 1e-3) / 1e12 / ALU_PEAK_TOPS, 4)
            line["registration_step_fps"] = round(w.n_views / (fwd_ms + pose_ms) * 1e3, 1)
            if res.workspace is not None:
                # a registration loop over the fixed volume: both calls read the
                # copies the previous step left in their workspaces
                res.forward()
                tr = time_graph([res.forward_reuse, res.pose_backward_reuse])
                line["forward_reuse_ms"] = round(tr[0], 4)
                line["forward_reuse_fps"] = round(w.n_views / tr[0] * 1e3, 1)
                line["pose_backward_reuse_ms"] = round(tr[1], 4)
                line["registration_step_reuse_fps"] = round(w.n_views / (tr[0] + tr[1]) * 1e3, 1)
        if len(t) > 1:
            line["backward_ms"] = round(t[1], 4)
            line["backward_gsamples_s"] = round(w.nominal_samples / t[1] / 1e6, 1)
            line["backward_alu_frac"] = round(hits * w.n_samples * OPS_BACKWARD_SAMPLE /
                                              (t[1] * 1e-3) / 1e12 / ALU_PEAK_TOPS, 4)
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
        wp = drr.drr_render_workspace_bytes(B, C, nz, ny, nx, dt, V, H, Wd, N, mode, clip, nk, 2)
        self.ws_f = torch.empty(wf, dtype=torch.uint8, device=dev) if wf else None
        self.ws_b = torch.empty(wb, dtype=torch.uint8, device=dev) if wb else None
        self.ws_p = torch.empty(wp, dtype=torch.uint8, device=dev)
        self.grad_poses = torch.empty((V, 3, 4), device=dev)
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

    def pose_backward(self, reuse_copy=False):
        import ct_forward_projection_amd as drr
        sp, K, P, H, Wd, N, mode, f, clip, margin, tf = self.args
        drr.drr_render_backward_pose(self.vol, sp, K, P, H, Wd, N, mode, self.g, f, clip, margin,
                                     tf, grad_poses=self.grad_poses, workspace=self.ws_p,
                                     reuse_copy=reuse_copy)

    def forward_reuse(self):
        """The render reading the copy the last render left in its workspace."""
        import ct_forward_projection_amd as drr
        sp, K, P, H, Wd, N, mode, f, clip, margin, tf = self.args
        drr.drr_render(self.vol, sp, K, P, H, Wd, N, mode, f, clip, margin, tf, out=self.out,
                       aux=self.aux, workspace=self.ws_f, reuse_copy=True)

    def pose_backward_reuse(self):
        self.pose_backward(reuse_copy=True)


def frontend_lines(dev):
    """The flashdrr front end (drr_render) at full size: the 16-view 200^2 batch
    rendered from the HU phantom through the transfer function (box clip with
    Beer-Lambert; near/far with a 30 mm margin and alpha compositing; fp32 and
    bf16 HU), four volumes of two channels, and the 1024^2 camera composited.
    Nominal samples count every ray's N samples (the near/far range marches
    its N samples whether or not they fall inside the volume); the ALU
    fraction prices the forward's algorithmic operations per nominal sample."""
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
        c.pose_backward()
        torch.cuda.synchronize()
        f_ms, b_ms, p_ms = time_graph([c.forward, c.backward, c.pose_backward])
        views = P.shape[0] * vol.shape[1]
        line = {"views_x_channels": views, "detector": [w.det_h, w.det_w],
                "n_samples": w.n_samples, "volumes": vol.shape[0], "channels": vol.shape[1],
                "dtype": "bf16" if vol.dtype == torch.bfloat16 else "f32",
                "mode": {0: "beer-lambert", 1: "line-integral", 2: "alpha"}[mode],
                "clip": "near-far-30mm" if clip else "box",
                "transfer": transfer is not None, "read": c.plan,
                "forward_ms": round(f_ms, 4), "forward_fps": round(views / f_ms * 1e3, 1),
                "forward_gsamples_s": round(c.samples / f_ms / 1e6, 1),
                "forward_alu_frac_nominal": round(c.samples * OPS_FORWARD_SAMPLE / (f_ms * 1e-3)
                                                  / 1e12 / ALU_PEAK_TOPS, 4),
                "backward_ms": round(b_ms, 4),
                "backward_gsamples_s": round(c.samples / b_ms / 1e6, 1),
                "pose_backward_ms": round(p_ms, 4),
                "pose_backward_gsamples_s": round(c.samples / p_ms / 1e6, 1),
                "registration_step_fps": round(views / (f_ms + p_ms) * 1e3, 1)}
        if c.ws_f is not None:
            # a registration loop over the fixed volume: both calls read the
            # copies the previous step left in their workspaces
            c.forward()
            c.pose_backward()
            fr_ms, pr_ms = time_graph([c.forward_reuse, c.pose_backward_reuse])
            line["forward_reuse_ms"] = round(fr_ms, 4)
            line["forward_reuse_fps"] = round(views / fr_ms * 1e3, 1)
            line["pose_backward_reuse_ms"] = round(pr_ms, 4)
            line["registration_step_reuse_fps"] = round(views / (fr_ms + pr_ms) * 1e3, 1)
        lines[name] = line
        log(f"front end {name}: {line}")
        del c
    return lines


# ---------------------------------------------------------------- profile runs

# Profile cases: every workload's passes, each run as a fixed short launch
# sequence (``--profile-run CASE``) under rocprofv3 -- one kernel-trace run and
# one run per counter set -- then summarised on the CPU (``--profile-summary``).
#   name: (workload, bf16 volume, passes)
PROFILE_CASES = {
    "tiny64": (1, False, ("forward",)),
    "batch200_f32": (2, False, ("forward", "backward", "pose")),
    "batch200_bf16": (2, True, ("forward",)),
    "train1024": (3, False, ("forward", "backward", "pose")),
    "hires2048": (4, False, ("forward",)),
    "helix360": (5, False, ("forward", "backward")),
    "siddon1024": (3, False, ("siddon_forward", "siddon_backward")),
    "siddon200": (2, False, ("siddon_forward", "siddon_backward")),
}
PROFILE_COMMANDS = {
    "trace": "rocprofv3 --kernel-trace --stats -d gpurun_out/prof/{case}/trace -o trace "
             "--output-format csv -- python3 bench.py --profile-run {case} --reps 10",
    "pmc": "rocprofv3 --pmc {counters} -d gpurun_out/prof/{case}/{tag} -o pmc "
           "--output-format csv -- python3 bench.py --profile-run {case} --reps 3",
}
# The default bench command itself under the kernel tracer: the trace's average
# launch durations sit beside the event-timed per-pass figures of the same run.
BENCH_STEP_CASE = "bench_step"
BENCH_TRACE_COMMAND = ("rocprofv3 --kernel-trace --stats -d gpurun_out/prof/bench_step/trace "
                       "-o trace --output-format csv -- python3 bench.py --no-workloads --no-cpu")
PMC_SETS = {
    "fetch": ["FETCH_SIZE"],
    "write": ["WRITE_SIZE", "TCC_HIT_sum", "TCC_MISS_sum"],
    "sq": ["SQ_WAVES", "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES", "SQ_INSTS_VALU", "SQ_INSTS_VMEM_RD",
           "SQ_INSTS_LDS", "SQ_ACTIVE_INST_VALU", "SQ_WAIT_INST_ANY", "GRBM_GUI_ACTIVE"],
    "ta": ["TA_TA_BUSY_sum", "TA_BUSY_avr", "TD_TD_BUSY_sum", "SQ_LDS_BANK_CONFLICT",
           "SQ_LDS_ADDR_CONFLICT"],
    # rocprofv3's own derived metrics: VALUBusy = 100 sum(SQ_ACTIVE_INST_VALU) / CU_NUM /
    # max(GRBM_GUI_ACTIVE); VALUUtilization = 100 sum(SQ_THREAD_CYCLES_VALU) /
    # (sum(SQ_ACTIVE_INST_VALU) x 64), the active lanes of the VALU instructions
    "valu": ["VALUBusy", "VALUUtilization"],
}
COPY_CASE = "copy1gib"          # the calibration run of the byte counters


def _case_resident(case, dev):
    import workloads as W
    wi, bf16, passes = PROFILE_CASES[case]
    w = W.make_workload(wi, with_bf16=bf16)
    if w.grad_out is None and any(p in ("backward", "siddon_backward") for p in passes):
        # upstream gradient of the batch's volume backward: U[-1, 1), seeded as
        # the front-end lines' (2100 + views)
        w.grad_out = np.random.default_rng(2100 + w.n_views).uniform(
            -1.0, 1.0, size=(w.n_views, w.det_h, w.det_w)).astype(np.float32)
    return Resident(w, dev, bf16=bf16), passes


def profile_run(case: str, reps: int, dev, meta_dir=None):
    """The fixed launch sequence of a profile case: every pass once (warm-up),
    then ``reps`` launches of each pass in turn.  With ``meta_dir`` it also
    writes the case's unit counts (hit rays, samples, voxels, ray-voxel pieces)
    as meta.json for the summary (no profiler attached)."""
    import torch
    if case == COPY_CASE:
        a = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        for _ in range(reps):
            b.copy_(a)
        torch.cuda.synchronize()
        log(f"profile run: {reps} x 1 GiB copy")
        return
    res, passes = _case_resident(case, dev)
    fns = {"forward": res.forward, "backward": res.backward, "pose": res.pose_backward,
           "siddon_forward": res.siddon_forward, "siddon_backward": res.siddon_backward}
    res.forward()
    if "siddon_backward" in passes:
        res.siddon_forward()
    for p in passes:
        fns[p]()
    torch.cuda.synchronize()
    if meta_dir is not None:
        w = res.w
        meta = {"case": case, "workload": w.name, "views": w.n_views, "det": [w.det_h, w.det_w],
                "n_samples": w.n_samples, "volume": list(w.volume.shape),
                "dtype": "bf16" if res.elem_bytes == 2 else "f32", "passes": list(passes),
                "hit_rays": res.hit_rays(), "rays": w.n_rays,
                "voxels": int(np.prod(w.volume.shape)), "kernel_revision": kernel_revision()}
        if any(p.startswith("siddon") for p in passes):
            meta["siddon_pieces"] = siddon_pieces(w)
        os.makedirs(meta_dir, exist_ok=True)
        with open(os.path.join(meta_dir, "meta.json"), "w") as f:
            json.dump(meta, f, indent=1)
        log(f"profile meta: {meta}")
        return
    for p in passes:
        for _ in range(reps):
            fns[p]()
        torch.cuda.synchronize()
    log(f"profile run: {case}: {reps} x {', '.join(passes)}")


# what one launch of each kernel computes, for its roofline in the summaries:
# (unit, ops per unit or None, algorithmic bytes per unit)
def _kernel_units(short, meta):
    eff = meta["hit_rays"] * meta["n_samples"]
    elem = 2 if meta["dtype"] == "bf16" else 4
    nz, ny, nx = meta["volume"]
    if short in ("drr_march_staged_kernel", "drr_march_kernel"):
        return "sample on a hit ray", eff, OPS_FORWARD_SAMPLE, 8 * elem
    if short in ("drr_scatter_kernel", "drr_brick_scatter_kernel"):
        return "sample on a hit ray", eff, OPS_BACKWARD_SAMPLE, 32
    if short in ("drr_pose_staged_kernel", "drr_pose_grad_kernel"):
        return "sample on a hit ray", eff, OPS_POSE_SAMPLE, 8 * elem
    if short == "drr_zpair_kernel":
        return "voxel pair", nx * ny * (nz - 1), None, 4 * elem
    if short == "drr_cells_kernel":
        return "cell", (nx + 1) * (ny + 1) * (nz + 1), None, 16 * elem
    if short == "drr_fill_kernel":
        return "voxel", meta["voxels"], None, 4
    if short in ("drr_siddon_march_kernel", "drr_siddon_scatter_kernel",
                 "drr_siddon_brick_kernel"):
        return "ray-voxel piece", meta.get("siddon_pieces", 0), None, elem
    return None


def _csv_rows(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _find(root, suffix):
    hits = []
    for d, _, files in os.walk(root):
        hits += [os.path.join(d, f) for f in files if f.endswith(suffix)]
    return sorted(hits)


def _short_name(name: str) -> str:
    """drr kernel name without namespace and template arguments."""
    import re
    m = re.search(r"drr::(drr_\w+?)(<|\()", name)
    return m.group(1) if m else name.split("(")[0][:60]


def _median_counters(root):
    """kernel short name -> counter -> median over its dispatches."""
    values = {}
    for tag in PMC_SETS:
        for path in _find(os.path.join(root, tag), "counter_collection.csv"):
            per = {}
            for r in _csv_rows(path):
                key = (_short_name(r.get("Kernel_Name", "")), r["Counter_Name"], r["Dispatch_Id"])
                per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
            for (kname, cname, _), v in per.items():
                values.setdefault(kname, {}).setdefault(cname, []).append(v)
    return {k: {c: float(np.median(v)) for c, v in d.items()} for k, d in values.items()}


def _trace_stats(trace_dir):
    """drr kernel short name -> calls, total, min, max (ns) from a kernel_stats.csv."""
    stats = _find(trace_dir, "kernel_stats.csv")
    trace = {}
    for r in (_csv_rows(stats[0]) if stats else []):
        short = _short_name(r.get("Name", ""))
        if short.startswith("drr_"):
            t = trace.setdefault(short, {"calls": 0, "total_ns": 0.0, "min": 1e30, "max": 0.0})
            t["calls"] += int(r.get("Calls", 0))
            t["total_ns"] += float(r.get("TotalDurationNs", 0) or 0) or \
                float(r.get("AverageNs", 0)) * int(r.get("Calls", 0))
            t["min"] = min(t["min"], float(r.get("MinNs", 0)))
            t["max"] = max(t["max"], float(r.get("MaxNs", 0)))
    return trace


def bench_step_summary(root: str, prof_dir: str, rev: str):
    """profiles/<backward kernel>__bench_step.md from the traced default bench
    run (root/bench_step/trace) and the JSON line it printed
    (root/bench_step/bench.json): the trace's average durations of the step's
    two kernels beside the run's own event-timed passes."""
    croot = os.path.join(root, BENCH_STEP_CASE)
    trace = _trace_stats(os.path.join(croot, "trace"))
    if not trace:
        return
    line = None
    try:
        with open(os.path.join(croot, "bench.json")) as f:
            for raw in f:
                if raw.startswith("{"):
                    line = json.loads(raw)
    except (OSError, ValueError):
        line = None
    bk = backward_kernel()
    lines = [f"# {bk} and the other kernels of the default bench run", "",
             "Command:", "", "- `" + BENCH_TRACE_COMMAND + "`", "",
             f"Kernel sources revision: `{rev}`.  Every launch of the run is traced: warm-up, the "
             "timed steps, the per-pass event timing and the hit-ray count (one "
             "`drr_march_kernel` launch of one sample per ray).", "",
             "| kernel | calls | avg (us) | min | max |", "|---|---|---|---|---|"]
    for short, t in sorted(trace.items(), key=lambda kv: -kv[1]["total_ns"]):
        lines.append(f"| `{short}` | {t['calls']} | {t['total_ns'] / max(t['calls'], 1) / 1e3:.2f} "
                     f"| {t['min'] / 1e3:.2f} | {t['max'] / 1e3:.2f} |")
    if line is not None:
        km = line.get("kernels_ms", {})
        lines += ["", "The same run's JSON line (HIP events on the launch stream, mean over the "
                      "timed steps): "
                      f"forward {km.get('forward')} ms (`drr_march_staged_kernel`), backward "
                      f"{km.get('backward')} ms (`drr_fill_kernel` + `{bk}`); "
                      f"{line.get('ms_per_step')} ms per step, {line.get('value')} "
                      f"{line.get('unit')}; dominant-kernel roofline: "
                      f"{json.dumps(line.get('roofline'))}."]
    path = os.path.join(prof_dir, f"{bk}__{BENCH_STEP_CASE}.md")
    with open(path, "w") as fo:
        fo.write("\n".join(lines) + "\n")
    log("wrote", path)


def profile_summary(root: str):
    """Summarise the rocprofv3 outputs under ``root`` (PROFILE_COMMANDS' layout:
    root/<case>/trace, root/<case>/<counter set>, root/<case>/meta.json) into
    profiles/<dominant kernel>__<case>.md and profiles/pmc_traffic.json."""
    prof_dir = os.path.join(ROOT, "profiles")
    os.makedirs(prof_dir, exist_ok=True)
    rev = kernel_revision()
    copy = _median_counters(os.path.join(root, COPY_CASE))
    # the copy kernel: the one that fetches the most (the run also fills its source)
    cm = max(copy.values(), key=lambda m: m.get("FETCH_SIZE", 0.0) + m.get("WRITE_SIZE", 0.0),
             default={})
    copy_bytes = float(1 << 30)
    fetch_factor = copy_bytes / (cm["FETCH_SIZE"] * 1024.0) if cm.get("FETCH_SIZE") else None
    write_factor = copy_bytes / (cm["WRITE_SIZE"] * 1024.0) if cm.get("WRITE_SIZE") else None
    traffic = {"kernel_revision": rev, "fetch_calibration": fetch_factor,
               "write_calibration": write_factor, "alu_peak_tops": ALU_PEAK_TOPS, "cases": {}}
    for case in PROFILE_CASES:
        croot = os.path.join(root, case)
        try:
            with open(os.path.join(croot, "meta.json")) as f:
                meta = json.load(f)
        except OSError:
            continue
        trace = _trace_stats(os.path.join(croot, "trace"))
        med = _median_counters(croot)
        rows, figures = [], {}
        for short, t in sorted(trace.items(), key=lambda kv: -kv[1]["total_ns"]):
            avg_ns = t["total_ns"] / max(t["calls"], 1)
            m = med.get(short, {})
            f = {"avg_us": round(avg_ns / 1e3, 2), "calls": t["calls"]}
            fb = m.get("FETCH_SIZE", 0.0) * 1024.0 * (fetch_factor or 1.0)
            wb = m.get("WRITE_SIZE", 0.0) * 1024.0 * (write_factor or 1.0)
            if "FETCH_SIZE" in m or "WRITE_SIZE" in m:
                f["hbm_bytes_per_launch"] = round(fb + wb)
                f["hbm_read_bytes"] = round(fb)
                f["hbm_write_bytes"] = round(wb)
                f["hbm_gbs"] = round((fb + wb) / (avg_ns * 1e-9) / 1e9, 1)
                f["hbm_frac"] = round(f["hbm_gbs"] / HBM_PEAK_GBS, 4)
            hit, miss = m.get("TCC_HIT_sum"), m.get("TCC_MISS_sum")
            if hit is not None and miss is not None and hit + miss > 0:
                f["l2_hit"] = round(hit / (hit + miss), 4)
            if m.get("GRBM_GUI_ACTIVE"):
                # GRBM_GUI_ACTIVE is summed over the XCDs
                f["clock_ghz"] = round(m["GRBM_GUI_ACTIVE"] / MI355X_XCDS / avg_ns, 3)
            if m.get("SQ_INSTS_VALU") and f.get("clock_ghz"):
                cycles = avg_ns * f["clock_ghz"]
                f["valu_busy"] = round(m["SQ_INSTS_VALU"] * 4 / (MI355X_SIMDS * cycles), 3)
            if m.get("VALUBusy") is not None:
                f["valu_busy_rocprof"] = round(m["VALUBusy"] / 100.0, 3)
            if m.get("VALUUtilization") is not None:
                f["valu_lane_util"] = round(m["VALUUtilization"] / 100.0, 3)
            if m.get("SQ_LDS_BANK_CONFLICT") is not None and f.get("clock_ghz"):
                f["lds_bank_conflict"] = round(
                    m["SQ_LDS_BANK_CONFLICT"] / (MI355X_CUS * avg_ns * f["clock_ghz"]), 3)
            u = _kernel_units(short, meta)
            if u is not None:
                unit, n_units, ops, abytes = u
                f["unit"], f["units_per_launch"] = unit, int(n_units)
                f["alg_bytes_per_launch"] = int(n_units * abytes)
                if ops is not None:
                    f["alg_ops_per_launch"] = int(n_units * ops)
                    f["alu_tops"] = round(n_units * ops / (avg_ns * 1e-9) / 1e12, 3)
                    f["alu_frac"] = round(f["alu_tops"] / ALU_PEAK_TOPS, 4)
                    if m.get("SQ_INSTS_VALU"):
                        f["issued_per_algorithmic"] = round(m["SQ_INSTS_VALU"] * 64 /
                                                            (n_units * ops), 3)
            figures[short] = f
            rows.append((short, t, m, f))
        traffic["cases"][case] = figures
        if not rows:
            continue
        # the file is named for the slowest kernel of the case's forward and
        # backward passes (the pose pass, when the case has others, times alike
        # and would swap the name from run to run)
        named = [r[0] for r in rows if not (r[0].startswith("drr_pose") and len(meta["passes"]) > 1)]
        dominant = named[0] if named else rows[0][0]
        lines = [f"# {dominant} and the other kernels of `{case}` ({meta['workload']})", "",
                 f"Workload: volume {meta['volume']} {meta['dtype']}, {meta['views']} view(s) "
                 f"{meta['det'][0]}x{meta['det'][1]}, {meta['n_samples']} samples per ray; "
                 f"{meta['hit_rays']} of {meta['rays']} rays hit the volume; passes: "
                 f"{', '.join(meta['passes'])}.", "",
                 "Commands:", "",
                 "- `" + PROFILE_COMMANDS["trace"].format(case=case) + "`"]
        for tag, counters in PMC_SETS.items():
            lines.append("- `" + PROFILE_COMMANDS["pmc"].format(counters=" ".join(counters),
                                                                case=case, tag=tag) + "`")
        lines += ["", f"Kernel sources revision: `{rev}`.  Byte counters calibrated by a plain "
                      f"1 GiB copy: FETCH_SIZE x {fetch_factor}, WRITE_SIZE x {write_factor}.",
                  "", f"ALU roofline: algorithmic VALU lane-operations per launch over the traced "
                      f"average duration, against {ALU_PEAK_TOPS:.2f} TOP/s (1024 SIMDs x 16 lanes "
                      f"x 2.4 GHz, no packed FP32).  VALU busy: SQ_INSTS_VALU x 4 cycles over 1024 "
                      f"SIMDs x the duration at the measured clock (GRBM_GUI_ACTIVE / 8 XCDs / "
                      f"duration).  VALUBusy and VALU lanes: rocprofv3's derived VALUBusy and "
                      f"VALUUtilization (as fractions).", "",
                  "| kernel | calls | avg (us) | min | max | unit x count | ALU TOP/s | ALU frac | "
                  "VALU busy | VALUBusy | VALU lanes | issued/alg | clock GHz | HBM MB/launch | "
                  "HBM GB/s | L2 hit | LDS conflict |",
                  "|---|---|---|---|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
        for short, t, m, f in rows:
            fmt = lambda k, d=3: "" if f.get(k) is None else f"{f[k]:.{d}f}"
            unit = f"{f['unit']} x {f['units_per_launch']}" if "unit" in f else ""
            mb = "" if "hbm_bytes_per_launch" not in f else f"{f['hbm_bytes_per_launch'] / 1e6:.1f}"
            lines.append(f"| `{short}` | {t['calls']} | {f['avg_us']:.2f} | {t['min'] / 1e3:.2f} "
                         f"| {t['max'] / 1e3:.2f} | {unit} | {fmt('alu_tops')} | "
                         f"{fmt('alu_frac', 4)} | {fmt('valu_busy')} | "
                         f"{fmt('valu_busy_rocprof')} | {fmt('valu_lane_util')} | "
                         f"{fmt('issued_per_algorithmic')} | {fmt('clock_ghz')} | {mb} | "
                         f"{fmt('hbm_gbs', 1)} | {fmt('l2_hit', 4)} | "
                         f"{fmt('lds_bank_conflict')} |")
        lines += ["", "Raw counters (median per dispatch):", ""]
        for short, t, m, f in rows:
            if not m:
                continue
            lines.append(f"- `{short}`: " + ", ".join(f"{c} {m[c]:.6g}" for c in sorted(m)))
        path = os.path.join(prof_dir, f"{dominant}__{case}.md")
        with open(path, "w") as fo:
            fo.write("\n".join(lines) + "\n")
        log("wrote", path)
    if traffic["cases"]:              # a root with the bench run only keeps the case counters
        with open(os.path.join(prof_dir, "pmc_traffic.json"), "w") as fo:
            json.dump(traffic, fo, indent=1)
    bench_step_summary(root, prof_dir, rev)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-workloads", action="store_true")
    ap.add_argument("--profile-run", metavar="CASE", choices=list(PROFILE_CASES) + [COPY_CASE],
                    help="run one profile case's fixed launch sequence (for rocprofv3)")
    ap.add_argument("--reps", type=int, default=3)
    ap.add_argument("--meta-dir", metavar="DIR",
                    help="with --profile-run: write the case's unit counts to DIR/meta.json")
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
    if args.profile_run:
        profile_run(args.profile_run, args.reps, dev, args.meta_dir)
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

    # per-pass GPU time of the same step, HIP events on the launch stream; each
    # pass is one ABI call: the forward is one launch of the LDS-staged march,
    # the backward the gradient pass named by backward_kernel()
    fwd_ms, bwd_ms = time_events([res.forward, res.backward], max(args.steps, 1))
    eff = hits * w.n_samples
    fk, bk = "drr_march_staged_kernel", backward_kernel()
    rf = roofline_alu(fk, eff * OPS_FORWARD_SAMPLE, fwd_ms, measured_counters("train1024", fk))
    rb = roofline_alu(bk, eff * OPS_BACKWARD_SAMPLE, bwd_ms, measured_counters("train1024", bk))
    rf["algorithmic_gbs"] = round(forward_bytes(res, hits) / (fwd_ms * 1e-3) / 1e9, 1)
    rb["algorithmic_gbs"] = round(backward_bytes(res, hits) / (bwd_ms * 1e-3) / 1e9, 1)
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
