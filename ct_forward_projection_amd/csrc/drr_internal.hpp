// drr_internal.hpp -- what the C-ABI layer passes to the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>

#include "drr_device.hpp"

namespace drr {

constexpr int kBeerLambert = 0;
constexpr int kLineIntegral = 1;
constexpr int kAlpha = 2;          // front-to-back alpha compositing
constexpr int kClipBox = 0;        // per-ray box clip
constexpr int kClipNearFar = 1;    // per-view near/far range, zero padding

// Per-channel piecewise-linear transfer function (flashdrr API, Transfer
// functions, piecewise_linear_channelwise): channel c's knots are entries
// [c * knots, (c + 1) * knots); m holds each segment's slope.  The map is
// applied to voxels before sampling.
constexpr int kMaxTransferEntries = 128;
struct TransferFn {
    int knots;
    float xp[kMaxTransferEntries];
    float yp[kMaxTransferEntries];
    float m[kMaxTransferEntries];
};

// Validated call arguments, already converted to the kernels' form.
struct LaunchArgs {
    VolumeDesc V;
    Intrinsics K;
    const float* poses;   // device, n_views x 12
    int n_views, H, W, N, mode;
    // front end: n_volumes volumes of C channels, density factor, clip mode,
    // transfer function (single volume, factor 1, box clip, none by default)
    int n_volumes, C;
    float f;
    int clip;
    float margin;
    bool has_tf;
    TransferFn tf;
};

// How the forward reads the volume.  The corner-cell copy (8 elements per
// trilinear cell, clamp to edge baked in) turns a sample into one (bf16) or two
// (fp32) 16-byte loads, but is 8x the volume and costs a relayout pass, so it
// pays only when samples reuse cells: measured on MI355X, from about 16
// samples per cell for fp32 (a 256^3 volume at 1024^2 x 512 samples: 1.48 ms
// -> 0.89 ms including the relayout; a 16 x 200^2 x 256 batch, ~10 samples per
// cell, got slower) and about 4 for bf16.  It must also fit 32-bit offsets.
//
// How a render call reads its volumes: the march reads either the caller's
// volumes, a corner-cell copy (the reuse rule above; always in the near/far
// mode, whose cells carry the zero padding), or -- with a transfer function
// and no cells -- an fp32 copy of the mapped volumes.  One channel-volume of
// what the march reads is per_volume_bytes (256-byte multiple in the
// workspace); workspace_bytes covers all n_volumes * C of them.
struct RenderPlan {
    bool staged;             // forward: LDS-staged boxes of the caller's volumes (no workspace)
    bool cells;
    bool zpair;              // the march reads the z-pair copy (Layout::ZPair)
    bool padded;             // ... zero-padded (near/far mode)
    bool mapped;             // the march reads fp32 mu made by the transfer function
    int read_elem;           // element bytes the march reads
    size_t per_volume_bytes;
    size_t workspace_bytes;
    bool fits;               // every channel-volume fits 32-bit byte offsets
};

// The forward and the pose gradient (allow_staged) may instead stage boxes of
// the caller's volumes in LDS, tile by tile (box clip, one lane per ray, i.e.
// launches of at least 65,536 rays): that needs neither a relayout pass nor a
// workspace, and the transfer function is applied as the boxes are filled.
// Staging pays when the rays of one tile are dense against the voxels, which
// the samples one view puts per cell measure.  Measured on MI355X, staged
// against the best copy: 1024^2 x 512 samples over 256^3 (32 per view-cell)
// 0.45 against 0.85 ms; the 360-view 256 x 384 helix over 128^3 at 256 samples
// (11.7) 10.0 against 11.0 ms, at 128 (5.9) 6.4 against 5.6 ms and at 64 (2.9)
// 6.8 against 3.4 ms; 16 views of 512^2 x 256 over 256^3 (3.9) 2.7 against
// 1.7 ms.  The crossover lies between 6 and 12 per view-cell.
constexpr long long kStagedMinRays = 65536;
constexpr double kStagedMinViewReuse = 8.0;

// Read plans of the other launches, by the samples the launch puts per cell of
// each volume: at 16 or more the corner-cell copy (eight values per cell, one
// or two loads per sample); from 4 the z-pair copy (twice the volume, written
// once; two loads per sample instead of four); below that the volume itself.
// Measured on MI355X: the 360-view 128^3 helix (4,200 per cell) reads cells in
// 11.0 ms against 15.0 ms from z-pairs; the 16-view 200^2 batch over 256^3 (9.6
// per cell) renders in 0.65 ms from z-pairs against 0.79 ms from the volume
// (fp32) and 0.51 ms against 0.74 ms from bf16 cells (bf16), whose 8x copy
// does not stay in the last-level cache as the z-pairs do; a 64^2 x 128 view
// of 64^3 (1.9 per cell) took 7.7 us with the copy against 6.0 us without, and
// 4 volumes x 2 channels of 4 such 200^2 views (2.4 per cell) 1.81 against 1.64 ms.
constexpr double kCellsMinReuse = 16.0;
constexpr double kZPairMinReuse = 4.0;

inline RenderPlan plan_render(int n_volumes, int C, int nz, int ny, int nx, int elem_bytes,
                              int n_views, int H, int W, int N, int clip, bool has_tf,
                              bool allow_staged = false)
{
    RenderPlan p{};
    p.mapped = has_tf;
    p.read_elem = has_tf ? 4 : elem_bytes;
    const double n_cells = (double)(nx + 1) * (double)(ny + 1) * (double)(nz + 1);
    const double cell_bytes = n_cells * 8.0 * p.read_elem;
    const double lin_bytes = (double)nx * (double)ny * (double)nz * p.read_elem;
    const long long rays_per_volume =
        n_volumes > 0 ? (long long)(n_views / n_volumes) * H * W : 0;
    const double samples_per_cell = (double)rays_per_volume * (double)N / n_cells;
    const double min_reuse = kCellsMinReuse;
    const bool cells_fit = cell_bytes < 4294967040.0;
    const bool reuse = rays_per_volume > 0 && samples_per_cell >= min_reuse;
    const double view_reuse = (double)H * (double)W * (double)N / n_cells;
    if (allow_staged && clip == kClipBox && view_reuse >= kStagedMinViewReuse &&
        (long long)n_views * C * H * W >= kStagedMinRays) {
        p.staged = true;
        p.mapped = false;
        p.read_elem = elem_bytes;
        p.per_volume_bytes = (size_t)((double)nx * ny * nz * elem_bytes);
        p.workspace_bytes = 0;
        p.fits = true;
        return p;
    }
    double zpair_bytes;
    if (clip == kClipNearFar) {
        // zero padding needs a copy: corner cells where they are reused
        // enough, else the zero-padded z-pairs (about 2x the volume)
        zpair_bytes = (double)(nx + 2) * (ny + 2) * (nz + 1) * 2.0 * p.read_elem;
        const bool zpair_fit = zpair_bytes < 4294967040.0;
        p.cells = (reuse || !zpair_fit) && cells_fit;
        p.zpair = p.padded = !p.cells && zpair_fit;
        if (!p.cells && !p.zpair) p.cells = true;            // reported as not fitting
    } else {
        zpair_bytes = (double)nx * ny * (nz - 1) * 2.0 * p.read_elem;
        p.cells = reuse && cells_fit;
        p.zpair = !p.cells && nx >= 2 && nz >= 2 && rays_per_volume > 0 &&
                  samples_per_cell >= kZPairMinReuse && zpair_bytes < 4294967040.0;
    }
    p.fits = p.cells ? cells_fit : (p.zpair ? true : lin_bytes < 4294967040.0);
    const double nv = (double)n_volumes * (double)C;
    if (p.cells) {
        p.per_volume_bytes = ((size_t)cell_bytes + 255) & ~(size_t)255;
        p.workspace_bytes = (size_t)(nv * (double)p.per_volume_bytes);
    } else if (p.zpair) {
        p.per_volume_bytes = ((size_t)zpair_bytes + 255) & ~(size_t)255;
        p.workspace_bytes = (size_t)(nv * (double)p.per_volume_bytes);
    } else if (p.mapped) {
        p.per_volume_bytes = ((size_t)lin_bytes + 255) & ~(size_t)255;
        p.workspace_bytes = (size_t)(nv * (double)p.per_volume_bytes);
    } else {
        p.per_volume_bytes = (size_t)lin_bytes;
        p.workspace_bytes = 0;
    }
    return p;
}

// Side of the bricks of the brick-owned backward (drr_brick.hip): B^3 voxels
// per workgroup, an LDS copy of (B + 2)^3 int64 entries.  Measured on MI355X
// (16 views of 200^2 x 256 samples over 256^3): 1.73 ms at B = 12 (four
// workgroups per CU), 2.10 ms at B = 16 (two).
constexpr int kBrickSide = 12;
constexpr double kBrickMergeMinViewReuse = 2.0;
// Views sparse against the voxels (fewer than this many samples per cell from
// one view) take the brick-owned backward; denser ones the tile scatter.
// Measured on MI355X, brick against tile: 64^2 x 128 over 64^3 (1.9 per
// view-cell) 0.021 against 0.045 ms; 16 views of 200^2 x 256 over 256^3 (0.6)
// 1.73 against 2.62 ms; 1024^2 x 512 over 256^3 (31.6) 2.56 against 0.58 ms;
// the 360-view 256 x 384 helix over 128^3 (11.7) 63 against 12.1 ms.
constexpr double kBrickMaxViewReuse = 4.0;

// How the volume backward runs.  Beer-Lambert and the line integral with the
// box clip, from views sparse against the voxels, use the brick-owned
// backward: a ray-record pass (64 bytes per ray of every (view, channel) pair
// and a float per 256 rays, in the workspace) and one workgroup per brick of
// the gradient, which writes its voxels once.  Denser views, the near/far
// mode and compositing scatter tile by tile through LDS windows and global
// atomics.
//
// What the compositing backward's coefficient passes read.  Both passes read
// every sample again, so from one sample per cell a z-pair copy in the
// workspace pays (two loads per sample; zero-padded in the near/far mode; fp32
// and mapped with a transfer function); below that they read the volume (the
// mapped fp32 linear copy with a transfer function).  The other modes read
// nothing.
struct BackwardRead {
    bool brick;            // the brick-owned backward (records at offset 0)
    bool zpair, padded, mapped;
    int read_elem;
    size_t per_volume_bytes, workspace_bytes;
    size_t bound_offset;   // with a copy: the value bounds after the copies (else 0)
};

// The brick-owned backward's workspace: 64-byte ray records, then one float
// per 256 records (their largest cell bound), ...
inline size_t ray_record_bytes(int n_views, int C, int H, int W)
{
    return ((size_t)n_views * (size_t)C * (size_t)H * (size_t)W * 64 + 255) & ~(size_t)255;
}

inline size_t ray_block_max_bytes(int n_views, int C, int H, int W)
{
    const size_t rays = (size_t)n_views * (size_t)C * (size_t)H * (size_t)W;
    return (((rays + 255) / 256) * 4 + 255) & ~(size_t)255;
}

// ... then 48 bytes per view (its fp32 projection).
inline size_t brick_view_bytes(int n_views) { return ((size_t)n_views * 48 + 255) & ~(size_t)255; }

inline BackwardRead plan_backward(int n_volumes, int C, int nz, int ny, int nx, int elem_bytes,
                                  int n_views, int H, int W, int N, int mode, int clip,
                                  bool has_tf)
{
    BackwardRead r{};
    if (mode != kAlpha) {
        const double cells = (double)(nx + 1) * (double)(ny + 1) * (double)(nz + 1);
        const double view_reuse = (double)H * (double)W * (double)N / cells;
        if (clip == kClipBox && view_reuse < kBrickMaxViewReuse) {
            r.brick = true;
            r.workspace_bytes = ray_record_bytes(n_views, C, H, W) +
                                ray_block_max_bytes(n_views, C, H, W) + brick_view_bytes(n_views);
        }
        return r;
    }
    r.mapped = has_tf;
    r.read_elem = has_tf ? 4 : elem_bytes;
    const double n_cells = (double)(nx + 1) * (double)(ny + 1) * (double)(nz + 1);
    const double rays = n_volumes > 0 ? (double)(n_views / n_volumes) * H * W : 0.0;
    const bool reuse = rays * N >= n_cells;
    double bytes = 0.0;
    if (reuse && clip == kClipNearFar) {
        bytes = (double)(nx + 2) * (ny + 2) * (nz + 1) * 2.0 * r.read_elem;
        r.zpair = r.padded = bytes < 4294967040.0;
    } else if (reuse && nx >= 2 && nz >= 2) {
        bytes = (double)nx * ny * (nz - 1) * 2.0 * r.read_elem;
        r.zpair = bytes < 4294967040.0;
    }
    if (!r.zpair) {
        r.padded = false;
        bytes = has_tf ? (double)nx * ny * nz * 4.0 : 0.0;
    }
    r.per_volume_bytes = ((size_t)bytes + 255) & ~(size_t)255;
    r.workspace_bytes = r.per_volume_bytes * (size_t)n_volumes * (size_t)C;
    // with a copy, one (flag, maximum) int pair per channel-volume of the
    // values the coefficient passes read, which bounds every coefficient in
    // closed form (drr_value_bound_kernel)
    if (r.workspace_bytes > 0) {
        r.bound_offset = r.workspace_bytes;
        r.workspace_bytes += ((size_t)8 * n_volumes * C + 255) & ~(size_t)255;
    }
    return r;
}

// With reuse_copy the workspace already holds the plan's read copy of `vol`
// (made by an earlier call with the same volume and plan) and no relayout runs.
hipError_t launch_forward(const LaunchArgs& a, const RenderPlan& plan, const void* vol, int dtype,
                          void* workspace, float* out, float* s_out, hipStream_t stream,
                          bool reuse_copy = false);
// What the plan's march reads, made in `workspace`: the corner cells (zero-padded
// and/or mapped as the call asks) or the mapped fp32 volumes; nothing when the
// march reads the caller's volumes.
hipError_t launch_read_copy(const LaunchArgs& a, const RenderPlan& plan, const void* vol,
                            int dtype, void* workspace, hipStream_t stream);
// The volume backward of a render call.  `vol` is read for alpha compositing
// and for the transfer function's slope; `out_in` (the forward's image) for
// alpha compositing; `s_in` (optical depth) for Beer-Lambert.
hipError_t launch_backward(const LaunchArgs& a, const void* vol, int dtype, const float* grad_out,
                           const float* out_in, const float* s_in, float* grad, void* workspace,
                           hipStream_t stream);
// The brick-owned backward (plan_backward's `brick`): ray records into
// `workspace`, then the bricks of every channel-volume's gradient.
hipError_t launch_brick_backward(const LaunchArgs& a, const float* grad_out, const float* s_in,
                                 float* grad, void* workspace, hipStream_t stream);
// zero n floats with a kernel (graph-capturable, unlike a memset node)
hipError_t launch_fill(float* p, size_t n, hipStream_t stream);

// The rendering frame of a ras2ijk affine: p = Q X + o for a RAS point X
// (Q orthonormal, o in mm), made on the host from ras2ijk and the volume size.
struct VolumeFrame {
    double Q[9];
    double o[3];
};

hipError_t launch_vtk_poses(const float* view_mats, int n_views, const VolumeFrame& F,
                            float* poses, hipStream_t stream);
hipError_t launch_vtk_poses_backward(const float* view_mats, int n_views, const VolumeFrame& F,
                                     const float* grad_poses, float* grad_view,
                                     hipStream_t stream);

// Gaussian-Poisson surrogate on a transmission map (elementwise).
hipError_t launch_poisson(const float* T, const float* z, size_t n, float i0, float* out,
                          hipStream_t stream);
hipError_t launch_poisson_backward(const float* T, const float* z, size_t n, float i0,
                                   const float* g, float* grad, hipStream_t stream);

// Cell-constant (Siddon) pair: no workspace.
hipError_t launch_siddon_forward(const LaunchArgs& a, const void* vol, int dtype, float* out,
                                 float* s_out, hipStream_t stream);
hipError_t launch_siddon_backward(const LaunchArgs& a, const float* grad_out, const float* s_in,
                                  float* grad, hipStream_t stream);
// Its brick-owned form (drr_brick.hip), for views sparse against the voxels:
// writes every voxel of the gradient itself.
hipError_t launch_siddon_brick_backward(const LaunchArgs& a, const float* grad_out,
                                        const float* s_in, float* grad, hipStream_t stream);

// Pose gradient: the march of the forward (same read plan: the caller's, mapped
// or corner-cell volumes in `read_buf`) with gradient accumulators; `acc` holds
// 12 doubles per view.  Beer-Lambert and line integral with the box clip.
inline size_t pose_acc_bytes(int n_views) { return ((size_t)n_views * 12 * 8 + 255) & ~(size_t)255; }

hipError_t launch_backward_pose(const LaunchArgs& a, const RenderPlan& plan, const void* vol,
                                int dtype, void* read_buf, double* acc, const float* grad_out,
                                float* grad_poses, hipStream_t stream, bool reuse_copy = false);

}  // namespace drr
