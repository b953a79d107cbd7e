// drr_internal.hpp -- what the C-ABI layer passes to the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>

#include "drr_device.hpp"

namespace drr {

constexpr int kBeerLambert = 0;
constexpr int kLineIntegral = 1;

// Validated call arguments, already converted to the kernels' form.
struct LaunchArgs {
    VolumeDesc V;
    Intrinsics K;
    const float* poses;   // device, n_views x 12
    int n_views, H, W, N, mode;
};

// How the forward reads the volume.  The corner-cell copy (8 elements per
// trilinear cell, clamp to edge baked in) turns a sample into one (bf16) or two
// (fp32) 16-byte loads, but is 8x the volume and costs a relayout pass, so it
// pays only when samples reuse cells: measured on MI355X, from about 16
// samples per cell for fp32 (a 256^3 volume at 1024^2 x 512 samples: 1.48 ms
// -> 0.89 ms including the relayout; a 16 x 200^2 x 256 batch, ~10 samples per
// cell, got slower) and about 4 for bf16.  It must also fit 32-bit offsets.
struct ForwardPlan {
    bool cells;
    size_t workspace_bytes;
};

inline ForwardPlan plan_forward(int nz, int ny, int nx, int elem_bytes, long long n_rays, int N)
{
    ForwardPlan p{false, 0};
    const double n_cells = (double)(nx + 1) * (double)(ny + 1) * (double)(nz + 1);
    const double cell_bytes = n_cells * 8.0 * elem_bytes;
    const double samples_per_cell = (double)n_rays * (double)N / n_cells;
    const double min_reuse = elem_bytes == 4 ? 16.0 : 4.0;
    if (n_rays > 0 && samples_per_cell >= min_reuse && cell_bytes < 4294967040.0) {
        p.cells = true;
        p.workspace_bytes = ((size_t)cell_bytes + 255) & ~(size_t)255;
    }
    return p;
}

hipError_t launch_forward(const LaunchArgs& a, const void* vol, int dtype, bool cells,
                          void* workspace, float* out, float* s_out, hipStream_t stream);
hipError_t launch_backward(const LaunchArgs& a, const float* grad_out, const float* s_in,
                           float* grad, hipStream_t stream);
// zero n floats with a kernel (graph-capturable, unlike a memset node)
hipError_t launch_fill(float* p, size_t n, hipStream_t stream);

// Cell-constant (Siddon) pair: no workspace.
hipError_t launch_siddon_forward(const LaunchArgs& a, const void* vol, int dtype, float* out,
                                 float* s_out, hipStream_t stream);
hipError_t launch_siddon_backward(const LaunchArgs& a, const float* grad_out, const float* s_in,
                                  float* grad, hipStream_t stream);

// Pose gradient: the march of the forward (same volume plan) with gradient
// accumulators; `acc` holds 12 doubles per view.
inline size_t pose_acc_bytes(int n_views) { return ((size_t)n_views * 12 * 8 + 255) & ~(size_t)255; }

hipError_t launch_backward_pose(const LaunchArgs& a, const void* vol, int dtype, bool cells,
                                void* cell_buf, double* acc, const float* grad_out,
                                float* grad_poses, hipStream_t stream);

}  // namespace drr
