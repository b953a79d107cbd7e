// drr_abi.hip -- the extern "C" boundary of libdrr (declared in include/drr.h):
// host-side validation, conversion of the arguments to the kernels' form and
// launches on the caller's stream.  Nothing here allocates device memory or
// synchronises.
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/drr.h"
#include "drr_internal.hpp"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return status;
}

int ok()
{
    g_last_error[0] = '\0';
    return DRR_OK;
}

constexpr long long kMaxDim = 16384;
// The pose kernels round in-box positions to fixed point with a 1.5 * 2^52
// add, exact only under 2^19 voxels per axis.
static_assert(kMaxDim < 524288, "axis limit must stay under 2^19");
constexpr long long kMaxElems = (1LL << 31) - 1;
constexpr long long kMaxVolumeBytes = (1LL << 32) - 1;  // 32-bit buffer offsets
constexpr int kMaxSamples = 1 << 24;

// Shared validation of the geometry arguments; fills `a` on success.
int check_geometry(int nz, int ny, int nx, int elem_bytes, const float* spacing, const float* K,
                   const float* poses, int n_views, int det_h, int det_w, int n_samples,
                   int mode, drr::LaunchArgs& a, int max_mode = DRR_LINE_INTEGRAL)
{
    if (nz < 1 || ny < 1 || nx < 1)
        return fail(DRR_ERR_INVALID_ARGUMENT, "volume dims must be >= 1 (got %d x %d x %d)", nz,
                    ny, nx);
    if (nz > kMaxDim || ny > kMaxDim || nx > kMaxDim ||
        (long long)nz * ny * nx > kMaxElems ||
        (long long)nz * ny * nx * elem_bytes > kMaxVolumeBytes)
        return fail(DRR_ERR_UNSUPPORTED, "volume %d x %d x %d exceeds the supported size", nz, ny,
                    nx);
    if (n_views < 0 || det_h < 0 || det_w < 0)
        return fail(DRR_ERR_INVALID_ARGUMENT, "n_views, det_h, det_w must be >= 0");
    if ((long long)n_views * det_h * det_w > kMaxElems)
        return fail(DRR_ERR_UNSUPPORTED, "more than 2^31 - 1 rays");
    if (n_samples < 1)
        return fail(DRR_ERR_INVALID_ARGUMENT, "n_samples must be >= 1 (got %d)", n_samples);
    if (n_samples > kMaxSamples)
        return fail(DRR_ERR_UNSUPPORTED, "n_samples above 2^24");
    if (mode < DRR_BEER_LAMBERT || mode > max_mode)
        return fail(DRR_ERR_INVALID_ARGUMENT, "unknown or unsupported mode %d", mode);
    if (!spacing) return fail(DRR_ERR_INVALID_ARGUMENT, "spacing is NULL");
    if (!K) return fail(DRR_ERR_INVALID_ARGUMENT, "K is NULL");
    for (int i = 0; i < 3; ++i)
        if (!(spacing[i] > 0.0f) || !isfinite(spacing[i]))
            return fail(DRR_ERR_INVALID_ARGUMENT, "spacing[%d] must be finite and > 0", i);
    double k[9];
    for (int i = 0; i < 9; ++i) {
        if (!isfinite(K[i])) return fail(DRR_ERR_INVALID_ARGUMENT, "K[%d] is not finite", i);
        k[i] = K[i];
    }
    const double det = k[0] * (k[4] * k[8] - k[5] * k[7]) - k[1] * (k[3] * k[8] - k[5] * k[6]) +
                       k[2] * (k[3] * k[7] - k[4] * k[6]);
    if (det == 0.0) return fail(DRR_ERR_INVALID_ARGUMENT, "K is singular");
    const long long n_rays = (long long)n_views * det_h * det_w;
    if (n_rays > 0 && !poses) return fail(DRR_ERR_INVALID_ARGUMENT, "poses is NULL");

    const int n[3] = {nx, ny, nz};
    for (int i = 0; i < 3; ++i) {
        a.V.n[i] = n[i];
        a.V.s[i] = (double)spacing[i];
        a.V.inv_s[i] = 1.0 / (double)spacing[i];
        a.V.half_e[i] = 0.5 * (double)n[i] * (double)spacing[i];
        a.V.q_off[i] = 0.5 * (double)(n[i] - 1);
    }
    a.V.cell_row_bytes = a.V.cell_slice_bytes = a.V.cell_total_bytes = 0;
    a.V.row_bytes = (uint32_t)nx * (uint32_t)elem_bytes;
    a.V.slice_bytes = (uint32_t)nx * (uint32_t)ny * (uint32_t)elem_bytes;
    a.V.total_bytes = (uint32_t)((long long)nz * ny * nx * elem_bytes);
    for (int i = 0; i < 9; ++i) a.K.k[i] = K[i];
    a.poses = poses;
    a.n_views = n_views;
    a.H = det_h;
    a.W = det_w;
    a.N = n_samples;
    a.mode = mode;
    a.n_volumes = 1;
    a.C = 1;
    a.f = 1.0f;
    a.clip = drr::kClipBox;
    a.margin = 0.0f;
    a.has_tf = false;
    a.tf.knots = 0;
    return DRR_OK;
}

// Byte geometry of what the march reads under `plan`: the linear volume (the
// caller's, or the fp32 mapped copy when a transfer function maps it) or its
// z-pair copy and, with the corner-cell copy, its cells, all of
// plan.read_elem-byte elements.
void set_read_geometry(drr::VolumeDesc& V, const drr::RenderPlan& plan)
{
    const uint32_t nx = (uint32_t)V.n[0], ny = (uint32_t)V.n[1], nz = (uint32_t)V.n[2];
    const uint32_t eb = (uint32_t)plan.read_elem;
    if (plan.zpair && plan.padded) {
        // zero-padded z-pairs: nz + 1 slices of (ny + 2) rows of nx + 2 pairs
        V.row_bytes = (nx + 2) * 2u * eb;
        V.slice_bytes = (ny + 2) * V.row_bytes;
        V.total_bytes = (uint32_t)((unsigned long long)(nz + 1) * V.slice_bytes);
    } else if (plan.zpair) {
        // z-pair copy: nz - 1 slices of (x, y) elements of two values each
        V.row_bytes = nx * 2u * eb;
        V.slice_bytes = nx * ny * 2u * eb;
        V.total_bytes = (uint32_t)((unsigned long long)(nz - 1) * V.slice_bytes);
    } else {
        V.row_bytes = nx * eb;
        V.slice_bytes = nx * ny * eb;
        V.total_bytes = (uint32_t)((unsigned long long)nz * ny * nx * eb);
    }
    if (plan.cells) {
        V.cell_row_bytes = (nx + 1) * 8u * eb;
        V.cell_slice_bytes = (ny + 1) * V.cell_row_bytes;
        V.cell_total_bytes = (uint32_t)((unsigned long long)(nz + 1) * V.cell_slice_bytes);
    }
}

// Validation of the front-end options of drr_render / drr_render_backward_volume;
// fills the batch, factor, clip and transfer fields of `a`.
int check_render(int n_volumes, int n_channels, int n_views, float density_factor, int clip,
                 float margin, const float* tf_xp, const float* tf_yp, int tf_knots,
                 drr::LaunchArgs& a)
{
    if (n_volumes < 1 || n_channels < 1)
        return fail(DRR_ERR_INVALID_ARGUMENT, "n_volumes and n_channels must be >= 1");
    if ((long long)n_volumes * n_channels > 65535)
        return fail(DRR_ERR_UNSUPPORTED, "more than 65535 channel-volumes");
    if (n_views % n_volumes != 0)
        return fail(DRR_ERR_INVALID_ARGUMENT,
                    "n_views (%d) must be a multiple of n_volumes (%d)", n_views, n_volumes);
    if ((long long)n_views * n_channels * a.H * a.W > kMaxElems)
        return fail(DRR_ERR_UNSUPPORTED, "more than 2^31 - 1 outputs");
    if (!isfinite(density_factor))
        return fail(DRR_ERR_INVALID_ARGUMENT, "density_factor must be finite");
    if (clip != DRR_CLIP_BOX && clip != DRR_CLIP_NEAR_FAR)
        return fail(DRR_ERR_INVALID_ARGUMENT, "unknown clip mode %d", clip);
    if (!isfinite(margin)) return fail(DRR_ERR_INVALID_ARGUMENT, "margin must be finite");
    if ((tf_xp == nullptr) != (tf_yp == nullptr))
        return fail(DRR_ERR_INVALID_ARGUMENT, "tf_xp and tf_yp must both be given or both NULL");
    a.n_volumes = n_volumes;
    a.C = n_channels;
    a.f = density_factor;
    a.clip = clip;
    a.margin = margin;
    a.has_tf = tf_xp != nullptr;
    a.tf.knots = 0;
    if (a.has_tf) {
        if (tf_knots < 2)
            return fail(DRR_ERR_INVALID_ARGUMENT, "tf_knots must be >= 2 (got %d)", tf_knots);
        if ((long long)tf_knots * n_channels > drr::kMaxTransferEntries)
            return fail(DRR_ERR_UNSUPPORTED, "n_channels * tf_knots above %d",
                        drr::kMaxTransferEntries);
        a.tf.knots = tf_knots;
        for (int c = 0; c < n_channels; ++c) {
            for (int k = 0; k < tf_knots; ++k) {
                const int i = c * tf_knots + k;
                if (!isfinite(tf_xp[i]) || !isfinite(tf_yp[i]))
                    return fail(DRR_ERR_INVALID_ARGUMENT, "transfer knot %d is not finite", i);
                if (k > 0 && !(tf_xp[i] > tf_xp[i - 1]))
                    return fail(DRR_ERR_INVALID_ARGUMENT,
                                "tf_xp of channel %d must be strictly increasing", c);
                a.tf.xp[i] = tf_xp[i];
                a.tf.yp[i] = tf_yp[i];
            }
            for (int k = 0; k + 1 < tf_knots; ++k) {
                const int i = c * tf_knots + k;
                a.tf.m[i] = (float)(((double)tf_yp[i + 1] - (double)tf_yp[i]) /
                                    ((double)tf_xp[i + 1] - (double)tf_xp[i]));
            }
            a.tf.m[c * tf_knots + tf_knots - 1] = 0.0f;
        }
    }
    return DRR_OK;
}

// The rendering frame of a ras2ijk affine (row-major 4 x 4): voxel sizes from
// the row norms of its linear part, which must be a scaled orthonormal matrix.
int frame_from_ras(const float* ras2ijk, int nz, int ny, int nx, drr::VolumeFrame& F, double s[3])
{
    if (!ras2ijk) return fail(DRR_ERR_INVALID_ARGUMENT, "ras2ijk is NULL");
    for (int i = 0; i < 16; ++i)
        if (!isfinite(ras2ijk[i]))
            return fail(DRR_ERR_INVALID_ARGUMENT, "ras2ijk[%d] is not finite", i);
    if (fabs(ras2ijk[12]) > 1e-6 || fabs(ras2ijk[13]) > 1e-6 || fabs(ras2ijk[14]) > 1e-6 ||
        fabs(ras2ijk[15] - 1.0) > 1e-6)
        return fail(DRR_ERR_INVALID_ARGUMENT, "ras2ijk's last row must be (0, 0, 0, 1)");
    const int n[3] = {nx, ny, nz};
    for (int a = 0; a < 3; ++a) {
        double norm = 0.0;
        for (int k = 0; k < 3; ++k) norm += (double)ras2ijk[a * 4 + k] * ras2ijk[a * 4 + k];
        norm = sqrt(norm);
        if (!(norm > 0.0)) return fail(DRR_ERR_INVALID_ARGUMENT, "ras2ijk row %d is zero", a);
        s[a] = 1.0 / norm;
        for (int k = 0; k < 3; ++k) F.Q[a * 3 + k] = (double)ras2ijk[a * 4 + k] * s[a];
        F.o[a] = s[a] * ((double)ras2ijk[a * 4 + 3] - 0.5 * (double)(n[a] - 1));
    }
    for (int a = 0; a < 3; ++a)
        for (int b = 0; b < 3; ++b) {
            double dot = 0.0;
            for (int k = 0; k < 3; ++k) dot += F.Q[a * 3 + k] * F.Q[b * 3 + k];
            if (fabs(dot - (a == b ? 1.0 : 0.0)) > 1e-4)
                return fail(DRR_ERR_INVALID_ARGUMENT,
                            "ras2ijk's voxel axes must be orthogonal (a scaled rotation)");
        }
    return DRR_OK;
}

// Fixed device scratch of drr_forward_no_alloc: the copy of the volume its read
// plan marches (corner cells or z-pairs) goes here instead of into a caller
// workspace, for callers that cannot allocate device memory.  Every GPU the
// library runs on holds its own copy of the array until the process ends.
// Host code never uses the array's name as a device address: its address on
// each device comes from hipGetSymbolAddress (scratch_on_stream_device).
constexpr size_t kScratchBytes = DRR_NO_ALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch must hold whole 256-byte blocks");
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the device `stream` runs on (the current
// device for the null stream), looked up once per device with that device
// current.
int scratch_on_stream_device(hipStream_t stream, void** ptr)
{
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return fail(DRR_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    int dev = cur;
    if (stream != nullptr) {
        e = hipStreamGetDevice(stream, &dev);
        if (e != hipSuccess)
            return fail(DRR_ERR_HIP, "hipStreamGetDevice failed: %s", hipGetErrorString(e));
    }
    if (dev < 0 || dev >= kMaxDevices)
        return fail(DRR_ERR_UNSUPPORTED, "device %d is beyond the %d the scratch table holds", dev,
                    kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess)
            return fail(DRR_ERR_HIP, "hipSetDevice(%d) failed: %s", dev, hipGetErrorString(e));
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        const hipError_t back = dev != cur ? hipSetDevice(cur) : hipSuccess;
        if (e != hipSuccess)
            return fail(DRR_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d failed: %s", dev,
                        hipGetErrorString(e));
        if (back != hipSuccess)
            return fail(DRR_ERR_HIP, "hipSetDevice(%d) failed: %s", cur, hipGetErrorString(back));
        if (p == nullptr || ((uintptr_t)p & 255u))
            return fail(DRR_ERR_HIP, "scratch on device %d is not 256-byte aligned", dev);
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return DRR_OK;
}

// drr_forward with the workspace the caller passes, or (no_alloc) with the
// fixed scratch of the stream's device.
int forward_into(const void* volume, int dtype, int nz, int ny, int nx, const float* spacing,
                 const float* K, const float* poses, int n_views, int det_h, int det_w,
                 int n_samples, int mode, float* out, float* line_integral, void* workspace,
                 size_t workspace_bytes, bool no_alloc, void* stream, bool reuse_copy = false)
{
    if (dtype != DRR_F32 && dtype != DRR_BF16)
        return fail(DRR_ERR_INVALID_ARGUMENT, "unknown dtype %d", dtype);
    drr::LaunchArgs a;
    int st = check_geometry(nz, ny, nx, dtype == DRR_F32 ? 4 : 2, spacing, K, poses, n_views,
                            det_h, det_w, n_samples, mode, a);
    if (st != DRR_OK) return st;
    if (!volume) return fail(DRR_ERR_INVALID_ARGUMENT, "volume is NULL");
    const long long n_rays = (long long)n_views * det_h * det_w;
    if (n_rays > 0 && !out) return fail(DRR_ERR_INVALID_ARGUMENT, "out is NULL");
    const int eb = dtype == DRR_F32 ? 4 : 2;
    const drr::RenderPlan plan = drr::plan_render(1, 1, nz, ny, nx, eb, n_views, det_h, det_w,
                                                  n_samples, drr::kClipBox, false, true);
    if (no_alloc) {
        if (plan.workspace_bytes > kScratchBytes)
            return fail(DRR_ERR_UNSUPPORTED,
                        "this call needs %zu bytes of scratch; the fixed scratch holds %zu",
                        plan.workspace_bytes, kScratchBytes);
        if (n_rays == 0) return ok();
        if (plan.workspace_bytes > 0) {
            st = scratch_on_stream_device(static_cast<hipStream_t>(stream), &workspace);
            if (st != DRR_OK) return st;
        }
    } else {
        if (workspace_bytes < plan.workspace_bytes)
            return fail(DRR_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes, %zu needed",
                        workspace_bytes, plan.workspace_bytes);
        if (plan.workspace_bytes > 0 && (!workspace || ((uintptr_t)workspace & 255u)))
            return fail(DRR_ERR_INVALID_ARGUMENT,
                        "workspace must be non-NULL and 256-byte aligned");
        if (n_rays == 0) return ok();
    }
    set_read_geometry(a.V, plan);
    hipError_t e = drr::launch_forward(a, plan, volume, dtype, workspace, out, line_integral,
                                       static_cast<hipStream_t>(stream), reuse_copy);
    if (e != hipSuccess)
        return fail(DRR_ERR_HIP, "forward launch failed: %s", hipGetErrorString(e));
    return ok();
}

// drr_render's body; with reuse_copy the workspace already holds the read copy.
int render_into(const void* volume, int dtype, int n_volumes, int n_channels, int nz, int ny,
                int nx, const float* spacing, const float* K, const float* poses, int n_views,
                int det_h, int det_w, int n_samples, int mode, float density_factor, int clip,
                float margin, const float* tf_xp, const float* tf_yp, int tf_knots, float* out,
                float* aux, void* workspace, size_t workspace_bytes, void* stream,
                bool reuse_copy)
{
    if (dtype != DRR_F32 && dtype != DRR_BF16)
        return fail(DRR_ERR_INVALID_ARGUMENT, "unknown dtype %d", dtype);
    const int eb = dtype == DRR_F32 ? 4 : 2;
    drr::LaunchArgs a;
    int st = check_geometry(nz, ny, nx, eb, spacing, K, poses, n_views, det_h, det_w, n_samples,
                            mode, a, DRR_ALPHA_COMPOSITE);
    if (st != DRR_OK) return st;
    st = check_render(n_volumes, n_channels, n_views, density_factor, clip, margin, tf_xp, tf_yp,
                      tf_knots, a);
    if (st != DRR_OK) return st;
    if (!volume) return fail(DRR_ERR_INVALID_ARGUMENT, "volume is NULL");
    const long long n_out = (long long)n_views * n_channels * det_h * det_w;
    if (n_out > 0 && !out) return fail(DRR_ERR_INVALID_ARGUMENT, "out is NULL");
    const drr::RenderPlan plan = drr::plan_render(n_volumes, n_channels, nz, ny, nx, eb, n_views,
                                                  det_h, det_w, n_samples, clip, a.has_tf, true);
    if (!plan.fits)
        return fail(DRR_ERR_UNSUPPORTED, "one channel-volume of the march's copy exceeds 4 GiB");
    if (workspace_bytes < plan.workspace_bytes)
        return fail(DRR_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes, %zu needed",
                    workspace_bytes, plan.workspace_bytes);
    if (plan.workspace_bytes > 0 && (!workspace || ((uintptr_t)workspace & 255u)))
        return fail(DRR_ERR_INVALID_ARGUMENT, "workspace must be non-NULL and 256-byte aligned");
    if (n_out == 0) return ok();
    set_read_geometry(a.V, plan);
    hipError_t e = drr::launch_forward(a, plan, volume, dtype, workspace, out, aux,
                                       static_cast<hipStream_t>(stream), reuse_copy);
    if (e != hipSuccess)
        return fail(DRR_ERR_HIP, "render launch failed: %s", hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

int drr_poisson_surrogate(const float* transmission, const float* noise, long long n, float i0,
                          float* out, void* stream)
{
    if (n < 0) return fail(DRR_ERR_INVALID_ARGUMENT, "n must be >= 0");
    if (!(i0 > 0.0f) || !isfinite(i0))
        return fail(DRR_ERR_INVALID_ARGUMENT, "i0 must be finite and > 0");
    if (n > 0 && (!transmission || !noise || !out))
        return fail(DRR_ERR_INVALID_ARGUMENT, "transmission, noise and out must be non-NULL");
    hipError_t e = drr::launch_poisson(transmission, noise, (size_t)n, i0, out,
                                       static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(DRR_ERR_HIP, "noise launch failed: %s", hipGetErrorString(e));
    return ok();
}

int drr_poisson_surrogate_backward(const float* transmission, const float* noise, long long n,
                                   float i0, const float* grad_out, float* grad_transmission,
                                   void* stream)
{
    if (n < 0) return fail(DRR_ERR_INVALID_ARGUMENT, "n must be >= 0");
    if (!(i0 > 0.0f) || !isfinite(i0))
        return fail(DRR_ERR_INVALID_ARGUMENT, "i0 must be finite and > 0");
    if (n > 0 && (!transmission || !noise || !grad_out || !grad_transmission))
        return fail(DRR_ERR_INVALID_ARGUMENT,
                    "transmission, noise, grad_out and grad_transmission must be non-NULL");
    hipError_t e = drr::launch_poisson_backward(transmission, noise, (size_t)n, i0, grad_out,
                                                grad_transmission,
                                                static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(DRR_ERR_HIP, "noise backward launch failed: %s", hipGetErrorString(e));
    return ok();
}

int drr_intrinsics_from_fov(float fov_deg, int det_h, int det_w, float* K)
{
    if (!K) return fail(DRR_ERR_INVALID_ARGUMENT, "K is NULL");
    if (!(fov_deg > 0.0f && fov_deg < 180.0f))
        return fail(DRR_ERR_INVALID_ARGUMENT, "fov_deg must lie in (0, 180)");
    if (det_h < 1 || det_w < 1)
        return fail(DRR_ERR_INVALID_ARGUMENT, "det_h and det_w must be >= 1");
    const double f = 0.5 * (double)det_h / tan(0.5 * (double)fov_deg * 3.14159265358979323846 / 180.0);
    const float k[9] = {(float)f, 0.0f, 0.5f * (float)det_w, 0.0f, (float)f, 0.5f * (float)det_h,
                        0.0f, 0.0f, 1.0f};
    for (int i = 0; i < 9; ++i) K[i] = k[i];
    return ok();
}

int drr_poses_from_view_matrices(const float* view_mats, int n_views, const float* ras2ijk,
                                 int nz, int ny, int nx, float* poses, float* spacing,
                                 void* stream)
{
    if (n_views < 0) return fail(DRR_ERR_INVALID_ARGUMENT, "n_views must be >= 0");
    if (nz < 1 || ny < 1 || nx < 1)
        return fail(DRR_ERR_INVALID_ARGUMENT, "volume dims must be >= 1");
    if (n_views > 0 && (!view_mats || !poses))
        return fail(DRR_ERR_INVALID_ARGUMENT, "view_mats and poses must be non-NULL");
    drr::VolumeFrame F;
    double s[3];
    int st = frame_from_ras(ras2ijk, nz, ny, nx, F, s);
    if (st != DRR_OK) return st;
    if (spacing)
        for (int a = 0; a < 3; ++a) spacing[a] = (float)s[a];
    hipError_t e = drr::launch_vtk_poses(view_mats, n_views, F, poses,
                                         static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(DRR_ERR_HIP, "pose conversion launch failed: %s", hipGetErrorString(e));
    return ok();
}

int drr_view_matrices_backward(const float* view_mats, int n_views, const float* ras2ijk, int nz,
                               int ny, int nx, const float* grad_poses, float* grad_view_mats,
                               void* stream)
{
    if (n_views < 0) return fail(DRR_ERR_INVALID_ARGUMENT, "n_views must be >= 0");
    if (nz < 1 || ny < 1 || nx < 1)
        return fail(DRR_ERR_INVALID_ARGUMENT, "volume dims must be >= 1");
    if (n_views > 0 && (!view_mats || !grad_poses || !grad_view_mats))
        return fail(DRR_ERR_INVALID_ARGUMENT,
                    "view_mats, grad_poses and grad_view_mats must be non-NULL");
    drr::VolumeFrame F;
    double s[3];
    int st = frame_from_ras(ras2ijk, nz, ny, nx, F, s);
    if (st != DRR_OK) return st;
    hipError_t e = drr::launch_vtk_poses_backward(view_mats, n_views, F, grad_poses,
                                                  grad_view_mats,
                                                  static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(DRR_ERR_HIP, "pose conversion backward launch failed: %s",
                    hipGetErrorString(e));
    return ok();
}

int drr_abi_version(void) { return DRR_ABI_VERSION; }

const char* drr_last_error(void) { return g_last_error; }

const char* drr_status_string(int status)
{
    switch (status) {
    case DRR_OK: return "ok";
    case DRR_ERR_INVALID_ARGUMENT: return "invalid argument";
    case DRR_ERR_UNSUPPORTED: return "unsupported size or option";
    case DRR_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case DRR_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
    }
}

size_t drr_workspace_bytes(int nz, int ny, int nx, int dtype, int n_views, int det_h,
                           int det_w, int n_samples, int for_backward)
{
    if (nz < 1 || ny < 1 || nx < 1 || n_views < 0 || det_h < 0 || det_w < 0 ||
        n_samples < 1 || (dtype != DRR_F32 && dtype != DRR_BF16))
        return 0;
    if (for_backward == DRR_WORKSPACE_VOLUME_BACKWARD)
        return drr::plan_backward(1, 1, nz, ny, nx, dtype == DRR_F32 ? 4 : 2, n_views, det_h,
                                  det_w, n_samples, DRR_BEER_LAMBERT, drr::kClipBox, false)
            .workspace_bytes;
    const bool fwd = for_backward == DRR_WORKSPACE_FORWARD;
    const size_t plan = drr::plan_render(1, 1, nz, ny, nx, dtype == DRR_F32 ? 4 : 2, n_views,
                                         det_h, det_w, n_samples, drr::kClipBox, false, true)
                            .workspace_bytes;
    if (for_backward == DRR_WORKSPACE_POSE_BACKWARD) return drr::pose_acc_bytes(n_views) + plan;
    return fwd ? plan : 0;
}

int drr_forward(const void* volume, int dtype, int nz, int ny, int nx, const float* spacing,
                const float* K, const float* poses, int n_views, int det_h, int det_w,
                int n_samples, int mode, float* out, float* line_integral, void* workspace,
                size_t workspace_bytes, void* stream)
{
    return forward_into(volume, dtype, nz, ny, nx, spacing, K, poses, n_views, det_h, det_w,
                        n_samples, mode, out, line_integral, workspace, workspace_bytes, false,
                        stream);
}

int drr_forward_reuse(const void* volume, int dtype, int nz, int ny, int nx, const float* spacing,
                      const float* K, const float* poses, int n_views, int det_h, int det_w,
                      int n_samples, int mode, float* out, float* line_integral, void* workspace,
                      size_t workspace_bytes, void* stream)
{
    return forward_into(volume, dtype, nz, ny, nx, spacing, K, poses, n_views, det_h, det_w,
                        n_samples, mode, out, line_integral, workspace, workspace_bytes, false,
                        stream, true);
}

int drr_forward_no_alloc(const void* volume, int dtype, int nz, int ny, int nx,
                         const float* spacing, const float* K, const float* poses, int n_views,
                         int det_h, int det_w, int n_samples, int mode, float* out,
                         float* line_integral, void* stream)
{
    return forward_into(volume, dtype, nz, ny, nx, spacing, K, poses, n_views, det_h, det_w,
                        n_samples, mode, out, line_integral, nullptr, 0, true, stream);
}

int drr_backward_volume(int nz, int ny, int nx, const float* spacing, const float* K,
                        const float* poses, int n_views, int det_h, int det_w, int n_samples,
                        int mode, const float* grad_out, const float* line_integral,
                        float* grad_volume, void* workspace, size_t workspace_bytes,
                        void* stream)
{
    drr::LaunchArgs a;
    int st = check_geometry(nz, ny, nx, 4, spacing, K, poses, n_views, det_h, det_w, n_samples,
                            mode, a);
    if (st != DRR_OK) return st;
    if (!grad_volume) return fail(DRR_ERR_INVALID_ARGUMENT, "grad_volume is NULL");
    const long long n_rays = (long long)n_views * det_h * det_w;
    if (n_rays > 0 && !grad_out) return fail(DRR_ERR_INVALID_ARGUMENT, "grad_out is NULL");
    if (n_rays > 0 && mode == DRR_BEER_LAMBERT && !line_integral)
        return fail(DRR_ERR_INVALID_ARGUMENT,
                    "line_integral is required for the Beer-Lambert backward");
    const size_t need =
        drr_workspace_bytes(nz, ny, nx, DRR_F32, n_views, det_h, det_w, n_samples, 1);
    if (workspace_bytes < need)
        return fail(DRR_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes, %zu needed",
                    workspace_bytes, need);
    if (need > 0 && (!workspace || ((uintptr_t)workspace & 255u)))
        return fail(DRR_ERR_INVALID_ARGUMENT, "workspace must be non-NULL and 256-byte aligned");
    hipError_t e = drr::launch_backward(a, nullptr, DRR_F32, grad_out, nullptr, line_integral,
                                        grad_volume, workspace, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(DRR_ERR_HIP, "backward launch failed: %s", hipGetErrorString(e));
    return ok();
}

size_t drr_render_workspace_bytes(int n_volumes, int n_channels, int nz, int ny, int nx,
                                  int dtype, int n_views, int det_h, int det_w, int n_samples,
                                  int mode, int clip, int tf_knots, int for_backward)
{
    if (n_volumes < 1 || n_channels < 1 || nz < 1 || ny < 1 || nx < 1 || n_views < 0 ||
        det_h < 0 || det_w < 0 || n_samples < 1 || (dtype != DRR_F32 && dtype != DRR_BF16) ||
        n_views % n_volumes != 0 || (clip != DRR_CLIP_BOX && clip != DRR_CLIP_NEAR_FAR))
        return 0;
    const bool has_tf = tf_knots > 0;
    if (for_backward == DRR_WORKSPACE_VOLUME_BACKWARD)
        return drr::plan_backward(n_volumes, n_channels, nz, ny, nx, dtype == DRR_F32 ? 4 : 2,
                                  n_views, det_h, det_w, n_samples, mode, clip, has_tf)
            .workspace_bytes;
    const bool fwd = for_backward == DRR_WORKSPACE_FORWARD;
    const size_t plan = drr::plan_render(n_volumes, n_channels, nz, ny, nx,
                                         dtype == DRR_F32 ? 4 : 2, n_views, det_h, det_w,
                                         n_samples, clip, has_tf, true)
                            .workspace_bytes;
    if (for_backward == DRR_WORKSPACE_POSE_BACKWARD) return drr::pose_acc_bytes(n_views) + plan;
    return fwd ? plan : 0;
}

int drr_render(const void* volume, int dtype, int n_volumes, int n_channels, int nz, int ny,
               int nx, const float* spacing, const float* K, const float* poses, int n_views,
               int det_h, int det_w, int n_samples, int mode, float density_factor, int clip,
               float margin, const float* tf_xp, const float* tf_yp, int tf_knots, float* out,
               float* aux, void* workspace, size_t workspace_bytes, void* stream)
{
    return render_into(volume, dtype, n_volumes, n_channels, nz, ny, nx, spacing, K, poses,
                       n_views, det_h, det_w, n_samples, mode, density_factor, clip, margin, tf_xp,
                       tf_yp, tf_knots, out, aux, workspace, workspace_bytes, stream, false);
}

int drr_render_reuse(const void* volume, int dtype, int n_volumes, int n_channels, int nz, int ny,
                     int nx, const float* spacing, const float* K, const float* poses,
                     int n_views, int det_h, int det_w, int n_samples, int mode,
                     float density_factor, int clip, float margin, const float* tf_xp,
                     const float* tf_yp, int tf_knots, float* out, float* aux, void* workspace,
                     size_t workspace_bytes, void* stream)
{
    return render_into(volume, dtype, n_volumes, n_channels, nz, ny, nx, spacing, K, poses,
                       n_views, det_h, det_w, n_samples, mode, density_factor, clip, margin, tf_xp,
                       tf_yp, tf_knots, out, aux, workspace, workspace_bytes, stream, true);
}

int drr_render_backward_volume(const void* volume, int dtype, int n_volumes, int n_channels,
                               int nz, int ny, int nx, const float* spacing, const float* K,
                               const float* poses, int n_views, int det_h, int det_w,
                               int n_samples, int mode, float density_factor, int clip,
                               float margin, const float* tf_xp, const float* tf_yp,
                               int tf_knots, const float* grad_out, const float* out,
                               const float* aux, float* grad_volume, void* workspace,
                               size_t workspace_bytes, void* stream)
{
    if (dtype != DRR_F32 && dtype != DRR_BF16)
        return fail(DRR_ERR_INVALID_ARGUMENT, "unknown dtype %d", dtype);
    drr::LaunchArgs a;
    int st = check_geometry(nz, ny, nx, 4, spacing, K, poses, n_views, det_h, det_w, n_samples,
                            mode, a, DRR_ALPHA_COMPOSITE);
    if (st != DRR_OK) return st;
    st = check_render(n_volumes, n_channels, n_views, density_factor, clip, margin, tf_xp, tf_yp,
                      tf_knots, a);
    if (st != DRR_OK) return st;
    if (!grad_volume) return fail(DRR_ERR_INVALID_ARGUMENT, "grad_volume is NULL");
    const long long n_out = (long long)n_views * n_channels * det_h * det_w;
    if (n_out > 0 && !grad_out) return fail(DRR_ERR_INVALID_ARGUMENT, "grad_out is NULL");
    if (n_out > 0 && mode == DRR_BEER_LAMBERT && !aux)
        return fail(DRR_ERR_INVALID_ARGUMENT, "aux (optical depth) is required for Beer-Lambert");
    if (n_out > 0 && mode == DRR_ALPHA_COMPOSITE && !out)
        return fail(DRR_ERR_INVALID_ARGUMENT, "out (the forward image) is required for alpha "
                                              "compositing");
    if ((mode == DRR_ALPHA_COMPOSITE || a.has_tf) && !volume)
        return fail(DRR_ERR_INVALID_ARGUMENT,
                    "volume is required for alpha compositing and for a transfer function");
    const size_t need =
        drr::plan_backward(n_volumes, n_channels, nz, ny, nx, dtype == DRR_F32 ? 4 : 2, n_views,
                           det_h, det_w, n_samples, mode, clip, a.has_tf)
            .workspace_bytes;
    if (workspace_bytes < need)
        return fail(DRR_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes, %zu needed",
                    workspace_bytes, need);
    if (need > 0 && (!workspace || ((uintptr_t)workspace & 255u)))
        return fail(DRR_ERR_INVALID_ARGUMENT, "workspace must be non-NULL and 256-byte aligned");
    hipError_t e = drr::launch_backward(a, volume, dtype, grad_out, out, aux, grad_volume,
                                        workspace, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(DRR_ERR_HIP, "render backward launch failed: %s", hipGetErrorString(e));
    return ok();
}

}  // extern "C"

namespace {

// The pose backward of a validated render call `a` (single-volume calls come
// here too): every mode, either clip.
int pose_backward(drr::LaunchArgs& a, const void* volume, int dtype, const float* grad_out,
                  float* grad_poses, void* workspace, size_t workspace_bytes, void* stream,
                  bool reuse_copy = false)
{
    if (!volume) return fail(DRR_ERR_INVALID_ARGUMENT, "volume is NULL");
    const long long n_out = (long long)a.n_views * a.C * a.H * a.W;
    if (n_out > 0 && !grad_out) return fail(DRR_ERR_INVALID_ARGUMENT, "grad_out is NULL");
    if (a.n_views > 0 && !grad_poses) return fail(DRR_ERR_INVALID_ARGUMENT, "grad_poses is NULL");
    const int eb = dtype == DRR_F32 ? 4 : 2;
    const drr::RenderPlan plan =
        drr::plan_render(a.n_volumes, a.C, a.V.n[2], a.V.n[1], a.V.n[0], eb, a.n_views, a.H, a.W,
                         a.N, a.clip, a.has_tf, true);
    if (!plan.fits)
        return fail(DRR_ERR_UNSUPPORTED, "one channel-volume of the march's copy exceeds 4 GiB");
    const size_t acc_bytes = drr::pose_acc_bytes(a.n_views);
    const size_t need = acc_bytes + plan.workspace_bytes;
    if (a.n_views == 0) return ok();
    if (workspace_bytes < need)
        return fail(DRR_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes, %zu needed",
                    workspace_bytes, need);
    if (!workspace || ((uintptr_t)workspace & 255u))
        return fail(DRR_ERR_INVALID_ARGUMENT, "workspace must be non-NULL and 256-byte aligned");
    set_read_geometry(a.V, plan);
    char* ws = static_cast<char*>(workspace);
    hipError_t e = drr::launch_backward_pose(a, plan, volume, dtype, ws + acc_bytes,
                                             reinterpret_cast<double*>(ws), grad_out, grad_poses,
                                             static_cast<hipStream_t>(stream), reuse_copy);
    if (e != hipSuccess)
        return fail(DRR_ERR_HIP, "pose backward launch failed: %s", hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

int drr_backward_pose(const void* volume, int dtype, int nz, int ny, int nx, const float* spacing,
                      const float* K, const float* poses, int n_views, int det_h, int det_w,
                      int n_samples, int mode, const float* grad_out, float* grad_poses,
                      void* workspace, size_t workspace_bytes, void* stream)
{
    if (dtype != DRR_F32 && dtype != DRR_BF16)
        return fail(DRR_ERR_INVALID_ARGUMENT, "unknown dtype %d", dtype);
    drr::LaunchArgs a;
    int st = check_geometry(nz, ny, nx, dtype == DRR_F32 ? 4 : 2, spacing, K, poses, n_views,
                            det_h, det_w, n_samples, mode, a);
    if (st != DRR_OK) return st;
    return pose_backward(a, volume, dtype, grad_out, grad_poses, workspace, workspace_bytes,
                         stream);
}

int drr_backward_pose_reuse(const void* volume, int dtype, int nz, int ny, int nx,
                            const float* spacing, const float* K, const float* poses, int n_views,
                            int det_h, int det_w, int n_samples, int mode, const float* grad_out,
                            float* grad_poses, void* workspace, size_t workspace_bytes,
                            void* stream)
{
    if (dtype != DRR_F32 && dtype != DRR_BF16)
        return fail(DRR_ERR_INVALID_ARGUMENT, "unknown dtype %d", dtype);
    drr::LaunchArgs a;
    int st = check_geometry(nz, ny, nx, dtype == DRR_F32 ? 4 : 2, spacing, K, poses, n_views,
                            det_h, det_w, n_samples, mode, a);
    if (st != DRR_OK) return st;
    return pose_backward(a, volume, dtype, grad_out, grad_poses, workspace, workspace_bytes,
                         stream, true);
}

int drr_render_backward_pose(const void* volume, int dtype, int n_volumes, int n_channels,
                             int nz, int ny, int nx, const float* spacing, const float* K,
                             const float* poses, int n_views, int det_h, int det_w,
                             int n_samples, int mode, float density_factor, int clip,
                             float margin, const float* tf_xp, const float* tf_yp, int tf_knots,
                             const float* grad_out, float* grad_poses, void* workspace,
                             size_t workspace_bytes, void* stream)
{
    if (dtype != DRR_F32 && dtype != DRR_BF16)
        return fail(DRR_ERR_INVALID_ARGUMENT, "unknown dtype %d", dtype);
    drr::LaunchArgs a;
    int st = check_geometry(nz, ny, nx, dtype == DRR_F32 ? 4 : 2, spacing, K, poses, n_views,
                            det_h, det_w, n_samples, mode, a, DRR_ALPHA_COMPOSITE);
    if (st != DRR_OK) return st;
    st = check_render(n_volumes, n_channels, n_views, density_factor, clip, margin, tf_xp, tf_yp,
                      tf_knots, a);
    if (st != DRR_OK) return st;
    return pose_backward(a, volume, dtype, grad_out, grad_poses, workspace, workspace_bytes,
                         stream);
}

int drr_render_backward_pose_reuse(const void* volume, int dtype, int n_volumes,
                                   int n_channels, int nz, int ny, int nx, const float* spacing,
                                   const float* K, const float* poses, int n_views, int det_h,
                                   int det_w, int n_samples, int mode, float density_factor,
                                   int clip, float margin, const float* tf_xp,
                                   const float* tf_yp, int tf_knots, const float* grad_out,
                                   float* grad_poses, void* workspace, size_t workspace_bytes,
                                   void* stream)
{
    if (dtype != DRR_F32 && dtype != DRR_BF16)
        return fail(DRR_ERR_INVALID_ARGUMENT, "unknown dtype %d", dtype);
    drr::LaunchArgs a;
    int st = check_geometry(nz, ny, nx, dtype == DRR_F32 ? 4 : 2, spacing, K, poses, n_views,
                            det_h, det_w, n_samples, mode, a, DRR_ALPHA_COMPOSITE);
    if (st != DRR_OK) return st;
    st = check_render(n_volumes, n_channels, n_views, density_factor, clip, margin, tf_xp, tf_yp,
                      tf_knots, a);
    if (st != DRR_OK) return st;
    return pose_backward(a, volume, dtype, grad_out, grad_poses, workspace, workspace_bytes,
                         stream, true);
}

int drr_forward_siddon(const void* volume, int dtype, int nz, int ny, int nx,
                       const float* spacing, const float* K, const float* poses, int n_views,
                       int det_h, int det_w, int mode, float* out, float* line_integral,
                       void* stream)
{
    if (dtype != DRR_F32 && dtype != DRR_BF16)
        return fail(DRR_ERR_INVALID_ARGUMENT, "unknown dtype %d", dtype);
    drr::LaunchArgs a;
    int st = check_geometry(nz, ny, nx, dtype == DRR_F32 ? 4 : 2, spacing, K, poses, n_views,
                            det_h, det_w, 1, mode, a);
    if (st != DRR_OK) return st;
    if (!volume) return fail(DRR_ERR_INVALID_ARGUMENT, "volume is NULL");
    const long long n_rays = (long long)n_views * det_h * det_w;
    if (n_rays > 0 && !out) return fail(DRR_ERR_INVALID_ARGUMENT, "out is NULL");
    if (n_rays == 0) return ok();
    hipError_t e = drr::launch_siddon_forward(a, volume, dtype, out, line_integral,
                                              static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(DRR_ERR_HIP, "Siddon forward launch failed: %s", hipGetErrorString(e));
    return ok();
}

int drr_backward_volume_siddon(int nz, int ny, int nx, const float* spacing, const float* K,
                               const float* poses, int n_views, int det_h, int det_w, int mode,
                               const float* grad_out, const float* line_integral,
                               float* grad_volume, void* stream)
{
    drr::LaunchArgs a;
    int st = check_geometry(nz, ny, nx, 4, spacing, K, poses, n_views, det_h, det_w, 1, mode, a);
    if (st != DRR_OK) return st;
    if (!grad_volume) return fail(DRR_ERR_INVALID_ARGUMENT, "grad_volume is NULL");
    const long long n_rays = (long long)n_views * det_h * det_w;
    if (n_rays > 0 && !grad_out) return fail(DRR_ERR_INVALID_ARGUMENT, "grad_out is NULL");
    if (n_rays > 0 && mode == DRR_BEER_LAMBERT && !line_integral)
        return fail(DRR_ERR_INVALID_ARGUMENT,
                    "line_integral is required for the Beer-Lambert backward");
    hipError_t e = drr::launch_siddon_backward(a, grad_out, line_integral, grad_volume,
                                               static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(DRR_ERR_HIP, "Siddon backward launch failed: %s", hipGetErrorString(e));
    return ok();
}

}  // extern "C"
