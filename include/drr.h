/*
 * drr.h -- C ABI of libdrr: differentiable cone-beam DRR ray casting on
 * AMD Instinct MI355X (gfx950).
 *
 * What is computed (source pages):
 *   - nanodrr project page, introduction: rays come from a Hartley-Zisserman
 *     pinhole camera, intrinsics K and a world-to-camera pose [R | t].
 *   - flashdrr.rendering API, VolumeRaycaster.__init__ and set_fov: ray_samples
 *     samples per ray along normalised per-pixel directions; with
 *     use_beer_lambert the image is 1 - exp(-integral of mu dz).
 *   - flashdrr.rendering API, VolumeRaycaster class text: samples are
 *     trilinear gathers of the volume; rendering is differentiable with
 *     respect to the volume.
 *   - diffct 2.1.0, Quickstart: project() returns raw line integrals and
 *     backproject() applies the matched adjoint A^T.
 *   - torchtomo, "Fast CUDA Kernels": kernels are launched on the caller's
 *     current stream.
 *
 * Conventions (readings where the pages are silent):
 *   - units: mm for geometry, 1/mm for mu; ray directions are unit vectors;
 *   - the volume vol[k][j][i] (x fastest, shape nz x ny x nx) fills the box
 *     [-E/2, E/2], E = (nx sx, ny sy, nz sz), centred at the world origin;
 *   - pixel (r, c) of a det_h x det_w detector is the image point
 *     (c + 1/2, r + 1/2, 1); its world ray is C + t d with
 *     d = normalize(R^T K^-1 (c + 1/2, r + 1/2, 1)) and C = -R^T t;
 *   - each ray is clipped to the box: t0 = max(t_entry, 0), t1 = t_exit; a ray
 *     with t1 <= t0 misses and produces exactly 0 and no gradient;
 *   - n_samples midpoint samples t_k = t0 + (k + 1/2) dz, dz = (t1 - t0) / N,
 *     each a trilinear interpolation with corner indices clamped to the
 *     volume (clamp to edge);
 *   - s = dz * sum_k mu(t_k); Beer-Lambert output 1 - exp(-s) (computed as
 *     -expm1(-s)), line-integral output s.
 *
 * Ownership and errors:
 *   - every buffer is owned by the caller; the library never allocates,
 *     frees or synchronises device memory, and keeps no state between calls
 *     (except drr_forward_no_alloc's fixed scratch array, see there);
 *   - calls are asynchronous: work is enqueued on `stream` (a hipStream_t;
 *     NULL = the default stream) and the call returns without waiting;
 *   - arguments are validated on the host before anything is enqueued; an
 *     invalid call returns a non-zero drr_status and enqueues nothing;
 *   - a failed kernel launch returns DRR_ERR_HIP; faults inside a kernel
 *     surface at the caller's next synchronisation;
 *   - drr_last_error() gives a thread-local description of the last failure;
 *   - no C++ exception crosses this interface; calls are reentrant.
 */
#ifndef DRR_H
#define DRR_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DRR_ABI_VERSION 1

/* Volume element types.  bf16 volumes are read as bf16 and widened exactly
 * to fp32; every sum is accumulated in fp32. */
typedef enum { DRR_F32 = 0, DRR_BF16 = 1 } drr_dtype;

/* Output modes: Beer-Lambert image 1 - exp(-s) (flashdrr use_beer_lambert),
 * the raw line integral s (diffct project), or -- drr_render only --
 * front-to-back alpha compositing (flashdrr use_beer_lambert = False, the
 * "over" operator; see drr_render). */
typedef enum { DRR_BEER_LAMBERT = 0, DRR_LINE_INTEGRAL = 1, DRR_ALPHA_COMPOSITE = 2 } drr_mode;

/* Sample range of a ray (drr_render only): the per-ray box clip of every other
 * call, or flashdrr's per-view near/far range (see drr_render). */
typedef enum { DRR_CLIP_BOX = 0, DRR_CLIP_NEAR_FAR = 1 } drr_clip;

typedef enum {
    DRR_OK = 0,
    DRR_ERR_INVALID_ARGUMENT = 1,     /* null pointer, bad size, bad enum ... */
    DRR_ERR_UNSUPPORTED = 2,          /* valid but beyond the documented limits */
    DRR_ERR_WORKSPACE_TOO_SMALL = 3,  /* workspace_bytes < drr_workspace_bytes(...) */
    DRR_ERR_HIP = 4                   /* a HIP runtime call or launch failed */
} drr_status;

/* Limits: 1 <= nx, ny, nz <= 16384 with nx*ny*nz < 2^31 voxels and the
 * volume (and, for the backward, the fp32 gradient) smaller than 4 GiB;
 * 0 <= n_views, det_h, det_w and n_views*det_h*det_w < 2^31 rays;
 * 1 <= n_samples <= 2^24. */

/* Which call a workspace query is for. */
#define DRR_WORKSPACE_FORWARD 0
#define DRR_WORKSPACE_VOLUME_BACKWARD 1
#define DRR_WORKSPACE_POSE_BACKWARD 2

/* Bytes of device workspace drr_forward (for_backward = 0), drr_backward_volume
 * (1) or drr_backward_pose (2) needs for these sizes; 0 means no workspace is
 * needed (a NULL workspace is then accepted).  Returns 0 as well for invalid
 * sizes (the call itself then reports the error).  The forward and the pose
 * backward use the workspace for a copy of the volume the march reads when
 * rays reuse cells enough for it to pay: corner cells (8 clamped trilinear
 * corners per cell) or z-pairs (each voxel next to its z neighbour); dense
 * views stage boxes of the volume in LDS and need none.  The pose backward
 * also keeps 12 fp64 sums per view there. */
size_t drr_workspace_bytes(int nz, int ny, int nx, int dtype, int n_views, int det_h,
                           int det_w, int n_samples, int for_backward);

/* Forward DRR (flashdrr VolumeRaycaster.forward / diffct project).
 *   volume        device, nz*ny*nx elements of `dtype`, C-contiguous, x fastest
 *   spacing       host, 3 floats: sx, sy, sz (mm), each > 0
 *   K             host, 9 floats, row-major 3x3 intrinsics (invertible)
 *   poses         device, n_views x 12 floats: row-major 3x4 world-to-camera [R | t]
 *   det_h, det_w  detector rows and columns
 *   n_samples     samples per ray (N)
 *   mode          DRR_BEER_LAMBERT or DRR_LINE_INTEGRAL
 *   out           device, n_views*det_h*det_w floats, [view][row][col]
 *   line_integral device or NULL: receives s in the same layout (the
 *                 Beer-Lambert backward needs it)
 *   workspace     device, workspace_bytes >= drr_workspace_bytes(..., 0), 256-byte aligned
 * n_views, det_h or det_w equal to 0 is a valid empty call. */
int drr_forward(const void *volume, int dtype, int nz, int ny, int nx, const float *spacing,
                const float *K, const float *poses, int n_views, int det_h, int det_w,
                int n_samples, int mode, float *out, float *line_integral, void *workspace,
                size_t workspace_bytes, void *stream);

/* drr_forward without the relayout, for renders of one volume from changing
 * poses (the 2D/3D registration and pose estimation that the flashdrr
 * overview names as its workloads).  `workspace` must already hold the read
 * copy that an earlier drr_forward call wrote into it (the volume's
 * corner-cell or z-pair copy) for the same volume contents, dtype, nz, ny,
 * nx, n_views, det_h, det_w and n_samples: those fix the read plan and
 * nothing else does, so the poses, K, spacing and mode may change between
 * the calls.  When the plan reads the
 * caller's volume itself (LDS-staged boxes, or launches too sparse for a copy)
 * the call is drr_forward.  Arguments, validation and errors are drr_forward's.
 * The library cannot check the copy: after the volume's contents change, or
 * with a workspace that holds no copy of it, the images are of whatever the
 * workspace holds (reads stay inside it). */
int drr_forward_reuse(const void *volume, int dtype, int nz, int ny, int nx,
                      const float *spacing, const float *K, const float *poses, int n_views,
                      int det_h, int det_w, int n_samples, int mode, float *out,
                      float *line_integral, void *workspace, size_t workspace_bytes,
                      void *stream);

/* drr_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, serving loops, harnesses that forbid hipMalloc): the same
 * arguments without the workspace, and the same launches and results.  What
 * drr_forward keeps in its workspace (the corner-cell or z-pair copy of the
 * volume its read plan marches) goes into a fixed device array of
 * DRR_NO_ALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends; the call itself allocates nothing.
 *   A call whose plan needs more than DRR_NO_ALLOC_SCRATCH_BYTES (i.e.
 *   drr_workspace_bytes(..., DRR_WORKSPACE_FORWARD) above it) returns
 *   DRR_ERR_UNSUPPORTED and enqueues nothing.
 *   Every call on one GPU shares that GPU's array (each call rewrites all of
 *   the copy it reads before reading it): calls that overlap on one GPU --
 *   on two streams, or from two threads -- race, and must be serialised by
 *   the caller.
 *   The array's device address is looked up once per device, on the first
 *   call that needs it, with that device current (a HIP runtime call, no
 *   allocation). */
#define DRR_NO_ALLOC_SCRATCH_BYTES ((size_t)256 << 20)

int drr_forward_no_alloc(const void *volume, int dtype, int nz, int ny, int nx,
                         const float *spacing, const float *K, const float *poses, int n_views,
                         int det_h, int det_w, int n_samples, int mode, float *out,
                         float *line_integral, void *stream);

/* Volume gradient of the forward (flashdrr autograd backward / diffct
 * backproject): for upstream dL/dI = grad_out,
 *   y_p = grad_out_p * exp(-s_p)  (Beer-Lambert; s from the forward's line_integral)
 *   y_p = grad_out_p              (line integral; this is exactly A^T grad_out)
 * and every sample adds y_p * dz * w_corner to each of its 8 trilinear corners.
 *   grad_out      device, n_views*det_h*det_w floats
 *   line_integral device, same layout; required for Beer-Lambert, ignored (may be
 *                 NULL) for the line integral
 *   grad_volume   device, nz*ny*nx floats, OVERWRITTEN (zeroed, then accumulated)
 * The volume itself is not needed.  Views sparse against the voxels (fewer
 * than four samples per cell from one view) run brick by brick: each voxel is
 * written once from exact fixed-point sums, the same on every run.  Denser
 * views accumulate with fp32 atomics, so the result may differ between runs in
 * the last bits. */
int drr_backward_volume(int nz, int ny, int nx, const float *spacing, const float *K,
                        const float *poses, int n_views, int det_h, int det_w, int n_samples,
                        int mode, const float *grad_out, const float *line_integral,
                        float *grad_volume, void *workspace, size_t workspace_bytes,
                        void *stream);

/* Pose gradient of the forward (flashdrr API, VolumeRaycaster class text:
 * rendering is differentiable with respect to the view matrices; flashdrr
 * README, Features: gradients through the camera parameters).  For
 * L = sum_p grad_out_p I_p it writes dL/dP_v for every view's 3x4
 * world-to-camera [R | t], the twelve entries treated as independent (chain
 * them through any rotation parameterisation on the caller's side).  The
 * derivative includes the motion of the clipped range's end points (the box
 * planes that bound it) and of the sample spacing dz; the trilinear field is
 * differentiated within each cell (one-sided on cell faces).
 *   volume, dtype, spacing, K, poses, det_h, det_w, n_samples, mode: as drr_forward
 *   grad_out      device, n_views*det_h*det_w floats (dL/dI)
 *   grad_poses    device, n_views x 12 floats, row-major 3x4, OVERWRITTEN
 *   workspace     device, >= drr_workspace_bytes(..., DRR_WORKSPACE_POSE_BACKWARD),
 *                 256-byte aligned (it is never empty for n_views > 0)
 * View sums use fp64 atomics, so the result may differ between runs in the
 * last bits. */
int drr_backward_pose(const void *volume, int dtype, int nz, int ny, int nx, const float *spacing,
                      const float *K, const float *poses, int n_views, int det_h, int det_w,
                      int n_samples, int mode, const float *grad_out, float *grad_poses,
                      void *workspace, size_t workspace_bytes, void *stream);

/* drr_backward_pose without the relayout, as drr_forward_reuse for the
 * forward: `workspace` must already hold the read copy that an earlier
 * drr_backward_pose call wrote into it for the same volume contents, dtype,
 * nz, ny, nx, n_views, det_h, det_w and n_samples (poses, K, spacing, mode and
 * grad_out may change).  When the plan reads the caller's volume itself the
 * call is drr_backward_pose.  Arguments, validation and errors are
 * drr_backward_pose's; the library cannot check the copy (see
 * drr_forward_reuse). */
int drr_backward_pose_reuse(const void *volume, int dtype, int nz, int ny, int nx,
                            const float *spacing, const float *K, const float *poses, int n_views,
                            int det_h, int det_w, int n_samples, int mode, const float *grad_out,
                            float *grad_poses, void *workspace, size_t workspace_bytes,
                            void *stream);

/* Forward DRR in the cell-constant (Siddon) model (diffct 2.1.0, "Why
 * diffct": project() and backproject() are an exact adjoint pair for the
 * cell-constant Siddon model).  Each voxel is a constant box
 * [i sx - Ex/2, (i + 1) sx - Ex/2] x ... and the line integral of a ray is
 *   s = sum over voxels v of mu_v l_v,  l_v = length of the clipped ray in v,
 * with the same cameras, box clip, outputs and layouts as drr_forward (no
 * sample count: the lengths are exact).  A ray that lies exactly in a voxel
 * plane is given the voxel on the side of increasing index.
 *   volume, dtype, spacing, K, poses, det_h, det_w, mode, out, line_integral:
 *                 as drr_forward
 * No workspace is needed.  n_views, det_h or det_w equal to 0 is a valid empty
 * call. */
int drr_forward_siddon(const void *volume, int dtype, int nz, int ny, int nx,
                       const float *spacing, const float *K, const float *poses, int n_views,
                       int det_h, int det_w, int mode, float *out, float *line_integral,
                       void *stream);

/* Volume gradient of drr_forward_siddon, its matched adjoint: every voxel
 * receives sum over rays of y_p l_v with y_p = grad_out_p * exp(-s_p)
 * (Beer-Lambert; s from drr_forward_siddon's line_integral) or grad_out_p
 * (line integral; this is A^T grad_out for the same A as the forward).
 *   grad_out, line_integral, grad_volume: as drr_backward_volume (grad_volume
 *                 is OVERWRITTEN)
 * The volume itself is not needed.  Views sparse against the voxels (fewer
 * than about four pieces per voxel from one view) run brick by brick: each
 * voxel is written once from exact fixed-point sums, the same on every run.
 * Denser views accumulate with fp32 atomics, so the result may differ between
 * runs in the last bits. */
int drr_backward_volume_siddon(int nz, int ny, int nx, const float *spacing, const float *K,
                               const float *poses, int n_views, int det_h, int det_w, int mode,
                               const float *grad_out, const float *line_integral,
                               float *grad_volume, void *stream);

/* ------------------------------------------------------------------------
 * The flashdrr front end: drr_render and its volume gradient.
 *
 * flashdrr.rendering API, VolumeRaycaster.forward: vol is (B, C, D, H, W)
 * in voxel space, view matrices number N = B * views_per_vol (view v renders
 * volume v / views_per_vol), output (N, C, H, W).  VolumeRaycaster.__init__:
 * density_factor scales the volume before integration; use_beer_lambert =
 * False selects front-to-back alpha compositing.  compute_clipping_distances:
 * one near and one far distance per view from the camera to the closest and
 * farthest volume point, widened by a margin.  Transfer functions,
 * piecewise_linear_channelwise: a per-channel piecewise-linear map over sorted
 * knots that extends its end segments, applied to the volume before ray
 * casting.
 *
 * Readings (the pages give no formulas):
 *   - mu = tf_c(x) voxel by voxel when a transfer function is given (else
 *     mu = x), then sampled trilinearly as in drr_forward;
 *   - optical depth tau = f dz sum_k mu(t_k) with f = density_factor;
 *     Beer-Lambert 1 - exp(-tau); line integral tau;
 *   - alpha compositing: sample k is a slab of thickness dz that emits mu_k
 *     with opacity alpha_k = 1 - exp(-f mu_k dz) behind the transmittance
 *     T_k = prod_{j<k} (1 - alpha_j); I = sum_k T_k alpha_k mu_k;
 *   - DRR_CLIP_NEAR_FAR: near = max(distance from the camera centre to the
 *     closest point of the box - margin, 0), far = distance to the farthest
 *     box corner + margin; every ray of the view samples the midpoints of
 *     [near, far] (far <= near renders 0) and reads 0 outside the volume
 *     (zero padding: a trilinear corner outside [0, n-1] holds 0);
 *   - transfer segment i spans [xp_i, xp_{i+1}); below xp_1 the first and from
 *     xp_{K-2} on the last segment applies; at a knot the slope is the right
 *     segment's. */

/* Workspace bytes of drr_render (for_backward = DRR_WORKSPACE_FORWARD),
 * drr_render_backward_volume (DRR_WORKSPACE_VOLUME_BACKWARD) or
 * drr_render_backward_pose (DRR_WORKSPACE_POSE_BACKWARD) for these sizes;
 * tf_knots = 0 means no transfer function.  0 for invalid sizes or when none
 * is needed.  The forward (and the pose backward) use it for a copy of every
 * channel-volume when rays reuse cells enough -- corner cells or z-pairs,
 * zero-padded in the near/far mode, which always reads a copy -- or for the
 * mapped fp32 volumes; the compositing backward for a z-pair copy its
 * coefficient passes read (from about one sample per cell), or for the mapped
 * fp32 volumes with a transfer function, followed by 8 bytes per channel-volume
 * (rounded up to 256) for the largest value of that copy, which bounds the
 * coefficients without a pass over the samples.  Values are mapped by the
 * transfer function in every copy. */
size_t drr_render_workspace_bytes(int n_volumes, int n_channels, int nz, int ny, int nx,
                                  int dtype, int n_views, int det_h, int det_w, int n_samples,
                                  int mode, int clip, int tf_knots, int for_backward);

/* Render n_volumes volumes of n_channels channels.
 *   volume        device, n_volumes x n_channels x nz x ny x nx elements of
 *                 dtype, C-contiguous (each channel-volume x fastest)
 *   spacing, K    host, as drr_forward
 *   poses         device, n_views x 12 fp32 world-to-camera [R | t];
 *                 n_views must be a multiple of n_volumes
 *   n_samples     samples per ray
 *   mode          DRR_BEER_LAMBERT, DRR_LINE_INTEGRAL or DRR_ALPHA_COMPOSITE
 *   density_factor  f (finite)
 *   clip, margin  DRR_CLIP_BOX (margin ignored) or DRR_CLIP_NEAR_FAR with the
 *                 margin in mm (finite; negative narrows the range)
 *   tf_xp, tf_yp  host or both NULL: n_channels x tf_knots floats, each
 *                 channel's knots strictly increasing; 2 <= tf_knots and
 *                 n_channels * tf_knots <= 128
 *   out           device, n_views x n_channels x det_h x det_w floats
 *   aux           device or NULL: the optical depth tau in the same layout
 *                 (the Beer-Lambert backward needs it)
 *   workspace     device, >= drr_render_workspace_bytes(..., DRR_WORKSPACE_FORWARD),
 *                 256-byte aligned
 * Limits as drr_forward per channel-volume; n_volumes * n_channels <= 65535.
 * drr_forward(...) equals drr_render with one volume, one channel, f = 1, the
 * box clip and no transfer function. */
int drr_render(const void *volume, int dtype, int n_volumes, int n_channels, int nz, int ny,
               int nx, const float *spacing, const float *K, const float *poses, int n_views,
               int det_h, int det_w, int n_samples, int mode, float density_factor, int clip,
               float margin, const float *tf_xp, const float *tf_yp, int tf_knots, float *out,
               float *aux, void *workspace, size_t workspace_bytes, void *stream);

/* drr_render without the relayout (as drr_forward_reuse for drr_forward):
 * `workspace` must already hold the read copy that an earlier drr_render call
 * wrote into it for the same volume contents, dtype, n_volumes, n_channels,
 * nz, ny, nx, n_views, det_h, det_w, n_samples, clip and transfer function
 * (the copy is of the mapped values when there is one); poses, K, spacing,
 * mode, density_factor and margin may change.  When the plan reads the
 * caller's volumes themselves the call is drr_render.  Arguments, validation
 * and errors are drr_render's; the library cannot check the copy. */
int drr_render_reuse(const void *volume, int dtype, int n_volumes, int n_channels, int nz,
                     int ny, int nx, const float *spacing, const float *K, const float *poses,
                     int n_views, int det_h, int det_w, int n_samples, int mode,
                     float density_factor, int clip, float margin, const float *tf_xp,
                     const float *tf_yp, int tf_knots, float *out, float *aux, void *workspace,
                     size_t workspace_bytes, void *stream);

/* Gradient of L = sum grad_out * out with respect to the input volume x of
 * drr_render (same arguments).  Per sample k of a ray, dL/dmu at its trilinear
 * corners receives grad_out * c_k * w_corner with
 *   Beer-Lambert       c_k = f dz exp(-tau)
 *   line integral      c_k = f dz
 *   alpha compositing  c_k = T_k (alpha_k + f dz (1 - alpha_k) mu_k)
 *                            - f dz sum_{j>k} T_j alpha_j mu_j
 * and with a transfer function dL/dx = dL/dmu tf'(x) per voxel.
 *   volume        device; required for alpha compositing and with a transfer
 *                 function, else may be NULL
 *   grad_out      device, n_views x n_channels x det_h x det_w floats
 *   out           device, the forward's image; required for alpha compositing
 *   aux           device, the forward's optical depth; required for Beer-Lambert
 *   grad_volume   device, n_volumes x n_channels x nz x ny x nx floats, OVERWRITTEN
 *   workspace     device, >= drr_render_workspace_bytes(..., DRR_WORKSPACE_VOLUME_BACKWARD),
 *                 256-byte aligned
 * Accumulation uses fp32 atomics, so the result may differ between runs in
 * the last bits. */
int drr_render_backward_volume(const void *volume, int dtype, int n_volumes, int n_channels,
                               int nz, int ny, int nx, const float *spacing, const float *K,
                               const float *poses, int n_views, int det_h, int det_w,
                               int n_samples, int mode, float density_factor, int clip,
                               float margin, const float *tf_xp, const float *tf_yp,
                               int tf_knots, const float *grad_out, const float *out,
                               const float *aux, float *grad_volume, void *workspace,
                               size_t workspace_bytes, void *stream);

/* Pose gradient of drr_render (flashdrr API, VolumeRaycaster class text:
 * rendering is differentiable with respect to the view matrices, in either
 * integration mode of VolumeRaycaster.__init__): for L = sum grad_out * out it
 * writes dL/dP_v for every view's 3x4 [R | t] as drr_backward_pose does,
 * summed over the view's channels, with the density factor, the transfer
 * function and the clip of the call.  Every mode: Beer-Lambert and the line
 * integral, and alpha compositing, whose per-sample coefficient (as in
 * drr_render_backward_volume) and dI/ddz come from one front-to-back pass
 * (the forward's image is not needed).  Either clip: with DRR_CLIP_BOX the
 * range ends move with the planes that bound each ray; with
 * DRR_CLIP_NEAR_FAR with the camera centre alone (near and far are distances
 * from it), and samples read the zero padding.
 *   grad_out      device, n_views x n_channels x det_h x det_w floats
 *   grad_poses    device, n_views x 12 floats, OVERWRITTEN
 *   workspace     device, >= drr_render_workspace_bytes(..., DRR_WORKSPACE_POSE_BACKWARD),
 *                 256-byte aligned (never empty for n_views > 0)
 * drr_backward_pose is this call for one volume, one channel, f = 1 and no
 * transfer function. */
int drr_render_backward_pose(const void *volume, int dtype, int n_volumes, int n_channels,
                             int nz, int ny, int nx, const float *spacing, const float *K,
                             const float *poses, int n_views, int det_h, int det_w,
                             int n_samples, int mode, float density_factor, int clip,
                             float margin, const float *tf_xp, const float *tf_yp, int tf_knots,
                             const float *grad_out, float *grad_poses, void *workspace,
                             size_t workspace_bytes, void *stream);

/* drr_render_backward_pose without the relayout: `workspace` must already
 * hold the read copy that an earlier drr_render_backward_pose call wrote into
 * it for the same volume contents and launch shape as drr_render_reuse lists
 * (poses, K, spacing, mode, density_factor, margin and grad_out may change).
 * Arguments, validation and errors are drr_render_backward_pose's; the
 * library cannot check the copy. */
int drr_render_backward_pose_reuse(const void *volume, int dtype, int n_volumes, int n_channels,
                                   int nz, int ny, int nx, const float *spacing, const float *K,
                                   const float *poses, int n_views, int det_h, int det_w,
                                   int n_samples, int mode, float density_factor, int clip,
                                   float margin, const float *tf_xp, const float *tf_yp,
                                   int tf_knots, const float *grad_out, float *grad_poses,
                                   void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Camera conventions of the flashdrr front end (flashdrr.rendering API:
 * get_vtk_view_mat builds a camera-to-world 4 x 4 whose 3 x 3 block holds the
 * camera axes [right, up, forward] as columns and whose fourth column is the
 * camera position, in RAS; VolumeRaycaster.forward takes the volume in IJK
 * voxel space with a ras2ijk affine; set_fov takes the vertical field of view).
 *
 * Readings: ras2ijk maps RAS to the continuous voxel index with voxel centres
 * at integers, i along x (the fastest axis), j along y, k along z; its linear
 * part must be a scaled orthonormal matrix (orthogonal voxel axes), whose row
 * norms are the inverse voxel sizes.  The rendering frame of every other call
 * (box centred at the origin) is then a rigid image of RAS.  The HZ camera's
 * image x axis is `right`, its image y axis is -`up` (rows grow downwards),
 * z is `forward`; the view matrix's 3 x 3 block is taken as orthonormal. */

/* K = [[f, 0, W/2], [0, f, H/2], [0, 0, 1]], f = (H/2) / tan(fov/2), for a
 * vertical field of view fov_deg in (0, 180) degrees.  Host only: K receives
 * 9 floats, row-major. */
int drr_intrinsics_from_fov(float fov_deg, int det_h, int det_w, float *K);

/* World-to-camera HZ poses for the rendering frame of a volume of nz x ny x nx
 * voxels placed by ras2ijk:
 *   view_mats  device, n_views x 16 floats, row-major camera-to-world 4 x 4
 *   ras2ijk    host, 16 floats, row-major 4 x 4 (last row 0 0 0 1)
 *   poses      device, n_views x 12 floats, OVERWRITTEN ([R | t] for drr_render,
 *              drr_forward, ...)
 *   spacing    host or NULL: receives the 3 voxel sizes (sx, sy, sz) in mm
 * With M the rotation block and c the position of a view matrix, Q X + o the
 * rendering frame of a RAS point X and D = diag(1, -1, 1):
 *   R = D M^T Q^T,  t = -R (Q c + o). */
int drr_poses_from_view_matrices(const float *view_mats, int n_views, const float *ras2ijk,
                                 int nz, int ny, int nx, float *poses, float *spacing,
                                 void *stream);

/* Chain rule of drr_poses_from_view_matrices: from grad_poses = dL/d[R | t]
 * (device, n_views x 12, e.g. from drr_backward_pose) it writes
 * grad_view_mats = dL/d(view_mats) (device, n_views x 16, OVERWRITTEN; the
 * bottom row is 0), every entry of the view matrix treated as independent. */
int drr_view_matrices_backward(const float *view_mats, int n_views, const float *ras2ijk, int nz,
                               int ny, int nx, const float *grad_poses, float *grad_view_mats,
                               void *stream);

/* Gaussian-Poisson noise surrogate (flashdrr.rendering API,
 * VolumeRaycaster.apply_poisson): Gaussian noise of standard deviation
 * sqrt(T / i0) added to a transmission map T, clamped to [0, 1]:
 *   out = clamp(T + z sqrt(max(T, 0) / i0), 0, 1)
 * with the standard-normal draws z supplied by the caller (so a run is
 * reproducible and the same draws serve the backward).
 *   transmission, noise, out  device, n floats each
 *   i0            mean photon count at the source, finite and > 0
 * Readings: a transmission below 0 gets no noise. */
int drr_poisson_surrogate(const float *transmission, const float *noise, long long n, float i0,
                          float *out, void *stream);

/* Gradient of the surrogate: grad_transmission = grad_out * d out / dT, with
 * dT passed through where T + z sqrt(T / i0) lies in [0, 1] (as torch.clamp
 * does) and 0 elsewhere; d/dT of the noise term is z / (2 sqrt(T i0)) for
 * T > 0 and is left out for T <= 0.  All device, n floats each. */
int drr_poisson_surrogate_backward(const float *transmission, const float *noise, long long n,
                                   float i0, const float *grad_out, float *grad_transmission,
                                   void *stream);

/* Static description of a drr_status value. */
const char *drr_status_string(int status);

/* Thread-local description of the last failing call on this thread ("" if none). */
const char *drr_last_error(void);

/* DRR_ABI_VERSION of the loaded library. */
int drr_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DRR_H */
