// drr_camera.hip -- the flashdrr camera conventions turned into the HZ poses the
// renderer takes, and the chain rule of that conversion for pose gradients.
//
// Source pages: flashdrr.rendering API, get_vtk_view_mat (camera-to-world 4 x 4
// with columns [right, up, forward] and the camera position, in RAS);
// VolumeRaycaster.forward (volume in IJK voxel space, ras2ijk affine);
// VolumeRaycaster.set_fov (vertical field of view); nanodrr introduction
// (P = K [R | t]).
//
// The rendering frame is centred on the volume: a RAS point X sits at
// p = Q X + o with Q = S L (L the linear part of ras2ijk, S = diag(s), s_a the
// voxel size 1 / |row a of L|) and o = S (b - (n - 1) / 2).  A view matrix with
// rotation block M and position c gives the HZ world-to-camera pose
//   R = D M^T Q^T,  t = -R (Q c + o),   D = diag(1, -1, 1)
// (image x = right, image y = -up, z = forward; M and Q orthonormal).  One
// thread per view, fp64 inside.
#include <hip/hip_runtime.h>

#include "drr_internal.hpp"

namespace drr {

__global__ __launch_bounds__(64) void drr_vtk_pose_kernel(const float* __restrict__ view_mats,
                                                          int n_views, VolumeFrame F,
                                                          float* __restrict__ poses)
{
    const int v = (int)(blockIdx.x * blockDim.x + threadIdx.x);
    if (v >= n_views) return;
    const float* m = view_mats + 16 * (size_t)v;
    double M[9], c[3];
#pragma unroll
    for (int r = 0; r < 3; ++r) {
#pragma unroll
        for (int k = 0; k < 3; ++k) M[r * 3 + k] = (double)m[r * 4 + k];
        c[r] = (double)m[r * 4 + 3];
    }
    const double D[3] = {1.0, -1.0, 1.0};
    double R[9], Cp[3];
#pragma unroll
    for (int a = 0; a < 3; ++a)
        Cp[a] = F.Q[a * 3 + 0] * c[0] + F.Q[a * 3 + 1] * c[1] + F.Q[a * 3 + 2] * c[2] + F.o[a];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
#pragma unroll
        for (int j = 0; j < 3; ++j)      // (M^T Q^T)_ij = sum_k M_ki Q_jk
            R[i * 3 + j] = D[i] * (M[0 * 3 + i] * F.Q[j * 3 + 0] + M[1 * 3 + i] * F.Q[j * 3 + 1] +
                                   M[2 * 3 + i] * F.Q[j * 3 + 2]);
    }
    float* out = poses + 12 * (size_t)v;
#pragma unroll
    for (int i = 0; i < 3; ++i) {
#pragma unroll
        for (int j = 0; j < 3; ++j) out[i * 4 + j] = (float)R[i * 3 + j];
        out[i * 4 + 3] = (float)-(R[i * 3 + 0] * Cp[0] + R[i * 3 + 1] * Cp[1] + R[i * 3 + 2] * Cp[2]);
    }
}

// Gradient of L with respect to the view matrices from dL/dR, dL/dt (the pose
// gradient): with G' = dL/dR - dL/dt Cp^T,
//   dL/dM = Q^T G'^T D,   dL/dc = -M D dL/dt,   bottom row 0.
__global__ __launch_bounds__(64) void drr_vtk_pose_backward_kernel(
    const float* __restrict__ view_mats, int n_views, VolumeFrame F,
    const float* __restrict__ grad_poses, float* __restrict__ grad_view)
{
    const int v = (int)(blockIdx.x * blockDim.x + threadIdx.x);
    if (v >= n_views) return;
    const float* m = view_mats + 16 * (size_t)v;
    const float* gp = grad_poses + 12 * (size_t)v;
    double M[9], c[3], GR[9], gt[3];
#pragma unroll
    for (int r = 0; r < 3; ++r) {
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            M[r * 3 + k] = (double)m[r * 4 + k];
            GR[r * 3 + k] = (double)gp[r * 4 + k];
        }
        c[r] = (double)m[r * 4 + 3];
        gt[r] = (double)gp[r * 4 + 3];
    }
    const double D[3] = {1.0, -1.0, 1.0};
    double Cp[3], Gp[9];
#pragma unroll
    for (int a = 0; a < 3; ++a)
        Cp[a] = F.Q[a * 3 + 0] * c[0] + F.Q[a * 3 + 1] * c[1] + F.Q[a * 3 + 2] * c[2] + F.o[a];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
#pragma unroll
        for (int j = 0; j < 3; ++j) Gp[i * 3 + j] = GR[i * 3 + j] - gt[i] * Cp[j];
    }
    float* out = grad_view + 16 * (size_t)v;
#pragma unroll
    for (int a = 0; a < 3; ++a) {
#pragma unroll
        for (int b = 0; b < 3; ++b)      // (Q^T G'^T D)_ab = sum_j Q_ja G'_bj D_b
            out[a * 4 + b] = (float)(D[b] * (F.Q[0 * 3 + a] * Gp[b * 3 + 0] +
                                             F.Q[1 * 3 + a] * Gp[b * 3 + 1] +
                                             F.Q[2 * 3 + a] * Gp[b * 3 + 2]));
        out[a * 4 + 3] = (float)-(M[a * 3 + 0] * D[0] * gt[0] + M[a * 3 + 1] * D[1] * gt[1] +
                                  M[a * 3 + 2] * D[2] * gt[2]);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) out[12 + k] = 0.0f;
}

hipError_t launch_vtk_poses(const float* view_mats, int n_views, const VolumeFrame& F,
                            float* poses, hipStream_t stream)
{
    if (n_views == 0) return hipSuccess;
    hipLaunchKernelGGL(drr_vtk_pose_kernel, dim3((n_views + 63) / 64), dim3(64), 0, stream,
                       view_mats, n_views, F, poses);
    return hipGetLastError();
}

hipError_t launch_vtk_poses_backward(const float* view_mats, int n_views, const VolumeFrame& F,
                                     const float* grad_poses, float* grad_view,
                                     hipStream_t stream)
{
    if (n_views == 0) return hipSuccess;
    hipLaunchKernelGGL(drr_vtk_pose_backward_kernel, dim3((n_views + 63) / 64), dim3(64), 0,
                       stream, view_mats, n_views, F, grad_poses, grad_view);
    return hipGetLastError();
}

}  // namespace drr
