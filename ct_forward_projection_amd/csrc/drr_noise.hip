// drr_noise.hip -- flashdrr's Gaussian-Poisson surrogate (flashdrr.rendering
// API, VolumeRaycaster.apply_poisson): Gaussian noise of standard deviation
// sqrt(T / i0) added to a transmission map T and clamped to [0, 1], with the
// standard-normal draws z given by the caller.  Elementwise and HBM-bound:
// 8 bytes in and 4 out per element forward, 12 in and 4 out backward; four
// elements per thread with 16-byte loads when every pointer is 16-byte
// aligned (n4 = n / 4 then, else 0 and the element loop does all).
//
// A transmission below 0 gets no noise; the derivative passes where the value
// lies in [0, 1] (as torch.clamp's does) and omits the noise term's
// z / (2 sqrt(T i0)) where T <= 0.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "drr_internal.hpp"

namespace drr {

__device__ inline float surrogate(float t, float z, float inv_i0, float& v)
{
    const float sd = t > 0.0f ? sqrtf(t * inv_i0) : 0.0f;
    v = fmaf(z, sd, t);
    return fminf(fmaxf(v, 0.0f), 1.0f);
}

__device__ inline float surrogate_grad(float t, float z, float i0, float inv_i0, float g)
{
    float v;
    surrogate(t, z, inv_i0, v);
    const bool pass = v >= 0.0f && v <= 1.0f;
    const float dv = t > 0.0f ? 1.0f + z / (2.0f * sqrtf(t * i0)) : 1.0f;
    return pass ? g * dv : 0.0f;
}

__global__ __launch_bounds__(256) void drr_poisson_kernel(const float* __restrict__ T,
                                                          const float* __restrict__ z, size_t n,
                                                          size_t n4, float inv_i0,
                                                          float* __restrict__ out)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    const float4* T4 = reinterpret_cast<const float4*>(T);
    const float4* z4 = reinterpret_cast<const float4*>(z);
    float4* o4 = reinterpret_cast<float4*>(out);
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
        const float4 t = T4[i], r = z4[i];
        float v;
        o4[i] = make_float4(surrogate(t.x, r.x, inv_i0, v), surrogate(t.y, r.y, inv_i0, v),
                            surrogate(t.z, r.z, inv_i0, v), surrogate(t.w, r.w, inv_i0, v));
    }
    for (size_t i = 4 * n4 + (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        float v;
        out[i] = surrogate(T[i], z[i], inv_i0, v);
    }
}

__global__ __launch_bounds__(256) void drr_poisson_backward_kernel(
    const float* __restrict__ T, const float* __restrict__ z, size_t n, size_t n4, float i0,
    float inv_i0, const float* __restrict__ g, float* __restrict__ grad)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    const float4* T4 = reinterpret_cast<const float4*>(T);
    const float4* z4 = reinterpret_cast<const float4*>(z);
    const float4* g4 = reinterpret_cast<const float4*>(g);
    float4* d4 = reinterpret_cast<float4*>(grad);
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
        const float4 t = T4[i], r = z4[i], u = g4[i];
        d4[i] = make_float4(surrogate_grad(t.x, r.x, i0, inv_i0, u.x),
                            surrogate_grad(t.y, r.y, i0, inv_i0, u.y),
                            surrogate_grad(t.z, r.z, i0, inv_i0, u.z),
                            surrogate_grad(t.w, r.w, i0, inv_i0, u.w));
    }
    for (size_t i = 4 * n4 + (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        grad[i] = surrogate_grad(T[i], z[i], i0, inv_i0, g[i]);
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

static int noise_blocks(size_t n)
{
    const size_t b = (n / 4 + 255) / 256;
    return (int)(b < 1 ? 1 : (b > 8192 ? 8192 : b));
}

hipError_t launch_poisson(const float* T, const float* z, size_t n, float i0, float* out,
                          hipStream_t stream)
{
    if (n == 0) return hipSuccess;
    const size_t n4 = aligned16(T) && aligned16(z) && aligned16(out) ? n / 4 : 0;
    hipLaunchKernelGGL(drr_poisson_kernel, dim3(noise_blocks(n)), dim3(256), 0, stream, T, z, n,
                       n4, 1.0f / i0, out);
    return hipGetLastError();
}

hipError_t launch_poisson_backward(const float* T, const float* z, size_t n, float i0,
                                   const float* g, float* grad, hipStream_t stream)
{
    if (n == 0) return hipSuccess;
    const size_t n4 =
        aligned16(T) && aligned16(z) && aligned16(g) && aligned16(grad) ? n / 4 : 0;
    hipLaunchKernelGGL(drr_poisson_backward_kernel, dim3(noise_blocks(n)), dim3(256), 0, stream,
                       T, z, n, n4, i0, 1.0f / i0, g, grad);
    return hipGetLastError();
}

}  // namespace drr
