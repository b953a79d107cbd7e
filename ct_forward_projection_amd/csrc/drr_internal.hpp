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

hipError_t launch_forward(const LaunchArgs& a, const void* vol, int dtype, float* out,
                          float* s_out, hipStream_t stream);
hipError_t launch_backward(const LaunchArgs& a, const float* grad_out, const float* s_in,
                           float* grad, hipStream_t stream);

}  // namespace drr
