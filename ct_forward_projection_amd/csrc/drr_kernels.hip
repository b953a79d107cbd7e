// drr_kernels.hip -- gfx950 kernels of the cone-beam DRR path.
//
//   drr_march_kernel    forward: ray generation, box clip, N midpoint samples of
//                       the clamped trilinear volume, fp32 accumulation,
//                       Beer-Lambert (-expm1(-s)) or raw line-integral epilogue.
//                       (flashdrr.rendering VolumeRaycaster.__init__ / forward;
//                       diffct Quickstart project.)
//   drr_scatter_kernel  backward: the same samples scatter y dz w_corner into the
//                       fp32 volume gradient, y = g exp(-s) (Beer-Lambert) or g
//                       (line integral), pre-reduced in fixed point in an LDS
//                       window.
//                       (flashdrr VolumeRaycaster: differentiable in the volume;
//                       diffct Quickstart backproject = A^T.)
//   drr_fill_kernel     zeroes the gradient before the scatter (a kernel rather
//                       than a memset so that the sequence is graph-capturable).
//
//   drr_cells_kernel    optional relayout: the corner-cell copy of the volume the
//                       march reads when samples reuse cells enough (always in
//                       the near/far mode, where the cells carry zero padding);
//                       with a transfer function it writes mapped fp32 cells.
//   drr_transfer_kernel the transfer function applied to every voxel (fp32 copy)
//                       when a mapped volume is marched without cells.
//   drr_slope_kernel    the backward's last step with a transfer function:
//                       dL/dx = dL/dmu tf'(x) per voxel.
//   drr_value_bound_kernel  the largest value of what the compositing backward
//                       reads, and whether any is negative or not finite: a
//                       closed-form bound on its coefficients.
//                       The compositing backward runs in the same kernel: each
//                       sample is gathered again for its own coefficient.
//
// Every kernel covers several volumes and channels per launch (flashdrr API,
// VolumeRaycaster.forward: (B, C, D, H, W) volumes, N = B * views_per_vol views,
// output (N, C, H, W)): a launch walks (view, channel) pairs.
//
// The march is gather-bound, not a contraction, so there is no MFMA here: the
// design levers are the number of vector-memory instructions per sample (x-pair
// loads: 4 per sample instead of 8; corner cells: 1 or 2), cheap full-rate
// integer position stepping, and wave-coherent 8 x 8 pixel tiles so
// neighbouring lanes gather from the same cache lines.
#include <limits.h>

#include "drr_device.hpp"
#include "drr_internal.hpp"
#include "drr_sample.hpp"
#include "drr_stage.hpp"
#include "drr_window.hpp"

namespace drr {

// Corner-cell relayout: cell (i, j, k), 0 <= i <= nx etc., holds the eight
// corners (x0, x1) x (y0, y1) x (z0, z1) of the trilinear cell whose low corner
// is voxel (i-1, j-1, k-1), in the CornerVals order: clamped to the volume
// (ZP = false) or 0 outside it (ZP, the near/far mode's zero padding).  With TF
// the corners are mapped by channel c's transfer function and written as fp32.
// One thread per cell, consecutive threads on consecutive cells;
// blockIdx.y = channel-volume (b * C + c).
template <typename Tin, typename Tout, bool ZP, bool TF>
__global__ __launch_bounds__(256) void drr_cells_kernel(const Tin* __restrict__ vol, int nx, int ny,
                                                        int nz, size_t in_stride,
                                                        Tout* __restrict__ cells,
                                                        size_t out_stride, int C, TransferFn tf)
{
    static_assert(TF || sizeof(Tin) == sizeof(Tout), "no transfer: cells keep the dtype");
    const int cv = (int)blockIdx.y, ch = cv % C;
    vol += (size_t)cv * in_stride;
    cells += (size_t)cv * out_stride;
    const int cx = nx + 1, cy = ny + 1;
    const long long n = (long long)cx * cy * (nz + 1);
    const size_t sy = (size_t)nx, sz = (size_t)nx * ny;
    for (long long id = (long long)blockIdx.x * blockDim.x + threadIdx.x; id < n;
         id += (long long)gridDim.x * blockDim.x) {
        const int i = (int)(id % cx);
        const long long rest = id / cx;
        const int j = (int)(rest % cy), k = (int)(rest / cy);
        const size_t x0 = (size_t)clampi(i - 1, 0, nx - 1), x1 = (size_t)clampi(i, 0, nx - 1);
        const size_t y0 = (size_t)clampi(j - 1, 0, ny - 1) * sy, y1 = (size_t)clampi(j, 0, ny - 1) * sy;
        const size_t z0 = (size_t)clampi(k - 1, 0, nz - 1) * sz, z1 = (size_t)clampi(k, 0, nz - 1) * sz;
        const Tin v[8] = {vol[z0 + y0 + x0], vol[z0 + y0 + x1], vol[z0 + y1 + x0], vol[z0 + y1 + x1],
                          vol[z1 + y0 + x0], vol[z1 + y0 + x1], vol[z1 + y1 + x0], vol[z1 + y1 + x1]};
        Tout o[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            if constexpr (TF) {
                float m;
                o[c] = transfer_eval(tf, ch, widen(v[c]), m);
            } else {
                o[c] = v[c];
            }
        }
        if constexpr (ZP) {
            // corner c of cell (i, j, k) is voxel (i - 1 + (c & 1), j - 1 + ..., ...)
            const bool xl = i >= 1, xh = i <= nx - 1, yl = j >= 1, yh = j <= ny - 1;
            const bool zl = k >= 1, zh = k <= nz - 1;
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const bool in = ((c & 1) ? xh : xl) && ((c & 2) ? yh : yl) && ((c & 4) ? zh : zl);
                if (!in) o[c] = Tout(0);
            }
        }
        Tout* dst = cells + (size_t)id * 8;
#pragma unroll
        for (int c = 0; c < 8; ++c) dst[c] = o[c];
    }
}

// Z-pair relayout: element (x, y, z) of the copy, 0 <= z <= nz - 2, holds
// voxels (x, y, z) and (x, y, z + 1) side by side (mapped by channel c's
// transfer function into fp32 with TF).  Each thread takes a run of up to
// kZRun pairs down one (x, y) column (blockIdx.z: the run, blockIdx.y: the
// channel-volume), so every voxel is read and mapped once; consecutive threads
// on consecutive x keep reads and writes coalesced.
constexpr int kZRun = 8;

template <typename Tin, typename Tout, bool TF>
__global__ __launch_bounds__(256) void drr_zpair_kernel(const Tin* __restrict__ vol, int nx,
                                                        int ny, int nz, size_t in_stride,
                                                        Tout* __restrict__ pairs,
                                                        size_t out_stride, int C, TransferFn tf)
{
    static_assert(TF || sizeof(Tin) == sizeof(Tout), "no transfer: pairs keep the dtype");
    const int cv = (int)blockIdx.y, ch = cv % C;
    const size_t slice = (size_t)nx * ny;
    const size_t xy = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (xy >= slice) return;
    const int z0 = (int)blockIdx.z * kZRun, z1 = min(z0 + kZRun, nz - 1);
    vol += (size_t)cv * in_stride + xy;
    pairs += (size_t)cv * out_stride;                // pair (z, xy) is pair z slice + xy
    auto value = [&](int z) -> Tout {
        if constexpr (TF) {
            float m;
            return transfer_eval(tf, ch, widen(vol[(size_t)z * slice]), m);
        } else {
            return vol[(size_t)z * slice];
        }
    };
    auto store = [&](int z, Tout lo, Tout hi) {
        const size_t id = (size_t)z * slice + xy;
        if constexpr (sizeof(Tout) == 4) {
            reinterpret_cast<float2*>(pairs)[id] = make_float2(lo, hi);
        } else {
            reinterpret_cast<uint32_t*>(pairs)[id] = (uint32_t)lo | ((uint32_t)hi << 16);
        }
    };
    if (z1 - z0 == kZRun) {
        // a full run: all kZRun + 1 loads issued before the first store
        Tout v[kZRun + 1];
#pragma unroll
        for (int i = 0; i <= kZRun; ++i) v[i] = value(z0 + i);
#pragma unroll
        for (int i = 0; i < kZRun; ++i) store(z0 + i, v[i], v[i + 1]);
    } else {
        Tout lo = value(z0);
        for (int z = z0; z < z1; ++z) {
            const Tout hi = value(z + 1);
            store(z, lo, hi);
            lo = hi;
        }
    }
}

// Zero-padded z-pair relayout (near/far mode): element (X, Y, Z) of the copy,
// 0 <= X <= nx + 1, 0 <= Y <= ny + 1, 0 <= Z <= nz, holds voxels
// (X - 1, Y - 1, Z - 1) and (X - 1, Y - 1, Z) side by side, 0 for a voxel
// outside the volume (mapped by channel c's transfer function into fp32 with
// TF; the padding stays 0).  One thread per element; blockIdx.y = channel-volume.
template <typename Tin, typename Tout, bool TF>
__global__ __launch_bounds__(256) void drr_zpair_pad_kernel(const Tin* __restrict__ vol, int nx,
                                                            int ny, int nz, size_t in_stride,
                                                            Tout* __restrict__ pairs,
                                                            size_t out_stride, int C,
                                                            TransferFn tf)
{
    static_assert(TF || sizeof(Tin) == sizeof(Tout), "no transfer: pairs keep the dtype");
    const int cv = (int)blockIdx.y, ch = cv % C;
    vol += (size_t)cv * in_stride;
    pairs += (size_t)cv * out_stride;
    const int px = nx + 2, py = ny + 2;
    const size_t n = (size_t)px * py * (size_t)(nz + 1);
    const size_t sy = (size_t)nx, sz = (size_t)nx * ny;
    for (size_t id = (size_t)blockIdx.x * blockDim.x + threadIdx.x; id < n;
         id += (size_t)gridDim.x * blockDim.x) {
        const int X = (int)(id % px);
        const size_t rest = id / px;
        const int Y = (int)(rest % py), Z = (int)(rest / py);
        const int x = X - 1, y = Y - 1, z = Z - 1;
        const bool xy = x >= 0 && x < nx && y >= 0 && y < ny;
        const size_t base = (size_t)y * sy + (size_t)x;
        float v[2] = {0.0f, 0.0f};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int zz = z + h;
            if (xy && zz >= 0 && zz < nz) {
                const float w = widen(vol[(size_t)zz * sz + base]);
                if constexpr (TF) {
                    float m;
                    v[h] = transfer_eval(tf, ch, w, m);
                } else {
                    v[h] = w;
                }
            }
        }
        if constexpr (sizeof(Tout) == 4) {
            reinterpret_cast<float2*>(pairs)[id] = make_float2(v[0], v[1]);
        } else {
            // no transfer: v holds the bf16 values exactly
            reinterpret_cast<uint32_t*>(pairs)[id] =
                (__float_as_uint(v[0]) >> 16) | (__float_as_uint(v[1]) & 0xffff0000u);
        }
    }
}

// mu = tf(x) for every voxel of every channel-volume (blockIdx.y), fp32 out.
template <typename Tin>
__global__ __launch_bounds__(256) void drr_transfer_kernel(const Tin* __restrict__ vol,
                                                           size_t n_vox, size_t in_stride,
                                                           float* __restrict__ mu,
                                                           size_t out_stride, int C,
                                                           TransferFn tf)
{
    const int cv = (int)blockIdx.y, ch = cv % C;
    vol += (size_t)cv * in_stride;
    mu += (size_t)cv * out_stride;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_vox;
         i += (size_t)gridDim.x * blockDim.x) {
        float m;
        mu[i] = transfer_eval(tf, ch, widen(vol[i]), m);
    }
}

// grad = grad * tf'(x) for every voxel of every channel-volume (blockIdx.y).
template <typename Tin>
__global__ __launch_bounds__(256) void drr_slope_kernel(const Tin* __restrict__ vol, size_t n_vox,
                                                        size_t in_stride, float* __restrict__ grad,
                                                        int C, TransferFn tf)
{
    const int cv = (int)blockIdx.y, ch = cv % C;
    vol += (size_t)cv * in_stride;
    grad += (size_t)cv * n_vox;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_vox;
         i += (size_t)gridDim.x * blockDim.x) {
        float m;
        transfer_eval(tf, ch, widen(vol[i]), m);
        grad[i] *= m;
    }
}

// Value bounds of a compositing backward's read copy, per channel-volume
// (blockIdx.y; n_elem values every `stride` values): out[2 cv] turns non-zero
// if any value is negative or not finite, out[2 cv + 1] is raised to the bit
// pattern of the largest value (non-negative floats order as their bits).
// out starts at zero.
template <typename T>
__global__ __launch_bounds__(256) void drr_value_bound_kernel(const T* __restrict__ src,
                                                              size_t n_elem, size_t stride,
                                                              int* __restrict__ out)
{
    const int cv = (int)blockIdx.y;
    src += (size_t)cv * stride;
    float vmax = 0.0f;
    bool bad = false;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_elem;
         i += (size_t)gridDim.x * blockDim.x) {
        const float v = widen(src[i]);
        bad = bad || !(v >= 0.0f) || !isfinite(v);          // NaN fails v >= 0
        vmax = fmaxf(vmax, v);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) vmax = fmaxf(vmax, __shfl_xor(vmax, off, 64));
    const bool any_bad = __ballot(bad) != 0;
    if ((threadIdx.x & 63) == 0) {
        if (any_bad) atomicOr(out + 2 * cv, 1);
        atomicMax(out + 2 * cv + 1, __float_as_int(vmax));
    }
}

// Samples a lane keeps in flight: their gathers are all issued before any is
// consumed, so each wave has 4 samples' loads outstanding (8 in the plain
// z-pair march, see drr_march_kernel).
constexpr int kInflight = 4;

// Pixel of a thread when SPLIT adjacent lanes share one ray (small launches):
// a workgroup covers a (256 / SPLIT)-ray square patch, ray-major.
template <int SPLIT>
__device__ inline PixelCoord split_pixel(int tile, int tiles_x, int tiles_per_view)
{
    constexpr int side = SPLIT == 4 ? 8 : (SPLIT == 16 ? 4 : 2);
    static_assert(side * side * SPLIT == kBlock, "SPLIT must be 4, 16 or 64");
    PixelCoord p;
    p.view = tile / tiles_per_view;
    const int t = tile - p.view * tiles_per_view;
    const int ty = t / tiles_x, tx = t - ty * tiles_x;
    const int ray = threadIdx.x / SPLIT;
    p.r = ty * side + ray / side;
    p.c = tx * side + ray % side;
    return p;
}

template <int SPLIT>
constexpr int march_tile_side() { return SPLIT == 1 ? kTile : (SPLIT == 4 ? 8 : (SPLIT == 16 ? 4 : 2)); }

// One sample of front-to-back alpha compositing (flashdrr API,
// VolumeRaycaster.__init__: use_beer_lambert = False): the sample is a slab of
// thickness dz emitting v with opacity alpha = 1 - exp(-f v dz) behind the
// transmittance T = exp(-tau) of the samples in front of it, carried as the
// running product T <- T (1 - alpha) = T - T alpha (one fp64 fma, no
// exponential per sample).  T and I run in fp64 so that neither drifts over
// long rays; the line integral (also returned) is summed like the other modes'.
__device__ inline void composite(float v, float fdz, double& T, double& I)
{
    const float alpha = -expm1f(-(fdz * v));
    I = fma(T, (double)(alpha * v), I);
    T = fma(-T, (double)alpha, T);
}

// Forward DRR.  SPLIT = 1: one ray per lane (16 x 16 tiles of four 8 x 8 wave
// sub-tiles).  SPLIT > 1 (launches with few rays): SPLIT adjacent lanes share
// a ray, lane j taking samples j, j + SPLIT, ... (neighbouring lanes still
// gather neighbouring voxels), and their partial sums meet in a cross-lane
// reduction, so a 64 x 64 detector still fills the chip.  `src` is the volume
// (Pair, Single) or its corner-cell copy (Cell); `src_bytes` the size of one
// channel-volume of it, b.src_stride the distance between them.  The tiles of
// a launch run over (view, channel) pairs.  MODE = kAlpha composites (one lane
// per ray: the over operator is sequential); CLIP = kClipNearFar samples the
// view's near/far range through zero-padded cells.
template <typename T, Layout L, int MODE, int SPLIT, int CLIP>
__global__ __launch_bounds__(kBlock) void drr_march_kernel(
    const T* __restrict__ src, uint32_t src_bytes, VolumeDesc V, Intrinsics K,
    const float* __restrict__ poses, int H, int W, int N, int tiles_x, int tiles_per_view,
    Batch b, float* __restrict__ out, float* __restrict__ s_out)
{
    constexpr bool ZP = CLIP == kClipNearFar;
    static_assert(!ZP || L == Layout::Cell || L == Layout::ZPair,
                  "the near/far mode reads zero-padded cells or z-pairs");
    static_assert(MODE != kAlpha || SPLIT == 1, "compositing runs one lane per ray");
    const int tile = xcd_contiguous_tile((int)blockIdx.x, (int)gridDim.x);
    PixelCoord px;
    int j = 0;
    if constexpr (SPLIT == 1) {
        px = tile_pixel_rows(tile, tiles_x, tiles_per_view);
    } else {
        px = split_pixel<SPLIT>(tile, tiles_x, tiles_per_view);
        j = (int)threadIdx.x % SPLIT;
    }
    // every lane of a ray sees the same pixel, so a ray's lanes leave together
    if (px.r >= H || px.c >= W) return;

    // px.view counts (view, channel) pairs
    const int view = px.view / b.C, ch = px.view - view * b.C;
    const int cvol = (view / b.vpv) * b.C + ch;
    ViewGeom G;
    view_setup(poses + 12 * view, K, G);
    MarchRay R;
    bool hit;
    if constexpr (CLIP == kClipBox) {
        hit = ray_setup(G, V, px.r, px.c, N, R);
    } else {
        double t_near, t_far;
        view_near_far(G, V, b.margin, t_near, t_far);
        hit = ray_setup_range(G, V, px.r, px.c, N, t_near, t_far, R);
    }
    float s = 0.0f;
    double T_c = 1.0, I_c = 0.0;   // compositing
    if (hit) {
        const char* base = reinterpret_cast<const char*>(src) + (uint64_t)cvol * b.src_stride;
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, (int)src_bytes, kBufferWord3);
        // samples [k_lo, k_hi): all of them, or in the near/far mode those
        // that can reach the volume (the rest read zero padding and add 0)
        int k_lo = 0, k_hi = N;
        if constexpr (ZP) padded_support(R, V, N, k_lo, k_hi);
        const int k_first = k_lo + j;
        int64_t qx = R.q0[0] + (int64_t)k_first * R.dq[0];
        int64_t qy = R.q0[1] + (int64_t)k_first * R.dq[1];
        int64_t qz = R.q0[2] + (int64_t)k_first * R.dq[2];
        const int64_t dqx = (int64_t)SPLIT * R.dq[0], dqy = (int64_t)SPLIT * R.dq[1];
        const int64_t dqz = (int64_t)SPLIT * R.dq[2];
        const int n_mine = k_first < k_hi ? (k_hi - k_first + SPLIT - 1) / SPLIT : 0;
        const float fdz = b.f * R.dz;
        // samples in flight per group: eight for plain z-pair reads with one ray
        // per lane, whose loads miss L2 about half the time (16 views of 200^2:
        // 0.652 -> 0.562 ms fp32, 0.509 -> 0.448 ms bf16); the zero-padded
        // compositing march (0.404 -> 0.436 ms), x-pair reads (1.64 -> 1.71 ms on
        // 4 volumes x 2 channels) and split lanes run better with four (fewer
        // registers, more waves), and ten measured no better than eight
        constexpr int kGroup =
            (SPLIT == 1 && L == Layout::ZPair && !ZP && MODE != kAlpha) ? 2 * kInflight : kInflight;
        // independent partial sums, one per in-flight sample: a shorter fp32
        // summation chain as well
        float acc[kGroup];
#pragma unroll
        for (int i = 0; i < kGroup; ++i) acc[i] = 0.0f;
        int k = 0;
        for (; k + kGroup <= n_mine; k += kGroup) {
            SampleAddr A[kGroup];
            CornerVals c[kGroup];
#pragma unroll
            for (int i = 0; i < kGroup; ++i) {
                A[i] = sample_addr<T, L, ZP>(V, qx, qy, qz);
                qx += dqx; qy += dqy; qz += dqz;
            }
#pragma unroll
            for (int i = 0; i < kGroup; ++i) gather<T, L>(rs, A[i], c[i]);
            // keep every gather of the group ahead of the first use: otherwise
            // the scheduler sinks each sample's loads to just before their use
            // and a wave never has more than one sample's loads in flight
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < kGroup; ++i) {
                const float v = ZP ? interpolate_exact(A[i], c[i]) : interpolate(A[i], c[i]);
                if constexpr (MODE == kAlpha) composite(v, fdz, T_c, I_c);
                acc[i] += v;
            }
        }
        for (; k < n_mine; ++k) {
            const SampleAddr A = sample_addr<T, L, ZP>(V, qx, qy, qz);
            qx += dqx; qy += dqy; qz += dqz;
            CornerVals c;
            gather<T, L>(rs, A, c);
            const float v = ZP ? interpolate_exact(A, c) : interpolate(A, c);
            if constexpr (MODE == kAlpha) composite(v, fdz, T_c, I_c);
            acc[0] += v;
        }
#pragma unroll
        for (int i = 0; i < kGroup; ++i) s += acc[i];
    }
    if constexpr (SPLIT > 1) {
        // all SPLIT lanes of this ray are here (hit or miss alike)
#pragma unroll
        for (int off = SPLIT / 2; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
        if (j != 0) return;
    }
    if (hit) s *= R.dz;
    const float tau = b.f * s;                 // optical depth f dz sum mu
    const float res = MODE == kAlpha ? (float)I_c
                                     : (MODE == kBeerLambert ? -expm1f(-tau) : tau);
    const size_t o = ((size_t)px.view * H + px.r) * W + px.c;
    out[o] = res;
    if (s_out) s_out[o] = tau;
}

// LDS-staged forward (box clip).  The rays of a 16 x 16 tile are close and
// straight, so the voxels a chunk of their samples touch form a small box:
// the workgroup loads that box once from the caller's volume into LDS -- in
// unclamped index space, each entry the clamped voxel (clamp to edge), mapped
// by the transfer function when there is one, widened to fp32 -- and every
// sample then reads its eight corners from LDS at fixed offsets (+1 in x, +ex
// in y, +ex ey in z), four ds_read2 per sample instead of two 16-byte global
// loads.  Chunks are sized like the backward's windows (halved until the box
// fits, doubled while it has room); a chunk whose box does not fit even for
// one sample gathers its corners from global memory.  No relayout pass and no
// workspace.
template <typename T, int MODE, bool TF>
__global__ __launch_bounds__(kBlock) void drr_march_staged_kernel(
    const T* __restrict__ src, uint32_t src_bytes, VolumeDesc V, Intrinsics K,
    const float* __restrict__ poses, int H, int W, int N, int tiles_x, int tiles_per_view,
    Batch b, TransferFn tf, float* __restrict__ out, float* __restrict__ s_out)
{
    // samples per group of the box march: LDS reads are short, and groups of
    // two measured best (1024^2: 4 -> 2 samples 0.438 -> 0.433 ms, 8: 0.470 ms)
    constexpr int kStagedGroup = 2;
    __shared__ float box[kStageCap];
    __shared__ int red[(kBlock / 64) * 6];
    __shared__ int bb[6];
    const int tile = xcd_contiguous_tile((int)blockIdx.x, (int)gridDim.x);
    const PixelCoord px = tile_pixel(tile, tiles_x, tiles_per_view);
    const int view = px.view / b.C, ch = px.view - view * b.C;
    const int cvol = (view / b.vpv) * b.C + ch;
    const bool mine = px.r < H && px.c < W;
    MarchRay R;
    bool hit = false;
    if (mine) {
        ViewGeom G;
        view_setup(poses + 12 * view, K, G);
        hit = ray_setup(G, V, px.r, px.c, N, R);
    }
    const char* base = reinterpret_cast<const char*>(src) + (uint64_t)cvol * b.src_stride;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, (int)src_bytes, kBufferWord3);
    const float fdz = hit ? b.f * R.dz : 0.0f;
    float acc[kStagedGroup];
#pragma unroll
    for (int i = 0; i < kStagedGroup; ++i) acc[i] = 0.0f;
    double T_c = 1.0, I_c = 0.0;

    int S = N;
    int k0 = 0;
    while (k0 < N) {
        S = min(S, N - k0);
        int ext[3] = {1, 1, 1}, lo[3] = {0, 0, 0};
        long long vol_cells = 1;
        bool any;
        for (;;) {
            // unclamped floor indices bounding the chunk's samples (its end samples)
            int lo_f[3] = {INT_MAX, INT_MAX, INT_MAX}, hi_f[3] = {INT_MAX, INT_MAX, INT_MAX};
            if (hit) {
#pragma unroll
                for (int a = 0; a < 3; ++a) {
                    const int fa = fixed_floor(R.q0[a] + (int64_t)k0 * R.dq[a]);
                    const int fb = fixed_floor(R.q0[a] + (int64_t)(k0 + S - 1) * R.dq[a]);
                    lo_f[a] = min(fa, fb);
                    hi_f[a] = max(fa, fb);
                }
            }
            any = chunk_box(lo_f, hi_f, red, bb, lo, ext, vol_cells);
            if (!any || vol_cells <= kStageCap || S == 1) break;
            S = max(1, S >> 1);
        }
        if (!any) break;                             // no ray of this tile hits the box
        const int ey = ext[0], ez = ext[0] * ext[1];
        if (vol_cells <= kStageCap) {
            stage_fill<T, TF>(box, (int)vol_cells, rs, V, lo, ext, tf, ch);
            __syncthreads();
            if (hit) {
                // positions relative to the box corner, so that the fixed-point
                // floor is the box index itself; byte strides of the box
                int64_t qx = R.q0[0] + (int64_t)k0 * R.dq[0] - (int64_t)lo[0] * kFixedOne;
                int64_t qy = R.q0[1] + (int64_t)k0 * R.dq[1] - (int64_t)lo[1] * kFixedOne;
                int64_t qz = R.q0[2] + (int64_t)k0 * R.dq[2] - (int64_t)lo[2] * kFixedOne;
                const uint32_t sy = 4u * (uint32_t)ey, sz = 4u * (uint32_t)ez;
                const char* bx = reinterpret_cast<const char*>(box);
                int k = k0;
                for (; k + kStagedGroup <= k0 + S; k += kStagedGroup) {
                    SampleAddr A[kStagedGroup];
                    CornerVals c[kStagedGroup];
#pragma unroll
                    for (int i = 0; i < kStagedGroup; ++i) {
                        A[i].fx = fixed_frac(qx);
                        A[i].fy = fixed_frac(qy);
                        A[i].fz = fixed_frac(qz);
                        A[i].o = box_offset(qx, qy, qz, sy, sz);
                        qx += R.dq[0]; qy += R.dq[1]; qz += R.dq[2];
                        serial_step(qx, qy, qz);
                    }
#pragma unroll
                    for (int i = 0; i < kStagedGroup; ++i) box_corners(bx + A[i].o, sy, sz, c[i]);
#pragma unroll
                    for (int i = 0; i < kStagedGroup; ++i) {
                        const float val = interpolate(A[i], c[i]);
                        if constexpr (MODE == kAlpha) composite(val, fdz, T_c, I_c);
                        acc[i] += val;
                    }
                }
                for (; k < k0 + S; ++k) {
                    SampleAddr A;
                    A.fx = fixed_frac(qx);
                    A.fy = fixed_frac(qy);
                    A.fz = fixed_frac(qz);
                    A.o = box_offset(qx, qy, qz, sy, sz);
                    qx += R.dq[0]; qy += R.dq[1]; qz += R.dq[2];
                    CornerVals c;
                    box_corners(bx + A.o, sy, sz, c);
                    const float val = interpolate(A, c);
                    if constexpr (MODE == kAlpha) composite(val, fdz, T_c, I_c);
                    acc[0] += val;
                }
            }
            __syncthreads();
        } else if (hit) {
            // the box does not fit: gather this chunk's corners from global memory
            int64_t qx = R.q0[0] + (int64_t)k0 * R.dq[0];
            int64_t qy = R.q0[1] + (int64_t)k0 * R.dq[1];
            int64_t qz = R.q0[2] + (int64_t)k0 * R.dq[2];
            for (int k = k0; k < k0 + S; ++k) {
                const int ix = fixed_floor(qx), iy = fixed_floor(qy), iz = fixed_floor(qz);
                SampleAddr A;
                A.fx = fixed_frac(qx);
                A.fy = fixed_frac(qy);
                A.fz = fixed_frac(qz);
                qx += R.dq[0]; qy += R.dq[1]; qz += R.dq[2];
                CornerVals c;
#pragma unroll
                for (int n = 0; n < 8; ++n)
                    c.v[n] = staged_value<T, TF>(rs, V, ix + (n & 1), iy + ((n >> 1) & 1),
                                                 iz + (n >> 2), tf, ch);
                const float val = interpolate(A, c);
                if constexpr (MODE == kAlpha) composite(val, fdz, T_c, I_c);
                acc[0] += val;
            }
        }
        k0 += S;
        if (vol_cells * 2 <= kStageCap) S *= 2;
    }
    if (!mine) return;
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < kStagedGroup; ++i) s += acc[i];
    if (hit) s *= R.dz;
    const float tau = b.f * s;                 // optical depth f dz sum mu
    const float res = MODE == kAlpha ? (float)I_c
                                     : (MODE == kBeerLambert ? -expm1f(-tau) : tau);
    const size_t o = ((size_t)px.view * H + px.r) * W + px.c;
    out[o] = res;
    if (s_out) s_out[o] = tau;
}

// Zero padding (near/far mode): 1 for a corner index inside [0, n - 1], 0
// outside, per axis and end: m = (x0, x1, y0, y1, z0, z1).  Used with the
// clamped Cell, whose indices then only serve as in-range addresses.
__device__ inline void pad_mask(const VolumeDesc& V, int64_t qx, int64_t qy, int64_t qz,
                                float m[6])
{
    const int i[3] = {fixed_floor(qx), fixed_floor(qy), fixed_floor(qz)};
#pragma unroll
    for (int a = 0; a < 3; ++a) {
        m[2 * a] = (uint32_t)i[a] < (uint32_t)V.n[a] ? 1.0f : 0.0f;
        m[2 * a + 1] = (uint32_t)(i[a] + 1) < (uint32_t)V.n[a] ? 1.0f : 0.0f;
    }
}

// Trilinear weights of one sample, scaled by yd = y dz: w[c] for corner c
// (bit 0 = x1, bit 1 = y1, bit 2 = z1); with ZP the pad mask drops corners
// outside the volume.
template <bool ZP = false>
__device__ inline void corner_weights(const Cell& C, float yd, float w[8],
                                      const float* m = nullptr)
{
    float wz1 = yd * C.fz, wz0 = yd * (1.0f - C.fz);
    float fy1 = C.fy, fy0 = 1.0f - C.fy;
    float fx1 = C.fx, fx0 = 1.0f - C.fx;
    if constexpr (ZP) {
        fx0 *= m[0]; fx1 *= m[1];
        fy0 *= m[2]; fy1 *= m[3];
        wz0 *= m[4]; wz1 *= m[5];
    }
    const float w11 = wz1 * fy1, w10 = wz1 * fy0;
    const float w01 = wz0 * fy1, w00 = wz0 * fy0;
    w[0] = w00 * fx0;
    w[1] = w00 * fx1;
    w[2] = w01 * fx0;
    w[3] = w01 * fx1;
    w[4] = w10 * fx0;
    w[5] = w10 * fx1;
    w[6] = w11 * fx0;
    w[7] = w11 * fx1;
}

template <bool ZP = false>
__device__ inline void scatter_sample_global(float* __restrict__ grad, uint32_t sy, uint32_t sz,
                                             const Cell& C, float yd, const float* m = nullptr)
{
    float w[8];
    corner_weights<ZP>(C, yd, w, m);
    const uint32_t r00 = (uint32_t)C.z0 * sz + (uint32_t)C.y0 * sy;
    const uint32_t r01 = (uint32_t)C.z0 * sz + (uint32_t)C.y1 * sy;
    const uint32_t r10 = (uint32_t)C.z1 * sz + (uint32_t)C.y0 * sy;
    const uint32_t r11 = (uint32_t)C.z1 * sz + (uint32_t)C.y1 * sy;
    const uint32_t x0 = (uint32_t)C.x0, x1 = (uint32_t)C.x1;
    unsafeAtomicAdd(grad + r00 + x0, w[0]);
    unsafeAtomicAdd(grad + r00 + x1, w[1]);
    unsafeAtomicAdd(grad + r01 + x0, w[2]);
    unsafeAtomicAdd(grad + r01 + x1, w[3]);
    unsafeAtomicAdd(grad + r10 + x0, w[4]);
    unsafeAtomicAdd(grad + r10 + x1, w[5]);
    unsafeAtomicAdd(grad + r11 + x0, w[6]);
    unsafeAtomicAdd(grad + r11 + x1, w[7]);
}

// Fixed-point value of a register sum for the window, rounded to nearest.
// TRUNC: the sum already carries +-1/2 with the sign of all its terms, so
// truncation toward zero rounds it (half away from zero) in one conversion.
template <bool TRUNC>
__device__ inline int to_window(float w)
{
    return TRUNC ? (int)w : __float2int_rn(w);
}

// Add eight fixed-point weights at the window entry of LDS byte address `at`
// and its corner offsets (row and slice strides wy, wz in bytes).
template <bool TRUNC = false>
__device__ inline void window_add_at(uint32_t at, int wy, int wz, const float w[8])
{
    char* p = (char*)(__attribute__((address_space(3))) char*)(uintptr_t)at;
    int* r0 = reinterpret_cast<int*>(p);
    int* r1 = reinterpret_cast<int*>(p + wy);
    int* r2 = reinterpret_cast<int*>(p + wz);
    int* r3 = reinterpret_cast<int*>(p + wz + wy);
    atomicAdd(r0, to_window<TRUNC>(w[0]));
    atomicAdd(r0 + 1, to_window<TRUNC>(w[1]));
    atomicAdd(r1, to_window<TRUNC>(w[2]));
    atomicAdd(r1 + 1, to_window<TRUNC>(w[3]));
    atomicAdd(r2, to_window<TRUNC>(w[4]));
    atomicAdd(r2 + 1, to_window<TRUNC>(w[5]));
    atomicAdd(r3, to_window<TRUNC>(w[6]));
    atomicAdd(r3 + 1, to_window<TRUNC>(w[7]));
}

// Per-sample coefficient of the compositing backward (MODE = kAlpha).  For
// I = sum_k T_k alpha_k v_k with alpha_k = 1 - exp(-f v_k dz) and
// T_k = exp(-f dz sum_{j<k} v_j), sample k's own weight is
//   dI/dv_k = T_k (alpha_k + f dz (1 - alpha_k) v_k) - f dz sum_{j>k} T_j alpha_j v_j
// (its emission and opacity, and the transmittance it takes from every later
// sample); the later-sample sum is the forward's I minus the running emission
// up to k.  Each call reads the sample's corners again from the linear volume
// (the caller's, or the fp32 mapped copy): four x-pair loads with clamp to edge,
// or eight single loads of the zero-padded cell in the near/far mode (and for
// volumes one voxel wide); it advances the running state, so samples are
// visited in order; the transmittance (a running product, as in the forward)
// and the running emission are fp64.
template <typename T, bool ZP, bool ZPAIR>
struct AlphaCoef {
    __amdgpu_buffer_rsrc_t rs;
    uint32_t sy, sz;               // element strides of the volume (linear reads)
    float fdz, g;
    double I, trans, run;          // forward image, transmittance, running emission

    // mu at a sample from its clamped (or zero-padded) cell: eight loads
    __device__ float value(const Cell& C, const float* m) const
    {
        float w[8];
        corner_weights<ZP>(C, 1.0f, w, m);
        const uint32_t r00 = (uint32_t)C.z0 * sz + (uint32_t)C.y0 * sy;
        const uint32_t r01 = (uint32_t)C.z0 * sz + (uint32_t)C.y1 * sy;
        const uint32_t r10 = (uint32_t)C.z1 * sz + (uint32_t)C.y0 * sy;
        const uint32_t r11 = (uint32_t)C.z1 * sz + (uint32_t)C.y1 * sy;
        const uint32_t idx[8] = {r00 + C.x0, r00 + C.x1, r01 + C.x0, r01 + C.x1,
                                 r10 + C.x0, r10 + C.x1, r11 + C.x0, r11 + C.x1};
        float val[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) val[c] = load_one<T>(rs, idx[c] * (uint32_t)sizeof(T));
        float v = 0.0f;
#pragma unroll
        for (int c = 0; c < 8; ++c) v = fmaf(w[c], val[c], v);
        return v;
    }

    // mu at a sample, clamp to edge, from four x-pair loads (nx >= 2): the pair
    // starts at clamp(ix, 0, nx - 2) and the x weight is pinned to 0 or 1 at the
    // clamped edges, rows y and z are clamped
    __device__ float value_pairs(const VolumeDesc& V, int64_t qx, int64_t qy, int64_t qz) const
    {
        const int ix = fixed_floor(qx), iy = fixed_floor(qy), iz = fixed_floor(qz);
        const int xp = clampi(ix, 0, V.n[0] - 2);
        const float fx = __builtin_amdgcn_fmed3f(fixed_frac(qx) + (float)(ix - xp), 0.0f, 1.0f);
        const float fy = fixed_frac(qy), fz = fixed_frac(qz);
        const uint32_t y0 = (uint32_t)clampi(iy, 0, V.n[1] - 1) * sy;
        const uint32_t y1 = (uint32_t)clampi(iy + 1, 0, V.n[1] - 1) * sy;
        const uint32_t z0 = (uint32_t)clampi(iz, 0, V.n[2] - 1) * sz;
        const uint32_t z1 = (uint32_t)clampi(iz + 1, 0, V.n[2] - 1) * sz;
        const uint32_t rows[4] = {z0 + y0, z0 + y1, z1 + y0, z1 + y1};
        float a[4], b[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
            load_pair<T>(rs, (rows[r] + (uint32_t)xp) * (uint32_t)sizeof(T), a[r], b[r]);
        const float c00 = fmaf(fx, b[0] - a[0], a[0]), c10 = fmaf(fx, b[1] - a[1], a[1]);
        const float c01 = fmaf(fx, b[2] - a[2], a[2]), c11 = fmaf(fx, b[3] - a[3], a[3]);
        const float c0 = fmaf(fy, c10 - c00, c00), c1 = fmaf(fy, c11 - c01, c01);
        return fmaf(fz, c1 - c0, c0);
    }

    // the coefficient of the next sample (in order) from its mu
    __device__ float next_of(float v)
    {
        const float alpha = -expm1f(-(fdz * v));
        const float Tk = (float)trans;
        run = fma(trans, (double)(alpha * v), run);
        const float later = (float)(I - run);
        trans = fma(-trans, (double)alpha, trans);
        return g * (Tk * (alpha + fdz * (1.0f - alpha) * v) - fdz * later);
    }

    __device__ float next(const Cell& C, const float* m) { return next_of(value(C, m)); }

    // the coefficient of the next sample (in order) at fixed-point position q;
    // Vc: the volume with the byte strides of the z-pair copy (ZPAIR)
    __device__ float next_at(const VolumeDesc& V, const VolumeDesc& Vc, int64_t qx, int64_t qy,
                             int64_t qz)
    {
        if constexpr (ZPAIR) {
            const SampleAddr A = sample_addr<T, Layout::ZPair, ZP>(Vc, qx, qy, qz);
            CornerVals c;
            gather<T, Layout::ZPair>(rs, A, c);
            return next_of(ZP ? interpolate_exact(A, c) : interpolate(A, c));
        }
        if constexpr (!ZP) {
            if (V.n[0] >= 2) return next_of(value_pairs(V, qx, qy, qz));
        }
        Cell C;
        float m[6];
        cell_of(V, qx, qy, qz, C);
        if constexpr (ZP) pad_mask(V, qx, qy, qz, m);
        return next(C, m);
    }

    // ZPAIR: the coefficients of the next G samples (in order) at q, q + dq,
    // ..., with all G samples' gathers issued before the first is used (one
    // sample at a time leaves each load's latency exposed)
    template <int G>
    __device__ void next_group(const VolumeDesc& Vc, int64_t qx, int64_t qy, int64_t qz,
                               int64_t dqx, int64_t dqy, int64_t dqz, float out[G])
    {
        static_assert(ZPAIR, "grouped coefficients read the z-pair copy");
        SampleAddr A[G];
        CornerVals c[G];
#pragma unroll
        for (int i = 0; i < G; ++i) {
            A[i] = sample_addr<T, Layout::ZPair, ZP>(Vc, qx, qy, qz);
            qx += dqx; qy += dqy; qz += dqz;
        }
#pragma unroll
        for (int i = 0; i < G; ++i) gather<T, Layout::ZPair>(rs, A[i], c[i]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < G; ++i)
            out[i] = next_of(ZP ? interpolate_exact(A[i], c[i]) : interpolate(A[i], c[i]));
    }
};

// Backward scatter with LDS pre-reduction in fixed point.
//
// The rays of a tile walk their samples in chunks.  For each chunk the tile's
// corner bounding box (rays are straight, so a chunk's end samples bound it) is
// reduced across the workgroup; if it fits the window, every ray adds its
// samples' weights into the LDS window -- consecutive samples in the same cell
// are summed in registers first -- and the window is flushed with one global
// float atomic per touched voxel.  Coherent neighbouring rays hit the same
// voxels many times, so most same-address global atomics become LDS adds.
//
// The LDS adds are integer atomics on fixed-point weights: gfx950's LDS float
// atomic add is an order of magnitude slower than its integer add, and integer
// sums are exact, so the window total does not depend on the order of the
// adds.  The scale 2^e is chosen per tile so that no window entry overflows:
// one sample puts at most |c| on any voxel (c its coefficient: y dz for a
// whole ray in the Beer-Lambert and line-integral backward, c_k per sample in
// the compositing one, bounded in closed form from the largest value read, or
// by a first pass over the ray when values can be negative) and a ray has at
// most n = min(N, floor(2 / |dq|_inf) + 1) samples inside a voxel's 2 x 2 x 2
// support, so an entry never exceeds B = sum over the tile's rays of
// max|c| n, and 2^e B <= 2^30.  (|y dz| n is about |y| times the ray's
// length inside that support, so B stays small even for short chords.)  Each
// rounding adds at most 1/2 and an entry receives at most Cs = sum of n
// roundings, which must stay below 2^31 as well.  A tile whose coefficients
// are not finite or whose Cs is too large, or a chunk whose box does not fit
// the window even for one sample, uses global float atomics directly.
//
// The tiles of a launch run over (view, channel) pairs; a pair's rays scatter
// into the gradient of its channel-volume, with y scaled by the density factor
// (y = g f exp(-tau) or g f).  CLIP = kClipNearFar samples the view's
// near/far range and drops corners outside the volume (zero padding); all
// rays of a workgroup belong to one view, so they share the range.  MODE =
// kAlpha reads the volume (`vol`, one channel-volume of `vol_bytes` every
// bt.src_stride bytes: the caller's, its mapped fp32 copy, or with ZPAIR its
// z-pair copy, zero-padded in the near/far mode, of row and slice strides
// copy_row, copy_slice bytes) and the forward image `out_in`.
template <int MODE, int CLIP, typename T, bool ZPAIR>
__global__ __launch_bounds__(kBlock) void drr_scatter_kernel(
    VolumeDesc V, Intrinsics K, const float* __restrict__ poses, int H, int W, int N,
    int tiles_x, int tiles_per_view, Batch bt, const float* __restrict__ grad_out,
    const float* __restrict__ s_in, const float* __restrict__ out_in,
    const T* __restrict__ vol, uint32_t vol_bytes, uint32_t copy_row, uint32_t copy_slice,
    const int* __restrict__ vbound, float* __restrict__ grad, int win_cap)
{
    constexpr bool ZP = CLIP == kClipNearFar;
    constexpr bool ALPHA = MODE == kAlpha;
    // box clip without compositing: sample positions are taken relative to the
    // window's corner (the compositing coefficient needs absolute cells)
    constexpr bool REBASE = !ZP && !ALPHA;
    extern __shared__ int win[];                  // win_cap entries (dynamic LDS)
    __shared__ int red[(kBlock / 64) * 6];
    __shared__ int box[6];

    const int tile = xcd_contiguous_tile((int)blockIdx.x, (int)gridDim.x);
    const PixelCoord px = scatter_pixel(tile, tiles_x, tiles_per_view);
    // px.view counts (view, channel) pairs; a tile lies in one pair
    const int view = px.view / bt.C, ch = px.view - view * bt.C;
    const int cvol = (view / bt.vpv) * bt.C + ch;
    grad += (size_t)cvol * bt.grad_stride;
    // element strides of the gradient volume
    const uint32_t sy = (uint32_t)V.n[0], sz = (uint32_t)V.n[0] * (uint32_t)V.n[1];
    bool active = px.r < H && px.c < W;
    MarchRay R;
    float yd = 0.0f;
    AlphaCoef<T, ZP, ZPAIR> coef;
    VolumeDesc Vc = V;                  // byte strides of the z-pair copy (ZPAIR)
    Vc.row_bytes = copy_row;
    Vc.slice_bytes = copy_slice;
    if (active) {
        ViewGeom G;
        view_setup(poses + 12 * view, K, G);
        if constexpr (CLIP == kClipBox) {
            active = ray_setup(G, V, px.r, px.c, N, R);
        } else {
            double t_near, t_far;
            view_near_far(G, V, bt.margin, t_near, t_far);
            active = ray_setup_range(G, V, px.r, px.c, N, t_near, t_far, R);
        }
        if (active) {
            const size_t o = ((size_t)px.view * H + px.r) * W + px.c;
            if constexpr (ALPHA) {
                const char* base = reinterpret_cast<const char*>(vol) + (uint64_t)cvol * bt.src_stride;
                coef.rs = __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, (int)vol_bytes,
                                                            kBufferWord3);
                coef.sy = sy;
                coef.sz = sz;
                coef.fdz = bt.f * R.dz;
                coef.g = grad_out[o];
                coef.I = (double)out_in[o];
                active = coef.g != 0.0f;
            } else {
                float y = grad_out[o] * bt.f;
                if (MODE == kBeerLambert) y *= expf(-s_in[o]);
                yd = y * R.dz;
                active = yd != 0.0f;
            }
        }
    }

    // samples [k_lo, k_hi) of this ray: all of them, or in the near/far mode
    // those that can reach the volume (the rest read zero padding: they add
    // nothing to the gradient and leave the compositing state unchanged)
    int k_lo = 0, k_hi = N;
    if constexpr (ZP) {
        if (active) padded_support(R, V, N, k_lo, k_hi);
        active = active && k_hi > k_lo;
    }

    // fixed-point scale of this tile
    float B = 0.0f, Cs = 0.0f;
    float ray_cmax = 0.0f, ray_n = 0.0f;          // this ray's coefficient bound and n
    // compositing with values known to be >= 0: the bound also holds per chunk
    // from the running state (see the chunk loop)
    const bool alpha_closed = ALPHA && vbound != nullptr && vbound[2 * cvol] == 0 && bt.f >= 0.0f;
    if (active) {
        const double dq_inf = fmax(fmax(fabs((double)R.dq[0]), fabs((double)R.dq[1])),
                                   fabs((double)R.dq[2])) * 2.3283064365386963e-10;
        const double n = fmin((double)N, floor(2.0 / dq_inf) + 1.0);
        float cmax = fabsf(yd);
        if constexpr (ALPHA) {
            // With values v >= 0 (so 0 <= alpha <= f v dz, T <= 1) and f >= 0,
            // a coefficient g (T (alpha + f dz (1 - alpha) v) - f dz later) is
            // a difference of T (alpha + ...) <= 2 f dz vmax and f dz later,
            // where later = I - run and the running emission run lies in
            // [0, vmax] (the opacities along a ray sum to at most 1), so
            // |c| <= |g| f dz max(2 vmax, |I| + vmax) for any finite image I
            // the caller passes (2 vmax for the forward's own, I <= vmax), with
            // a margin for rounding, without visiting the samples; otherwise
            // (a negative or non-finite value, or no bounds) a first pass takes
            // the largest coefficient of the ray (NaN if any is not finite).
            // The closed form grows with a = f dz vmax, but a sample's opacity
            // saturates at 1: in media opaque within a sample or two (a > 2)
            // the coefficients stay near |g| while the bound keeps growing, and
            // a unit sized from it rounds the ray's smaller contributions away,
            // so such rays take the first pass's exact largest coefficient.
            const float fdz = coef.fdz;
            const float vmax = vbound != nullptr ? __int_as_float(vbound[2 * cvol + 1]) : 0.0f;
            if (vbound != nullptr && vbound[2 * cvol] == 0 && fdz >= 0.0f && fdz * vmax <= 2.0f) {
                const float I = (float)coef.I;
                cmax = (isfinite(I) && isfinite(coef.g))
                           ? fabsf(coef.g) * fdz * fmaxf(2.0f * vmax, fabsf(I) + vmax) * 1.0625f
                           : __builtin_nanf("");
            } else {
                coef.trans = 1.0;
                coef.run = 0.0;
                int64_t qx = R.q0[0] + (int64_t)k_lo * R.dq[0];
                int64_t qy = R.q0[1] + (int64_t)k_lo * R.dq[1];
                int64_t qz = R.q0[2] + (int64_t)k_lo * R.dq[2];
                bool finite = true;
                int k = k_lo;
                if constexpr (ZPAIR) {
                    for (; k + kInflight <= k_hi; k += kInflight) {
                        float ck[kInflight];
                        coef.template next_group<kInflight>(Vc, qx, qy, qz, R.dq[0], R.dq[1],
                                                            R.dq[2], ck);
                        qx += kInflight * R.dq[0]; qy += kInflight * R.dq[1];
                        qz += kInflight * R.dq[2];
#pragma unroll
                        for (int i = 0; i < kInflight; ++i) {
                            finite = finite && isfinite(ck[i]);
                            cmax = fmaxf(cmax, fabsf(ck[i]));
                        }
                    }
                }
                for (; k < k_hi; ++k) {
                    const float ck = coef.next_at(V, Vc, qx, qy, qz);
                    qx += R.dq[0]; qy += R.dq[1]; qz += R.dq[2];
                    finite = finite && isfinite(ck);
                    cmax = fmaxf(cmax, fabsf(ck));
                }
                if (!finite) cmax = __builtin_nanf("");
            }
            coef.trans = 1.0;
            coef.run = 0.0;
            // a ray whose coefficients are all 0 (through air: emission times
            // opacity is quadratic in mu) adds nothing
            active = cmax != 0.0f;
        }
        if (active) {
            B = (float)((double)cmax * n);
            Cs = (float)n;
            ray_cmax = cmax;
            ray_n = (float)n;
        }
    }
    // the window starts zeroed here; each flush zeroes the entries it read, so
    // every chunk finds the entries it uses at zero (block_sum2 synchronises)
    for (int i = threadIdx.x; i < win_cap; i += kBlock) win[i] = 0;
    block_sum2(B, Cs, reinterpret_cast<float*>(red));
    if (Cs == 0.0f) return;                        // no ray of this tile contributes
    const bool fixed_ok = isfinite(B) && B > 0.0f && Cs <= 1073741824.0f;
    float scale = 0.0f, inv_scale = 0.0f;
    if (fixed_ok) {
        const int e = clampi((int)floor(log2(1073741824.0 / (double)B)), -126, 126);
        scale = ldexpf(1.0f, e);
        inv_scale = ldexpf(1.0f, -e);
    }
    const float ys = yd * scale;

    int S = N;
    int k0 = 0;
    while (k0 < N) {
        S = min(S, N - k0);
        int ext[3], lo[3];
        long long vol_cells;
        for (;;) {
            int v[6] = {INT_MAX, INT_MAX, INT_MAX, INT_MAX, INT_MAX, INT_MAX};
            const int ka = max(k0, k_lo), kb = min(k0 + S, k_hi);   // this ray's samples
            if (active && ka < kb) {
#pragma unroll
                for (int a = 0; a < 3; ++a) {
                    const int64_t qa = R.q0[a] + (int64_t)ka * R.dq[a];
                    const int64_t qb = R.q0[a] + (int64_t)(kb - 1) * R.dq[a];
                    int fa = fixed_floor(qa), fb = fixed_floor(qb);
                    if constexpr (!REBASE) {
                        fa = clampi(fa, -1, V.n[a] - 1);
                        fb = clampi(fb, -1, V.n[a] - 1);
                    }
                    v[a] = min(fa, fb);
                    v[3 + a] = -(max(fa, fb) + 1);
                }
            }
            block_min6(v, red, box);
            if (box[0] == INT_MAX) break;            // no ray of the tile has samples here
            vol_cells = 1;
#pragma unroll
            for (int a = 0; a < 3; ++a) {
                lo[a] = box[a];
                ext[a] = max(-box[3 + a] - box[a] + 1, 1);
                vol_cells *= ext[a];
            }
            if (!fixed_ok || vol_cells <= win_cap || S == 1) break;
            S = max(1, S >> 1);
        }
        if (box[0] == INT_MAX) {                     // (near/far only) nothing to add
            k0 += S;
            continue;
        }
        if (fixed_ok && vol_cells <= win_cap) {
            const int n_win = (int)vol_cells;
            // this chunk's fixed-point scale.  Compositing's coefficients shrink
            // along the ray with the transmittance T and the emission still to
            // come, I - R: for samples k >= k0, T_k <= T_k0, the first term of
            // c_k is at most 2 f dz vmax T_k0, and |I - R_k| <= |I - R_k0-1| +
            // vmax T_k0 (the opacities from k0 on sum to at most T_k0), so
            // |c_k| <= |g| f dz (3 vmax T_k0 + |I - R_k0-1|).  Bounding each
            // chunk by the state at its start keeps the window's unit in step
            // with the coefficients: with the tile's bound alone, late samples'
            // contributions fall below half a unit and round to zero, a loss
            // that builds up where the rays leave the volume.
            float cs = scale, ci = inv_scale;
            if constexpr (ALPHA) {
                if (alpha_closed) {
                    float b = 0.0f, unused = 0.0f;
                    if (active && max(k0, k_lo) < min(k0 + S, k_hi)) {
                        const float vmax = __int_as_float(vbound[2 * cvol + 1]);
                        const float later = (float)fabs(coef.I - coef.run);
                        const float cb = fabsf(coef.g) * coef.fdz *
                                         (3.0f * vmax * (float)coef.trans + later) * 1.0625f;
                        b = fminf(ray_cmax, cb) * ray_n;
                    }
                    block_sum2(b, unused, reinterpret_cast<float*>(red));
                    if (isfinite(b) && b > 0.0f) {
                        const int e = clampi((int)floor(log2(1073741824.0 / (double)b)), -126, 126);
                        cs = ldexpf(1.0f, e);
                        ci = ldexpf(1.0f, -e);
                    }
                }
            }
            if (active) {
                // the window lives in unclamped index space: a sample's floor
                // places its eight corners at fixed offsets; entries at -1 or n
                // stand for the clamped edge voxel (clamp to edge) or for
                // nothing (zero padding) and are mapped when the window is
                // flushed.  With box clip every sample lies inside the box
                // [-0.5, n - 0.5], so its floor is in [-1, n - 1] already, and
                // the window bounds come from the same unclamped floors of the
                // chunk's end samples (positions are linear in k, so they bound
                // every sample between); otherwise floors are clamped to
                // [-1, n - 1], which keeps every corner on the voxel the clamped
                // corners would hit.
                const int wy = ext[0], wz = ext[0] * ext[1];
                const int64_t shift[3] = {REBASE ? (int64_t)lo[0] * kFixedOne : 0,
                                          REBASE ? (int64_t)lo[1] * kFixedOne : 0,
                                          REBASE ? (int64_t)lo[2] * kFixedOne : 0};
                // Without compositing the order of a chunk's samples is free:
                // the four lanes of each 2 x 2 block of the wave's pixel lattice
                // (neighbouring rays, often in the same cell at the same step)
                // walk the chunk's quarters starting from different ones, so
                // that one LDS atomic instruction rarely has several lanes on one
                // address (those serialise).  Compositing visits samples in order.
                constexpr int kParts = ALPHA ? 1 : 4;
                const int lane = (int)threadIdx.x & 63;
                const int first = ALPHA ? 0 : ((lane & 1) | ((lane >> 2) & 2));
                const int part = (S + kParts - 1) / kParts;
                // window strides in bytes and the window's LDS byte address
                const int wy4 = 4 * wy, wz4 = 4 * wz;
                const int w0 = (int)(uint32_t)(uintptr_t)(__attribute__((address_space(3))) int*)win;
                // the register sums' cell as the LDS address of its window
                // entry; without compositing it starts on a cell of one of the
                // lane's samples (sums still zero after truncation), so a window
                // add needs no test for a first sample
                int pbase = -1;
                if constexpr (REBASE) {
                    const int ki = min(k0 + first * part, k0 + S - 1);
                    const int ix = fixed_floor(R.q0[0] + (int64_t)ki * R.dq[0] - shift[0]);
                    const int iy = fixed_floor(R.q0[1] + (int64_t)ki * R.dq[1] - shift[1]);
                    const int iz = fixed_floor(R.q0[2] + (int64_t)ki * R.dq[2] - shift[2]);
                    pbase = w0 + 4 * ix + __mul24(iy, wy4) + __mul24(iz, wz4);
                }
                // a cell's register sums start at 0, or, without compositing
                // (one coefficient per ray), at +-1/2 with its sign, which lets
                // the window conversion truncate (see to_window)
                const float start = REBASE ? copysignf(0.5f, ys) : 0.0f;
                const float c96 = ys * 1.2621774483536189e-29f;     // ys 2^-96
                const float c64 = ys * 5.421010862427522e-20f;      // ys 2^-64
                float acc[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] = start;
                // ca: the compositing coefficient of the sample (ALPHA)
                auto sample = [&](int64_t& qx, int64_t& qy, int64_t& qz, float ca) {
                    const int fx = fixed_floor(qx), fy = fixed_floor(qy), fz = fixed_floor(qz);
                    float c = ys;
                    int base;
                    if constexpr (REBASE) {
                        // fy, fz >= 0: floors relative to the window corner
                        base = (int)fixed_floor_x4_add(
                            qx, mad_u24((uint32_t)fz, (uint32_t)wz4,
                                        mad_u24((uint32_t)fy, (uint32_t)wy4, (uint32_t)w0)));
                    } else {
                        const int ix = clampi(fx, -1, V.n[0] - 1);
                        const int iy = clampi(fy, -1, V.n[1] - 1);
                        const int iz = clampi(fz, -1, V.n[2] - 1);
                        if constexpr (ALPHA) c = ca * cs;
                        if constexpr (ZP) {
                            // a sample with every corner outside the volume adds nothing
                            if (fx != ix || fy != iy || fz != iz) c = 0.0f;
                        }
                        // clamped floors lie between the chunk's clamped end
                        // floors (clamping is monotone), so each is >= lo
                        base = (int)mad_u24((uint32_t)(iz - lo[2]), (uint32_t)wz4,
                                            mad_u24((uint32_t)(iy - lo[1]), (uint32_t)wy4,
                                                    (uint32_t)(w0 + 4 * (ix - lo[0]))));
                    }
                    // fractions: as they are (REBASE: times 2^32, the scale folded
                    // into the coefficient) or in [0, 1)
                    const float tx = REBASE ? (float)(uint32_t)qx : fixed_frac(qx);
                    const float ty = REBASE ? (float)(uint32_t)qy : fixed_frac(qy);
                    const float tz = REBASE ? (float)(uint32_t)qz : fixed_frac(qz);
                    serial_step_after(qx, qy, qz, tx, ty, tz);
                    qx += R.dq[0]; qy += R.dq[1]; qz += R.dq[2];
                    // consecutive samples in one cell are summed in registers;
                    // a new cell adds the finished sum to the window
                    const bool same = base == pbase;
                    if (!same && (REBASE || pbase >= 0))
                        window_add_at<REBASE>((uint32_t)pbase, wy4, wz4, acc);
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc[i] = same ? acc[i] : start;
                    if constexpr (REBASE)
                        add_weights8_scaled(tx, ty, tz, c96, c64, acc);
                    else
                        add_weights8(tx, ty, tz, c, acc);
                    pbase = base;
                };
                // without compositing every lane walks all S samples; when the
                // quarters are equal, every part has the same (uniform) length
                const bool even = REBASE && S % kParts == 0;
                for (int r = 0; r < kParts; ++r) {
                    const int kp = k0 + ((first + r) & (kParts - 1)) * part;
                    const int ka = max(kp, k_lo), kb = min(min(kp + part, k0 + S), k_hi);
                    int64_t qx = R.q0[0] + (int64_t)ka * R.dq[0] - shift[0];
                    int64_t qy = R.q0[1] + (int64_t)ka * R.dq[1] - shift[1];
                    int64_t qz = R.q0[2] + (int64_t)ka * R.dq[2] - shift[2];
                    if (even) {
                        // two samples per trip: the cell register alternates
                        // without a copy
                        for (int j = 0; j + 1 < part; j += 2) {
                            sample(qx, qy, qz, 0.0f);
                            sample(qx, qy, qz, 0.0f);
                        }
                        if (part & 1) sample(qx, qy, qz, 0.0f);
                    } else {
                        int k = ka;
                        if constexpr (ALPHA && ZPAIR) {
                            for (; k + kInflight <= kb; k += kInflight) {
                                float ca[kInflight];
                                coef.template next_group<kInflight>(Vc, qx, qy, qz, R.dq[0],
                                                                    R.dq[1], R.dq[2], ca);
#pragma unroll
                                for (int i = 0; i < kInflight; ++i) sample(qx, qy, qz, ca[i]);
                            }
                        }
                        for (; k < kb; ++k) {
                            float ca = 0.0f;
                            if constexpr (ALPHA) ca = coef.next_at(V, Vc, qx, qy, qz);
                            sample(qx, qy, qz, ca);
                        }
                    }
                }
                if (pbase >= 0) window_add_at<REBASE>((uint32_t)pbase, wy4, wz4, acc);
            }
            __syncthreads();
            BoxWalk bw(ext);
            bool interior = true;
#pragma unroll
            for (int a = 0; a < 3; ++a)
                interior = interior && lo[a] >= 0 && lo[a] + ext[a] <= V.n[a];
            if (interior) {
                // every entry is a voxel of the volume: no clamping, and the
                // gradient offset steps with the walk
                BoxAddr ba(bw, lo, sy, sz);
                int i = threadIdx.x;
                // four entries' LDS reads in flight before the first is tested
                for (; i + 3 * kBlock < n_win; i += 4 * kBlock) {
                    int val[4];
                    uint32_t at[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        val[u] = win[i + u * kBlock];
                        at[u] = ba.addr;
                        int cx, cy;
                        bw.next(cx, cy);
                        ba.next(cx, cy);
                    }
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        if (val[u] != 0) {
                            win[i + u * kBlock] = 0;
                            unsafeAtomicAdd(grad + at[u], (float)val[u] * ci);
                        }
                    }
                }
                for (; i < n_win; i += kBlock) {
                    const int val = win[i];
                    if (val != 0) {
                        win[i] = 0;
                        unsafeAtomicAdd(grad + ba.addr, (float)val * ci);
                    }
                    int cx, cy;
                    bw.next(cx, cy);
                    ba.next(cx, cy);
                }
            }
            if (!interior) {
                // entries at -1 or n stand for the clamped edge voxel (clamp to
                // edge) or for nothing (zero padding)
                auto flush_entry = [&](int i, int val, int x, int y, int z) {
                    if (val == 0) return;
                    win[i] = 0;
                    int g[3] = {lo[0] + x, lo[1] + y, lo[2] + z};
                    bool inside = true;
#pragma unroll
                    for (int a = 0; a < 3; ++a) {
                        inside = inside && g[a] >= 0 && g[a] <= V.n[a] - 1;
                        g[a] = clampi(g[a], 0, V.n[a] - 1);
                    }
                    if (ZP && !inside) return;
                    unsafeAtomicAdd(grad + (uint32_t)g[2] * sz + (uint32_t)g[1] * sy +
                                        (uint32_t)g[0],
                                    (float)val * ci);
                };
                int i = threadIdx.x;
                // near/far: boxes reach into the padding and take this path
                // most of the time, so four entries' LDS reads are put in
                // flight before the first is tested (box clip keeps the plain
                // loop: measured faster on dense views)
                for (; ZP && i + 3 * kBlock < n_win; i += 4 * kBlock) {
                    int val[4], x[4], y[4], z[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        val[u] = win[i + u * kBlock];
                        x[u] = bw.x;
                        y[u] = bw.y;
                        z[u] = bw.z;
                        bw.next();
                    }
#pragma unroll
                    for (int u = 0; u < 4; ++u) flush_entry(i + u * kBlock, val[u], x[u], y[u], z[u]);
                }
                for (; i < n_win; i += kBlock, bw.next()) flush_entry(i, win[i], bw.x, bw.y, bw.z);
            }
            __syncthreads();
        } else if (active) {
            const int ka = max(k0, k_lo), kb = min(k0 + S, k_hi);
            int64_t qx = R.q0[0] + (int64_t)ka * R.dq[0];
            int64_t qy = R.q0[1] + (int64_t)ka * R.dq[1];
            int64_t qz = R.q0[2] + (int64_t)ka * R.dq[2];
            for (int k = ka; k < kb; ++k) {
                Cell C;
                float m[6];
                cell_of(V, qx, qy, qz, C);
                if constexpr (ZP) pad_mask(V, qx, qy, qz, m);
                float c = yd;
                if constexpr (ALPHA) c = coef.next_at(V, Vc, qx, qy, qz);
                qx += R.dq[0]; qy += R.dq[1]; qz += R.dq[2];
                scatter_sample_global<ZP>(grad, sy, sz, C, c, m);
            }
        }
        k0 += S;
        // a chunk that left room in the window: try a longer one next
        if (vol_cells * 2 <= win_cap) S *= 2;
    }
}

__global__ __launch_bounds__(256) void drr_fill_kernel(float* __restrict__ p, size_t n, float v)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = v;
}

// ----------------------------------------------------------------- launchers

static void tile_grid(int n_pairs, int H, int W, int side, int& tiles_x, int& tiles_per_view,
                      int& n_tiles)
{
    tiles_x = (W + side - 1) / side;
    const int tiles_y = (H + side - 1) / side;
    tiles_per_view = tiles_x * tiles_y;
    n_tiles = tiles_per_view * n_pairs;
}

static Batch make_batch(const LaunchArgs& a, const RenderPlan* plan, size_t in_volume_bytes)
{
    Batch b;
    b.src_stride = plan ? (uint64_t)plan->per_volume_bytes : (uint64_t)in_volume_bytes;
    b.grad_stride = (uint32_t)((size_t)a.V.n[0] * a.V.n[1] * a.V.n[2]);
    b.C = a.C;
    b.vpv = a.n_views / a.n_volumes;
    b.f = a.f;
    b.margin = a.margin;
    return b;
}

template <typename T, Layout L, int MODE, int SPLIT, int CLIP>
static void launch_march(const LaunchArgs& a, const T* src, uint32_t src_bytes, const Batch& b,
                         float* out, float* s_out, hipStream_t stream)
{
    int tiles_x, tiles_per_view, n_tiles;
    tile_grid(a.n_views * a.C, a.H, a.W, march_tile_side<SPLIT>(), tiles_x, tiles_per_view,
              n_tiles);
    hipLaunchKernelGGL((drr_march_kernel<T, L, MODE, SPLIT, CLIP>), dim3(n_tiles), dim3(kBlock), 0,
                       stream, src, src_bytes, a.V, a.K, a.poses, a.H, a.W, a.N, tiles_x,
                       tiles_per_view, b, out, s_out);
}

// Lanes per ray: one, unless the launch has too few rays to give every SIMD of
// the chip a wave (65536 lanes).
static int march_split(long long n_rays, int N)
{
    const long long target = 65536;
    if (n_rays >= target || N < 8) return 1;
    if (n_rays * 4 >= target || N < 32) return 4;
    if (n_rays * 16 >= target || N < 128) return 16;
    return 64;
}

template <typename T, Layout L, int MODE, int CLIP>
static void launch_march_split(const LaunchArgs& a, const T* src, uint32_t src_bytes,
                               const Batch& b, float* out, float* s_out, hipStream_t stream)
{
    if constexpr (MODE == kAlpha) {
        launch_march<T, L, MODE, 1, CLIP>(a, src, src_bytes, b, out, s_out, stream);
    } else {
        switch (march_split((long long)a.n_views * a.C * a.H * a.W, a.N)) {
        case 1: launch_march<T, L, MODE, 1, CLIP>(a, src, src_bytes, b, out, s_out, stream); break;
        case 4: launch_march<T, L, MODE, 4, CLIP>(a, src, src_bytes, b, out, s_out, stream); break;
        case 16: launch_march<T, L, MODE, 16, CLIP>(a, src, src_bytes, b, out, s_out, stream); break;
        default: launch_march<T, L, MODE, 64, CLIP>(a, src, src_bytes, b, out, s_out, stream); break;
        }
    }
}

template <typename T, Layout L, int CLIP>
static void launch_march_mode(const LaunchArgs& a, const T* src, uint32_t src_bytes,
                              const Batch& b, float* out, float* s_out, hipStream_t stream)
{
    if (a.mode == kBeerLambert)
        launch_march_split<T, L, kBeerLambert, CLIP>(a, src, src_bytes, b, out, s_out, stream);
    else if (a.mode == kLineIntegral)
        launch_march_split<T, L, kLineIntegral, CLIP>(a, src, src_bytes, b, out, s_out, stream);
    else
        launch_march_split<T, L, kAlpha, CLIP>(a, src, src_bytes, b, out, s_out, stream);
}

static int grid_blocks(long long n, int cap)
{
    const long long b = (n + 255) / 256;
    return (int)(b < cap ? (b > 0 ? b : 1) : cap);
}

// Corner cells of all n_volumes * C channel-volumes into `cells` (stride
// per_volume_bytes), zero-padded in the near/far mode, mapped by the transfer
// function when there is one (then fp32).
template <typename Tin>
static hipError_t launch_cells_typed(const LaunchArgs& a, const RenderPlan& p, const Tin* vol,
                                     void* cells, hipStream_t stream)
{
    const long long n_cells = (long long)(a.V.n[0] + 1) * (a.V.n[1] + 1) * (a.V.n[2] + 1);
    const dim3 grid(grid_blocks(n_cells, 16384), a.n_volumes * a.C);
    const size_t in_stride = (size_t)a.V.n[0] * a.V.n[1] * a.V.n[2];
    const bool zp = a.clip == kClipNearFar;
    if (p.mapped) {
        const size_t out_stride = p.per_volume_bytes / sizeof(float);
        float* c = static_cast<float*>(cells);
        if (zp)
            hipLaunchKernelGGL((drr_cells_kernel<Tin, float, true, true>), grid, dim3(256), 0,
                               stream, vol, a.V.n[0], a.V.n[1], a.V.n[2], in_stride, c,
                               out_stride, a.C, a.tf);
        else
            hipLaunchKernelGGL((drr_cells_kernel<Tin, float, false, true>), grid, dim3(256), 0,
                               stream, vol, a.V.n[0], a.V.n[1], a.V.n[2], in_stride, c,
                               out_stride, a.C, a.tf);
    } else {
        const size_t out_stride = p.per_volume_bytes / sizeof(Tin);
        Tin* c = static_cast<Tin*>(cells);
        if (zp)
            hipLaunchKernelGGL((drr_cells_kernel<Tin, Tin, true, false>), grid, dim3(256), 0,
                               stream, vol, a.V.n[0], a.V.n[1], a.V.n[2], in_stride, c,
                               out_stride, a.C, a.tf);
        else
            hipLaunchKernelGGL((drr_cells_kernel<Tin, Tin, false, false>), grid, dim3(256), 0,
                               stream, vol, a.V.n[0], a.V.n[1], a.V.n[2], in_stride, c,
                               out_stride, a.C, a.tf);
    }
    return hipGetLastError();
}

// Z-pair copies of all n_volumes * C channel-volumes into `pairs` (stride
// per_volume_bytes), mapped by the transfer function when there is one (then fp32).
template <typename Tin>
static hipError_t launch_zpair_typed(const LaunchArgs& a, const RenderPlan& p, const Tin* vol,
                                     void* pairs, hipStream_t stream)
{
    if (p.padded) {
        const long long np = (long long)(a.V.n[0] + 2) * (a.V.n[1] + 2) * (a.V.n[2] + 1);
        const dim3 grid(grid_blocks(np, 16384), a.n_volumes * a.C);
        const size_t in_stride = (size_t)a.V.n[0] * a.V.n[1] * a.V.n[2];
        if (p.mapped)
            hipLaunchKernelGGL((drr_zpair_pad_kernel<Tin, float, true>), grid, dim3(256), 0,
                               stream, vol, a.V.n[0], a.V.n[1], a.V.n[2], in_stride,
                               static_cast<float*>(pairs), p.per_volume_bytes / sizeof(float),
                               a.C, a.tf);
        else
            hipLaunchKernelGGL((drr_zpair_pad_kernel<Tin, Tin, false>), grid, dim3(256), 0,
                               stream, vol, a.V.n[0], a.V.n[1], a.V.n[2], in_stride,
                               static_cast<Tin*>(pairs), p.per_volume_bytes / sizeof(Tin), a.C,
                               a.tf);
        return hipGetLastError();
    }
    const long long slice = (long long)a.V.n[0] * a.V.n[1];
    const dim3 grid((unsigned)((slice + 255) / 256), a.n_volumes * a.C,
                    (unsigned)((a.V.n[2] - 1 + kZRun - 1) / kZRun));
    const size_t in_stride = (size_t)a.V.n[0] * a.V.n[1] * a.V.n[2];
    if (p.mapped)
        hipLaunchKernelGGL((drr_zpair_kernel<Tin, float, true>), grid, dim3(256), 0, stream, vol,
                           a.V.n[0], a.V.n[1], a.V.n[2], in_stride, static_cast<float*>(pairs),
                           p.per_volume_bytes / sizeof(float), a.C, a.tf);
    else
        hipLaunchKernelGGL((drr_zpair_kernel<Tin, Tin, false>), grid, dim3(256), 0, stream, vol,
                           a.V.n[0], a.V.n[1], a.V.n[2], in_stride, static_cast<Tin*>(pairs),
                           p.per_volume_bytes / sizeof(Tin), a.C, a.tf);
    return hipGetLastError();
}

template <typename Tin>
static hipError_t launch_transfer_typed(const LaunchArgs& a, const RenderPlan& p, const Tin* vol,
                                        float* mu, hipStream_t stream)
{
    const size_t n_vox = (size_t)a.V.n[0] * a.V.n[1] * a.V.n[2];
    const dim3 grid(grid_blocks((long long)n_vox, 4096), a.n_volumes * a.C);
    hipLaunchKernelGGL((drr_transfer_kernel<Tin>), grid, dim3(256), 0, stream, vol, n_vox, n_vox,
                       mu, p.per_volume_bytes / sizeof(float), a.C, a.tf);
    return hipGetLastError();
}

hipError_t launch_read_copy(const LaunchArgs& a, const RenderPlan& p, const void* vol, int dtype,
                            void* workspace, hipStream_t stream)
{
    if (p.zpair) {
        if (dtype == 0)
            return launch_zpair_typed<float>(a, p, static_cast<const float*>(vol), workspace,
                                             stream);
        return launch_zpair_typed<uint16_t>(a, p, static_cast<const uint16_t*>(vol), workspace,
                                            stream);
    }
    if (p.cells) {
        if (dtype == 0)
            return launch_cells_typed<float>(a, p, static_cast<const float*>(vol), workspace,
                                             stream);
        return launch_cells_typed<uint16_t>(a, p, static_cast<const uint16_t*>(vol), workspace,
                                            stream);
    }
    if (p.mapped) {
        float* mu = static_cast<float*>(workspace);
        if (dtype == 0)
            return launch_transfer_typed<float>(a, p, static_cast<const float*>(vol), mu, stream);
        return launch_transfer_typed<uint16_t>(a, p, static_cast<const uint16_t*>(vol), mu,
                                               stream);
    }
    return hipSuccess;
}

template <typename Tin, int MODE>
static void launch_staged_mode(const LaunchArgs& a, const Tin* vol, const Batch& b, float* out,
                               float* s_out, hipStream_t stream)
{
    int tiles_x, tiles_per_view, n_tiles;
    tile_grid(a.n_views * a.C, a.H, a.W, kTile, tiles_x, tiles_per_view, n_tiles);
    const uint32_t bytes = (uint32_t)((size_t)a.V.n[0] * a.V.n[1] * a.V.n[2] * sizeof(Tin));
    if (a.has_tf)
        hipLaunchKernelGGL((drr_march_staged_kernel<Tin, MODE, true>), dim3(n_tiles), dim3(kBlock),
                           0, stream, vol, bytes, a.V, a.K, a.poses, a.H, a.W, a.N, tiles_x,
                           tiles_per_view, b, a.tf, out, s_out);
    else
        hipLaunchKernelGGL((drr_march_staged_kernel<Tin, MODE, false>), dim3(n_tiles),
                           dim3(kBlock), 0, stream, vol, bytes, a.V, a.K, a.poses, a.H, a.W, a.N,
                           tiles_x, tiles_per_view, b, a.tf, out, s_out);
}

template <typename Tin>
static hipError_t forward_typed(const LaunchArgs& a, const RenderPlan& p, const Tin* vol,
                                void* workspace, float* out, float* s_out, hipStream_t stream,
                                bool reuse_copy)
{
    const Batch b = make_batch(a, &p, 0);
    if (p.staged) {
        if (a.mode == kBeerLambert)
            launch_staged_mode<Tin, kBeerLambert>(a, vol, b, out, s_out, stream);
        else if (a.mode == kLineIntegral)
            launch_staged_mode<Tin, kLineIntegral>(a, vol, b, out, s_out, stream);
        else
            launch_staged_mode<Tin, kAlpha>(a, vol, b, out, s_out, stream);
        return hipGetLastError();
    }
    const uint32_t bytes = p.cells ? a.V.cell_total_bytes : a.V.total_bytes;
    if (p.zpair) {
        if (!reuse_copy) {
            hipError_t e = launch_zpair_typed<Tin>(a, p, vol, workspace, stream);
            if (e != hipSuccess) return e;
        }
        const float* mu = static_cast<const float*>(workspace);
        const Tin* pr = static_cast<const Tin*>(workspace);
        if (p.padded) {
            if (p.mapped)
                launch_march_mode<float, Layout::ZPair, kClipNearFar>(a, mu, bytes, b, out, s_out,
                                                                      stream);
            else
                launch_march_mode<Tin, Layout::ZPair, kClipNearFar>(a, pr, bytes, b, out, s_out,
                                                                    stream);
        } else {
            if (p.mapped)
                launch_march_mode<float, Layout::ZPair, kClipBox>(a, mu, bytes, b, out, s_out,
                                                                  stream);
            else
                launch_march_mode<Tin, Layout::ZPair, kClipBox>(a, pr, bytes, b, out, s_out,
                                                                stream);
        }
        return hipGetLastError();
    }
    if (p.cells) {
        if (!reuse_copy) {
            hipError_t e = launch_cells_typed<Tin>(a, p, vol, workspace, stream);
            if (e != hipSuccess) return e;
        }
        if (p.mapped) {
            const float* c = static_cast<const float*>(workspace);
            if (a.clip == kClipNearFar)
                launch_march_mode<float, Layout::Cell, kClipNearFar>(a, c, bytes, b, out, s_out, stream);
            else
                launch_march_mode<float, Layout::Cell, kClipBox>(a, c, bytes, b, out, s_out, stream);
        } else {
            const Tin* c = static_cast<const Tin*>(workspace);
            if (a.clip == kClipNearFar)
                launch_march_mode<Tin, Layout::Cell, kClipNearFar>(a, c, bytes, b, out, s_out, stream);
            else
                launch_march_mode<Tin, Layout::Cell, kClipBox>(a, c, bytes, b, out, s_out, stream);
        }
        return hipGetLastError();
    }
    // linear reads: the caller's volume, or its mapped fp32 copy
    if (p.mapped) {
        float* mu = static_cast<float*>(workspace);
        if (!reuse_copy) {
            hipError_t e = launch_transfer_typed<Tin>(a, p, vol, mu, stream);
            if (e != hipSuccess) return e;
        }
        if (a.V.n[0] >= 2)
            launch_march_mode<float, Layout::Pair, kClipBox>(a, mu, bytes, b, out, s_out, stream);
        else
            launch_march_mode<float, Layout::Single, kClipBox>(a, mu, bytes, b, out, s_out, stream);
    } else if (a.V.n[0] >= 2) {
        launch_march_mode<Tin, Layout::Pair, kClipBox>(a, vol, bytes, b, out, s_out, stream);
    } else {
        launch_march_mode<Tin, Layout::Single, kClipBox>(a, vol, bytes, b, out, s_out, stream);
    }
    return hipGetLastError();
}

hipError_t launch_forward(const LaunchArgs& a, const RenderPlan& plan, const void* vol, int dtype,
                          void* workspace, float* out, float* s_out, hipStream_t stream,
                          bool reuse_copy)
{
    if ((long long)a.n_views * a.C * a.H * a.W == 0) return hipSuccess;
    if (dtype == 0)
        return forward_typed<float>(a, plan, static_cast<const float*>(vol), workspace, out, s_out,
                                    stream, reuse_copy);
    return forward_typed<uint16_t>(a, plan, static_cast<const uint16_t*>(vol), workspace, out,
                                   s_out, stream, reuse_copy);
}

hipError_t launch_fill(float* p, size_t n, hipStream_t stream)
{
    if (n == 0) return hipSuccess;
    const int blocks = (int)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
    hipLaunchKernelGGL(drr_fill_kernel, dim3(blocks), dim3(256), 0, stream, p, n, 0.0f);
    return hipGetLastError();
}

template <int MODE, typename T, bool ZPAIR = false>
static void launch_scatter(const LaunchArgs& a, const Batch& b, const float* grad_out,
                           const float* s_in, const float* out_in, const T* vol,
                           uint32_t vol_bytes, float* grad, int tiles_x, int tiles_per_view,
                           int n_tiles, hipStream_t stream, uint32_t copy_row = 0,
                           uint32_t copy_slice = 0, const int* vbound = nullptr)
{
    const double cells = (double)(a.V.n[0] + 1) * (a.V.n[1] + 1) * (a.V.n[2] + 1);
    const int cap = window_cap((double)a.H * a.W * a.N / cells);
    const size_t lds = (size_t)cap * sizeof(int);
    if (a.clip == kClipNearFar)
        hipLaunchKernelGGL((drr_scatter_kernel<MODE, kClipNearFar, T, ZPAIR>), dim3(n_tiles),
                           dim3(kBlock), lds, stream, a.V, a.K, a.poses, a.H, a.W, a.N, tiles_x,
                           tiles_per_view, b, grad_out, s_in, out_in, vol, vol_bytes, copy_row,
                           copy_slice, vbound, grad, cap);
    else
        hipLaunchKernelGGL((drr_scatter_kernel<MODE, kClipBox, T, ZPAIR>), dim3(n_tiles),
                           dim3(kBlock), lds, stream, a.V, a.K, a.poses, a.H, a.W, a.N, tiles_x,
                           tiles_per_view, b, grad_out, s_in, out_in, vol, vol_bytes, copy_row,
                           copy_slice, vbound, grad, cap);
}

// Value bounds of a read copy (n_elem values of type T every `stride` values per
// channel-volume) into `vbound` (two ints per channel-volume), zeroed first.
template <typename T>
static hipError_t launch_value_bound(const LaunchArgs& a, const T* src, size_t n_elem,
                                     size_t stride, int* vbound, hipStream_t stream)
{
    const int n_cv = a.n_volumes * a.C;
    hipError_t e = launch_fill(reinterpret_cast<float*>(vbound), 2 * (size_t)n_cv, stream);
    if (e != hipSuccess) return e;
    const dim3 grid(grid_blocks((long long)n_elem, 2048), n_cv);
    hipLaunchKernelGGL((drr_value_bound_kernel<T>), grid, dim3(256), 0, stream, src, n_elem,
                       stride, vbound);
    return hipGetLastError();
}

template <typename Tin>
static hipError_t backward_typed(const LaunchArgs& a, const Tin* vol, const float* grad_out,
                                 const float* out_in, const float* s_in, float* grad,
                                 void* workspace, hipStream_t stream)
{
    const size_t n_vox = (size_t)a.V.n[0] * a.V.n[1] * a.V.n[2];
    hipError_t e;
    const BackwardRead plan = plan_backward(a.n_volumes, a.C, a.V.n[2], a.V.n[1], a.V.n[0],
                                            (int)sizeof(Tin), a.n_views, a.H, a.W, a.N, a.mode,
                                            a.clip, a.has_tf);
    if (plan.brick) {
        // the brick-owned backward writes every voxel itself
        e = launch_brick_backward(a, grad_out, s_in, grad, workspace, stream);
        if (e != hipSuccess || !a.has_tf) return e;
        const dim3 sgrid(grid_blocks((long long)n_vox, 4096), a.n_volumes * a.C);
        hipLaunchKernelGGL((drr_slope_kernel<Tin>), sgrid, dim3(256), 0, stream, vol, n_vox,
                           n_vox, grad, a.C, a.tf);
        return hipGetLastError();
    }
    e = launch_fill(grad, n_vox * (size_t)a.n_volumes * a.C, stream);
    if (e != hipSuccess) return e;
    int tiles_x, tiles_per_view, n_tiles;
    tile_grid(a.n_views * a.C, a.H, a.W, kTile, tiles_x, tiles_per_view, n_tiles);
    if (n_tiles == 0) return hipSuccess;
    if (a.mode == kAlpha) {
        const BackwardRead r = plan_backward(a.n_volumes, a.C, a.V.n[2], a.V.n[1], a.V.n[0],
                                             (int)sizeof(Tin), a.n_views, a.H, a.W, a.N, kAlpha,
                                             a.clip, a.has_tf);
        if (r.zpair) {
            // gather from a z-pair copy in the workspace (zero-padded in the
            // near/far mode, fp32 and mapped with a transfer function)
            RenderPlan p{};
            p.zpair = true;
            p.padded = r.padded;
            p.mapped = r.mapped;
            p.per_volume_bytes = r.per_volume_bytes;
            e = launch_zpair_typed<Tin>(a, p, vol, workspace, stream);
            if (e != hipSuccess) return e;
            const uint32_t eb = (uint32_t)r.read_elem, nx = (uint32_t)a.V.n[0];
            const uint32_t ny = (uint32_t)a.V.n[1], nz = (uint32_t)a.V.n[2];
            const uint32_t row = (r.padded ? nx + 2 : nx) * 2u * eb;
            const uint32_t slice = (r.padded ? ny + 2 : ny) * row;
            const uint32_t total = (r.padded ? nz + 1 : nz - 1) * slice;
            const Batch b = make_batch(a, &p, 0);
            int* vbound = reinterpret_cast<int*>(static_cast<char*>(workspace) + r.bound_offset);
            if (r.mapped) {
                const float* cp = static_cast<const float*>(workspace);
                e = launch_value_bound<float>(a, cp, total / eb, r.per_volume_bytes / eb, vbound,
                                              stream);
                if (e != hipSuccess) return e;
                launch_scatter<kAlpha, float, true>(a, b, grad_out, s_in, out_in, cp, total, grad,
                                                    tiles_x, tiles_per_view, n_tiles, stream, row,
                                                    slice, vbound);
            } else {
                const Tin* cp = static_cast<const Tin*>(workspace);
                e = launch_value_bound<Tin>(a, cp, total / eb, r.per_volume_bytes / eb, vbound,
                                            stream);
                if (e != hipSuccess) return e;
                launch_scatter<kAlpha, Tin, true>(a, b, grad_out, s_in, out_in, cp, total, grad,
                                                  tiles_x, tiles_per_view, n_tiles, stream, row,
                                                  slice, vbound);
            }
        } else if (a.has_tf) {
            // gather the mapped volumes: their fp32 copy in the workspace
            RenderPlan p{};
            p.mapped = true;
            p.per_volume_bytes = (n_vox * 4 + 255) & ~(size_t)255;
            float* mu = static_cast<float*>(workspace);
            e = launch_transfer_typed<Tin>(a, p, vol, mu, stream);
            if (e != hipSuccess) return e;
            int* vbound = reinterpret_cast<int*>(static_cast<char*>(workspace) + r.bound_offset);
            e = launch_value_bound<float>(a, mu, n_vox, p.per_volume_bytes / 4, vbound, stream);
            if (e != hipSuccess) return e;
            const Batch b = make_batch(a, &p, 0);
            launch_scatter<kAlpha, float>(a, b, grad_out, s_in, out_in, mu,
                                          (uint32_t)(n_vox * 4), grad, tiles_x, tiles_per_view,
                                          n_tiles, stream, 0, 0, vbound);
        } else {
            const Batch b = make_batch(a, nullptr, n_vox * sizeof(Tin));
            launch_scatter<kAlpha, Tin>(a, b, grad_out, s_in, out_in, vol,
                                        (uint32_t)(n_vox * sizeof(Tin)), grad, tiles_x,
                                        tiles_per_view, n_tiles, stream);
        }
    } else {
        const Batch b = make_batch(a, nullptr, 0);
        if (a.mode == kBeerLambert)
            launch_scatter<kBeerLambert, float>(a, b, grad_out, s_in, out_in, nullptr, 0, grad,
                                                tiles_x, tiles_per_view, n_tiles, stream);
        else
            launch_scatter<kLineIntegral, float>(a, b, grad_out, s_in, out_in, nullptr, 0, grad,
                                                 tiles_x, tiles_per_view, n_tiles, stream);
    }
    e = hipGetLastError();
    if (e != hipSuccess || !a.has_tf) return e;
    // dL/dx = dL/dmu tf'(x)
    const dim3 sgrid(grid_blocks((long long)n_vox, 4096), a.n_volumes * a.C);
    hipLaunchKernelGGL((drr_slope_kernel<Tin>), sgrid, dim3(256), 0, stream, vol, n_vox, n_vox,
                       grad, a.C, a.tf);
    return hipGetLastError();
}

hipError_t launch_backward(const LaunchArgs& a, const void* vol, int dtype, const float* grad_out,
                           const float* out_in, const float* s_in, float* grad, void* workspace,
                           hipStream_t stream)
{
    if (dtype == 0)
        return backward_typed<float>(a, static_cast<const float*>(vol), grad_out, out_in, s_in,
                                     grad, workspace, stream);
    return backward_typed<uint16_t>(a, static_cast<const uint16_t*>(vol), grad_out, out_in, s_in,
                                    grad, workspace, stream);
}

}  // namespace drr
