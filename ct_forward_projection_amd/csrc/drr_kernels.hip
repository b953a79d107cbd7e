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
//                       march reads when samples reuse cells enough.
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
#include "drr_window.hpp"

namespace drr {

// Corner-cell relayout: cell (i, j, k), 0 <= i <= nx etc., holds the eight
// clamped corners (x0, x1) x (y0, y1) x (z0, z1) of the trilinear cell whose
// low corner is voxel (i-1, j-1, k-1), in the CornerVals order.  One thread
// per cell; consecutive threads write consecutive cells.
template <typename T>
__global__ __launch_bounds__(256) void drr_cells_kernel(const T* __restrict__ vol, int nx, int ny,
                                                        int nz, T* __restrict__ cells)
{
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
        const T v[8] = {vol[z0 + y0 + x0], vol[z0 + y0 + x1], vol[z0 + y1 + x0], vol[z0 + y1 + x1],
                        vol[z1 + y0 + x0], vol[z1 + y0 + x1], vol[z1 + y1 + x0], vol[z1 + y1 + x1]};
        T* o = cells + (size_t)id * 8;
#pragma unroll
        for (int c = 0; c < 8; ++c) o[c] = v[c];
    }
}

// Samples a lane keeps in flight: their gathers are all issued before any is
// consumed, so each wave has 4 samples' loads outstanding.
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

// Forward DRR.  SPLIT = 1: one ray per lane (16 x 16 tiles of four 8 x 8 wave
// sub-tiles).  SPLIT > 1 (launches with few rays): SPLIT adjacent lanes share
// a ray, lane j taking samples j, j + SPLIT, ... (neighbouring lanes still
// gather neighbouring voxels), and their partial sums meet in a cross-lane
// reduction, so a 64 x 64 detector still fills the chip.  `src` is the volume
// (Pair, Single) or its corner-cell copy (Cell); `src_bytes` its size.
template <typename T, Layout L, int MODE, int SPLIT>
__global__ __launch_bounds__(kBlock) void drr_march_kernel(
    const T* __restrict__ src, uint32_t src_bytes, VolumeDesc V, Intrinsics K,
    const float* __restrict__ poses, int H, int W, int N, int tiles_x, int tiles_per_view,
    float* __restrict__ out, float* __restrict__ s_out)
{
    const int tile = xcd_contiguous_tile((int)blockIdx.x, (int)gridDim.x);
    PixelCoord px;
    int j = 0;
    if constexpr (SPLIT == 1) {
        px = tile_pixel(tile, tiles_x, tiles_per_view);
    } else {
        px = split_pixel<SPLIT>(tile, tiles_x, tiles_per_view);
        j = (int)threadIdx.x % SPLIT;
    }
    // every lane of a ray sees the same pixel, so a ray's lanes leave together
    if (px.r >= H || px.c >= W) return;

    ViewGeom G;
    view_setup(poses + 12 * px.view, K, G);
    MarchRay R;
    float s = 0.0f;
    const bool hit = ray_setup(G, V, px.r, px.c, N, R);
    if (hit) {
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc((void*)src, 0, (int)src_bytes, kBufferWord3);
        int64_t qx = R.q0[0] + (int64_t)j * R.dq[0];
        int64_t qy = R.q0[1] + (int64_t)j * R.dq[1];
        int64_t qz = R.q0[2] + (int64_t)j * R.dq[2];
        const int64_t dqx = (int64_t)SPLIT * R.dq[0], dqy = (int64_t)SPLIT * R.dq[1];
        const int64_t dqz = (int64_t)SPLIT * R.dq[2];
        const int n_mine = j < N ? (N - j + SPLIT - 1) / SPLIT : 0;
        // independent partial sums, one per in-flight sample: a shorter fp32
        // summation chain as well
        float acc[kInflight];
#pragma unroll
        for (int i = 0; i < kInflight; ++i) acc[i] = 0.0f;
        int k = 0;
        for (; k + kInflight <= n_mine; k += kInflight) {
            SampleAddr A[kInflight];
            CornerVals c[kInflight];
#pragma unroll
            for (int i = 0; i < kInflight; ++i) {
                A[i] = sample_addr<T, L>(V, qx, qy, qz);
                qx += dqx; qy += dqy; qz += dqz;
            }
#pragma unroll
            for (int i = 0; i < kInflight; ++i) gather<T, L>(rs, A[i], c[i]);
            // keep every gather of the group ahead of the first use: otherwise
            // the scheduler sinks each sample's loads to just before their use
            // and a wave never has more than one sample's loads in flight
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < kInflight; ++i) acc[i] += interpolate(A[i], c[i]);
        }
        for (; k < n_mine; ++k) {
            const SampleAddr A = sample_addr<T, L>(V, qx, qy, qz);
            qx += dqx; qy += dqy; qz += dqz;
            CornerVals c;
            gather<T, L>(rs, A, c);
            acc[0] += interpolate(A, c);
        }
#pragma unroll
        for (int i = 0; i < kInflight; ++i) s += acc[i];
    }
    if constexpr (SPLIT > 1) {
        // all SPLIT lanes of this ray are here (hit or miss alike)
#pragma unroll
        for (int off = SPLIT / 2; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
        if (j != 0) return;
    }
    if (hit) s *= R.dz;
    const size_t o = ((size_t)px.view * H + px.r) * W + px.c;
    out[o] = (MODE == kBeerLambert) ? -expm1f(-s) : s;
    if (s_out) s_out[o] = s;
}

// Trilinear weights of one sample, scaled by yd = y dz: w[c] for corner c
// (bit 0 = x1, bit 1 = y1, bit 2 = z1).
__device__ inline void corner_weights(const Cell& C, float yd, float w[8])
{
    const float wz1 = yd * C.fz, wz0 = yd * (1.0f - C.fz);
    const float w11 = wz1 * C.fy, w10 = wz1 * (1.0f - C.fy);
    const float w01 = wz0 * C.fy, w00 = wz0 * (1.0f - C.fy);
    const float fx1 = C.fx, fx0 = 1.0f - C.fx;
    w[0] = w00 * fx0;
    w[1] = w00 * fx1;
    w[2] = w01 * fx0;
    w[3] = w01 * fx1;
    w[4] = w10 * fx0;
    w[5] = w10 * fx1;
    w[6] = w11 * fx0;
    w[7] = w11 * fx1;
}

__device__ inline void scatter_sample_global(float* __restrict__ grad, uint32_t sy, uint32_t sz,
                                             const Cell& C, float yd)
{
    float w[8];
    corner_weights(C, yd, w);
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

// Add the eight (scaled) weights of one cell to the LDS window.
__device__ inline void window_add(int* win, const Cell& C, const int lo[3], int wy, int wz,
                                  const float w[8])
{
    const int x0 = C.x0 - lo[0], x1 = C.x1 - lo[0];
    // window extents are below 2^13, so 24-bit multiplies are exact (full rate)
    const int y0 = __mul24(C.y0 - lo[1], wy), y1 = __mul24(C.y1 - lo[1], wy);
    const int z0 = __mul24(C.z0 - lo[2], wz), z1 = __mul24(C.z1 - lo[2], wz);
    atomicAdd(&win[z0 + y0 + x0], __float2int_rn(w[0]));
    atomicAdd(&win[z0 + y0 + x1], __float2int_rn(w[1]));
    atomicAdd(&win[z0 + y1 + x0], __float2int_rn(w[2]));
    atomicAdd(&win[z0 + y1 + x1], __float2int_rn(w[3]));
    atomicAdd(&win[z1 + y0 + x0], __float2int_rn(w[4]));
    atomicAdd(&win[z1 + y0 + x1], __float2int_rn(w[5]));
    atomicAdd(&win[z1 + y1 + x0], __float2int_rn(w[6]));
    atomicAdd(&win[z1 + y1 + x1], __float2int_rn(w[7]));
}

__device__ inline bool same_cell(const Cell& a, const Cell& b)
{
    return a.x0 == b.x0 && a.x1 == b.x1 && a.y0 == b.y0 && a.y1 == b.y1 && a.z0 == b.z0 &&
           a.z1 == b.z1;
}

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
// one sample puts at most |y dz| on any voxel and a ray has at most
// c = min(N, floor(2 / |dq|_inf) + 1) samples inside a voxel's 2 x 2 x 2
// support, so an entry never exceeds B = sum over the tile's rays of
// |y dz| c, and 2^e B <= 2^30.  (|y dz| c is about |y| times the ray's
// length inside that support, so B stays small even for short chords.)  Each
// rounding adds at most 1/2 and an entry receives at most Cs = sum of c
// roundings, which must stay below 2^31 as well.  A tile whose weights are not
// finite or whose Cs is too large, or a chunk whose box does not fit the window
// even for one sample, uses global float atomics directly.
template <int MODE>
__global__ __launch_bounds__(kBlock) void drr_scatter_kernel(
    VolumeDesc V, Intrinsics K, const float* __restrict__ poses, int H, int W, int N,
    int tiles_x, int tiles_per_view, const float* __restrict__ grad_out,
    const float* __restrict__ s_in, float* __restrict__ grad)
{
    __shared__ int win[kWinCap];
    __shared__ int red[(kBlock / 64) * 6];
    __shared__ int box[6];

    const int tile = xcd_contiguous_tile((int)blockIdx.x, (int)gridDim.x);
    const PixelCoord px = scatter_pixel(tile, tiles_x, tiles_per_view);
    bool active = px.r < H && px.c < W;
    MarchRay R;
    float yd = 0.0f;
    if (active) {
        ViewGeom G;
        view_setup(poses + 12 * px.view, K, G);
        active = ray_setup(G, V, px.r, px.c, N, R);
        if (active) {
            const size_t o = ((size_t)px.view * H + px.r) * W + px.c;
            float y = grad_out[o];
            if (MODE == kBeerLambert) y *= expf(-s_in[o]);
            yd = y * R.dz;
            active = yd != 0.0f;
        }
    }
    // element strides of the gradient volume
    const uint32_t sy = (uint32_t)V.n[0], sz = (uint32_t)V.n[0] * (uint32_t)V.n[1];

    // fixed-point scale of this tile
    float B = 0.0f, Cs = 0.0f;
    if (active) {
        const double dq_inf = fmax(fmax(fabs((double)R.dq[0]), fabs((double)R.dq[1])),
                                   fabs((double)R.dq[2])) * 2.3283064365386963e-10;
        const double c = fmin((double)N, floor(2.0 / dq_inf) + 1.0);
        B = (float)(fabs((double)yd) * c);
        Cs = (float)c;
    }
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
        long long vol;
        for (;;) {
            int v[6] = {INT_MAX, INT_MAX, INT_MAX, INT_MAX, INT_MAX, INT_MAX};
            if (active) {
#pragma unroll
                for (int a = 0; a < 3; ++a) {
                    const int64_t qa = R.q0[a] + (int64_t)k0 * R.dq[a];
                    const int64_t qb = R.q0[a] + (int64_t)(k0 + S - 1) * R.dq[a];
                    const int fa = fixed_floor(qa), fb = fixed_floor(qb);
                    v[a] = clampi(min(fa, fb), 0, V.n[a] - 1);
                    v[3 + a] = -clampi(max(fa, fb) + 1, 0, V.n[a] - 1);
                }
            }
            block_min6(v, red, box);
            vol = 1;
#pragma unroll
            for (int a = 0; a < 3; ++a) {
                lo[a] = box[a];
                ext[a] = max(-box[3 + a] - box[a] + 1, 1);
                vol *= ext[a];
            }
            if (!fixed_ok || vol <= kWinCap || S == 1) break;
            S = max(1, S >> 1);
        }
        if (fixed_ok && vol <= kWinCap) {
            const int n_win = (int)vol;
            for (int i = threadIdx.x; i < n_win; i += kBlock) win[i] = 0;
            __syncthreads();
            if (active) {
                const int wy = ext[0], wz = ext[0] * ext[1];
                int64_t qx = R.q0[0] + (int64_t)k0 * R.dq[0];
                int64_t qy = R.q0[1] + (int64_t)k0 * R.dq[1];
                int64_t qz = R.q0[2] + (int64_t)k0 * R.dq[2];
                Cell P;
                float acc[8];
                cell_of(V, qx, qy, qz, P);
                corner_weights(P, ys, acc);
                qx += R.dq[0]; qy += R.dq[1]; qz += R.dq[2];
                for (int k = k0 + 1; k < k0 + S; ++k) {
                    Cell C;
                    cell_of(V, qx, qy, qz, C);
                    qx += R.dq[0]; qy += R.dq[1]; qz += R.dq[2];
                    float w[8];
                    corner_weights(C, ys, w);
                    if (same_cell(C, P)) {
#pragma unroll
                        for (int i = 0; i < 8; ++i) acc[i] += w[i];
                    } else {
                        window_add(win, P, lo, wy, wz, acc);
                        P = C;
#pragma unroll
                        for (int i = 0; i < 8; ++i) acc[i] = w[i];
                    }
                }
                window_add(win, P, lo, wy, wz, acc);
            }
            __syncthreads();
            for (int i = threadIdx.x; i < n_win; i += kBlock) {
                const int val = win[i];
                if (val != 0) {
                    const int ix = i % ext[0];
                    const int rest = i / ext[0];
                    const int iy = rest % ext[1];
                    const int iz = rest / ext[1];
                    unsafeAtomicAdd(grad + (uint32_t)(lo[2] + iz) * sz +
                                        (uint32_t)(lo[1] + iy) * sy + (uint32_t)(lo[0] + ix),
                                    (float)val * inv_scale);
                }
            }
            __syncthreads();
        } else if (active) {
            int64_t qx = R.q0[0] + (int64_t)k0 * R.dq[0];
            int64_t qy = R.q0[1] + (int64_t)k0 * R.dq[1];
            int64_t qz = R.q0[2] + (int64_t)k0 * R.dq[2];
            for (int k = k0; k < k0 + S; ++k) {
                Cell C;
                cell_of(V, qx, qy, qz, C);
                qx += R.dq[0]; qy += R.dq[1]; qz += R.dq[2];
                scatter_sample_global(grad, sy, sz, C, yd);
            }
        }
        k0 += S;
        // a chunk that left room in the window: try a longer one next
        if (vol * 2 <= kWinCap) S *= 2;
    }
}

__global__ __launch_bounds__(256) void drr_fill_kernel(float* __restrict__ p, size_t n, float v)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = v;
}

// ----------------------------------------------------------------- launchers

static void tile_grid(int n_views, int H, int W, int side, int& tiles_x, int& tiles_per_view,
                      int& n_tiles)
{
    tiles_x = (W + side - 1) / side;
    const int tiles_y = (H + side - 1) / side;
    tiles_per_view = tiles_x * tiles_y;
    n_tiles = tiles_per_view * n_views;
}

template <typename T, Layout L, int SPLIT>
static void launch_march(const LaunchArgs& a, const T* src, uint32_t src_bytes, float* out,
                         float* s_out, hipStream_t stream)
{
    int tiles_x, tiles_per_view, n_tiles;
    tile_grid(a.n_views, a.H, a.W, march_tile_side<SPLIT>(), tiles_x, tiles_per_view, n_tiles);
    const dim3 grid(n_tiles), block(kBlock);
    if (a.mode == kBeerLambert)
        hipLaunchKernelGGL((drr_march_kernel<T, L, kBeerLambert, SPLIT>), grid, block, 0, stream,
                           src, src_bytes, a.V, a.K, a.poses, a.H, a.W, a.N, tiles_x,
                           tiles_per_view, out, s_out);
    else
        hipLaunchKernelGGL((drr_march_kernel<T, L, kLineIntegral, SPLIT>), grid, block, 0, stream,
                           src, src_bytes, a.V, a.K, a.poses, a.H, a.W, a.N, tiles_x,
                           tiles_per_view, out, s_out);
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

template <typename T, Layout L>
static void launch_march_split(const LaunchArgs& a, const T* src, uint32_t src_bytes, float* out,
                               float* s_out, hipStream_t stream)
{
    switch (march_split((long long)a.n_views * a.H * a.W, a.N)) {
    case 1: launch_march<T, L, 1>(a, src, src_bytes, out, s_out, stream); break;
    case 4: launch_march<T, L, 4>(a, src, src_bytes, out, s_out, stream); break;
    case 16: launch_march<T, L, 16>(a, src, src_bytes, out, s_out, stream); break;
    default: launch_march<T, L, 64>(a, src, src_bytes, out, s_out, stream); break;
    }
}

hipError_t launch_cells(const VolumeDesc& V, const void* vol, int dtype, void* cells,
                        hipStream_t stream)
{
    const long long n_cells = (long long)(V.n[0] + 1) * (V.n[1] + 1) * (V.n[2] + 1);
    const int blocks = (int)((n_cells + 255) / 256 < 16384 ? (n_cells + 255) / 256 : 16384);
    if (dtype == 0)
        hipLaunchKernelGGL((drr_cells_kernel<float>), dim3(blocks), dim3(256), 0, stream,
                           static_cast<const float*>(vol), V.n[0], V.n[1], V.n[2],
                           static_cast<float*>(cells));
    else
        hipLaunchKernelGGL((drr_cells_kernel<uint16_t>), dim3(blocks), dim3(256), 0, stream,
                           static_cast<const uint16_t*>(vol), V.n[0], V.n[1], V.n[2],
                           static_cast<uint16_t*>(cells));
    return hipGetLastError();
}

template <typename T>
static hipError_t forward_typed(const LaunchArgs& a, const T* vol, bool cells, T* cell_buf,
                               float* out, float* s_out, hipStream_t stream)
{
    if (cells) {
        const hipError_t e = launch_cells(a.V, vol, sizeof(T) == 4 ? 0 : 1, cell_buf, stream);
        if (e != hipSuccess) return e;
        launch_march_split<T, Layout::Cell>(a, cell_buf, a.V.cell_total_bytes, out, s_out, stream);
    } else if (a.V.n[0] >= 2) {
        launch_march_split<T, Layout::Pair>(a, vol, a.V.total_bytes, out, s_out, stream);
    } else {
        launch_march_split<T, Layout::Single>(a, vol, a.V.total_bytes, out, s_out, stream);
    }
    return hipGetLastError();
}

hipError_t launch_forward(const LaunchArgs& a, const void* vol, int dtype, bool cells,
                          void* workspace, float* out, float* s_out, hipStream_t stream)
{
    if ((long long)a.n_views * a.H * a.W == 0) return hipSuccess;
    if (dtype == 0)
        return forward_typed<float>(a, static_cast<const float*>(vol), cells,
                                    static_cast<float*>(workspace), out, s_out, stream);
    return forward_typed<uint16_t>(a, static_cast<const uint16_t*>(vol), cells,
                                   static_cast<uint16_t*>(workspace), out, s_out, stream);
}

hipError_t launch_fill(float* p, size_t n, hipStream_t stream)
{
    if (n == 0) return hipSuccess;
    const int blocks = (int)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
    hipLaunchKernelGGL(drr_fill_kernel, dim3(blocks), dim3(256), 0, stream, p, n, 0.0f);
    return hipGetLastError();
}

hipError_t launch_backward(const LaunchArgs& a, const float* grad_out, const float* s_in,
                           float* grad, hipStream_t stream)
{
    hipError_t e = launch_fill(grad, (size_t)a.V.n[0] * a.V.n[1] * a.V.n[2], stream);
    if (e != hipSuccess) return e;
    int tiles_x, tiles_per_view, n_tiles;
    tile_grid(a.n_views, a.H, a.W, kTile, tiles_x, tiles_per_view, n_tiles);
    if (n_tiles == 0) return hipSuccess;
    const dim3 grid(n_tiles), block(kBlock);
    if (a.mode == kBeerLambert)
        hipLaunchKernelGGL((drr_scatter_kernel<kBeerLambert>), grid, block, 0, stream, a.V, a.K,
                           a.poses, a.H, a.W, a.N, tiles_x, tiles_per_view, grad_out, s_in, grad);
    else
        hipLaunchKernelGGL((drr_scatter_kernel<kLineIntegral>), grid, block, 0, stream, a.V, a.K,
                           a.poses, a.H, a.W, a.N, tiles_x, tiles_per_view, grad_out, s_in, grad);
    return hipGetLastError();
}

}  // namespace drr
