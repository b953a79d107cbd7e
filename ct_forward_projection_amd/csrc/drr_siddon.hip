// drr_siddon.hip -- the cell-constant (Siddon) projector pair.
//
// diffct 2.1.0, "Why diffct" feature list: project() and backproject() form an
// exact adjoint pair for the cell-constant Siddon model.  Each voxel is a
// constant box; a ray's line integral is sum_v mu_v l_v with l_v the exact length
// of the clipped ray inside voxel v.  Cameras, box clip and output stage are the
// trilinear path's (nanodrr introduction: Hartley-Zisserman pinhole;
// flashdrr.rendering VolumeRaycaster.__init__: Beer-Lambert 1 - exp(-s)).
//
// Traversal: a 3-D digital differential analyser.  The walk starts in the voxel
// that holds the entry point and moves, one axis at a time, to the nearest of
// the three next plane crossings.  Every crossing is evaluated directly from its
// plane index p, t = p k_a + b_a with k_a = s_a / d_a and
// b_a = (-E_a/2 - C_a) / d_a, in fp64 and never accumulated; the box faces are
// planes 0 and n_a of the same expression, so the walk ends exactly at t1.  A
// piece's length is rounded to fp32 once.
//
//   drr_siddon_march_kernel    forward: s = sum mu_v l_v, eight (or twelve)
//                              pieces' loads in flight per lane, fp32
//                              accumulation
//   drr_siddon_scatter_kernel  backward: y l_v into the fp32 gradient, the
//                              rays of a tile walked chunk by chunk into an LDS
//                              window of fixed-point integer sums
#include <limits.h>

#include "drr_device.hpp"
#include "drr_internal.hpp"
#include "drr_sample.hpp"
#include "drr_siddon.hpp"
#include "drr_window.hpp"

namespace drr {

// Forward.  Pieces are produced eight at a time (walk only), then their eight
// loads are issued together, then accumulated into four partial sums.  Loads of
// pieces past the end of the walk stay memory-safe (a raw buffer load outside
// the buffer's range returns 0), and pieces of zero length add an explicit 0,
// so no voxel the ray does not cross (a NaN, say) leaks into the sum.
template <typename T, int MODE, int NG>
__global__ __launch_bounds__(kBlock) void drr_siddon_march_kernel(
    const T* __restrict__ src, uint32_t src_bytes, VolumeDesc V, Intrinsics K,
    const float* __restrict__ poses, int H, int W, int tiles_x, int tiles_per_view,
    float* __restrict__ out, float* __restrict__ s_out)
{
    const int tile = xcd_contiguous_tile((int)blockIdx.x, (int)gridDim.x);
    const PixelCoord px = tile_pixel(tile, tiles_x, tiles_per_view);
    if (px.r >= H || px.c >= W) return;
    ViewGeom G;
    view_setup(poses + 12 * px.view, K, G);
    SiddonRay S;
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (siddon_setup(G, V, px.r, px.c, S)) {
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc((void*)src, 0, (int)src_bytes, kBufferWord3);
        const int ex = (int)sizeof(T), ey = (int)V.row_bytes, ez = (int)V.slice_bytes;
        uint32_t off = (uint32_t)S.i[0] * (uint32_t)ex + (uint32_t)S.i[1] * (uint32_t)ey +
                       (uint32_t)S.i[2] * (uint32_t)ez;
        const int dx = S.step[0] * ex, dy = S.step[1] * ey, dz = S.step[2] * ez;
        double tc = S.t0;
        int guard = V.n[0] + V.n[1] + V.n[2] + 3;
        bool live = true;
        constexpr int kGroup = NG;  // pieces' loads in flight per lane
        while (live) {
            uint32_t o[kGroup];
            float l[kGroup];
#pragma unroll
            for (int g = 0; g < kGroup; ++g) {
                const NextAxis m = next_axis(S);
                const double te = fmin(m.t, S.t1);
                const float len = live ? (float)fmax(te - tc, 0.0) : 0.0f;
                l[g] = len;
                o[g] = off;
                tc = fmax(tc, te);
                live = live && m.t < S.t1 && --guard > 0;
                if (live) {
                    live = advance(S, m, V);
                    off += (uint32_t)(m.x ? dx : (m.y ? dy : dz));
                }
            }
            float mu[kGroup];
#pragma unroll
            for (int g = 0; g < kGroup; ++g) mu[g] = load_one<T>(rs, o[g]);
#pragma unroll
            for (int g = 0; g < kGroup; ++g)
                acc[g & 3] = fmaf(l[g] > 0.0f ? mu[g] : 0.0f, l[g], acc[g & 3]);
        }
    }
    const float s = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    const size_t o = ((size_t)px.view * H + px.r) * W + px.c;
    out[o] = MODE == kBeerLambert ? -expm1f(-s) : s;
    if (s_out) s_out[o] = s;
}

// Backward (matched adjoint of the forward above): every piece adds y l_v to
// its voxel, y = g exp(-s) (Beer-Lambert) or g (line integral).  This tile
// form serves views dense against the voxels; sparse ones take the
// brick-owned backward (drr_brick.hip).
//
// The tile's rays are walked in M common chunks of their own ranges (chunk k of
// a ray covers t0 + [k, k + S) (t1 - t0) / M).  For each chunk the workgroup
// reduces the voxel box its rays' chunk segments span (their end points, one
// voxel of margin each side for rounding); if the box fits the LDS window the
// pieces add into it as fixed-point integers and the window is flushed with one
// global float atomic per touched voxel, as in the trilinear scatter.  A voxel
// receives at most one piece per ray per chunk, no longer than the voxel
// diagonal D, so with B = sum over the tile of |y| D a scale 2^e with
// 2^e B <= 2^30 keeps every entry in range (plus at most 256 roundings of 1/2).
// A piece whose voxel falls outside the box, a tile whose weights are not
// finite, or a chunk whose box does not fit even for one step, uses global
// atomics directly.
template <int MODE>
__global__ __launch_bounds__(kBlock) void drr_siddon_scatter_kernel(
    VolumeDesc V, Intrinsics K, const float* __restrict__ poses, int H, int W, int M,
    int tiles_x, int tiles_per_view, const float* __restrict__ grad_out,
    const float* __restrict__ s_in, float* __restrict__ grad, int win_cap)
{
    extern __shared__ int win[];                  // win_cap entries (dynamic LDS)
    __shared__ int red[(kBlock / 64) * 6];
    __shared__ int box[6];

    const int tile = xcd_contiguous_tile((int)blockIdx.x, (int)gridDim.x);
    const PixelCoord px = scatter_pixel(tile, tiles_x, tiles_per_view);
    bool live = px.r < H && px.c < W;
    SiddonRay S;
    float y = 0.0f;
    if (live) {
        ViewGeom G;
        view_setup(poses + 12 * px.view, K, G);
        live = siddon_setup(G, V, px.r, px.c, S);
        if (live) {
            const size_t o = ((size_t)px.view * H + px.r) * W + px.c;
            y = grad_out[o];
            if (MODE == kBeerLambert) y *= expf(-s_in[o]);
            live = y != 0.0f;
        }
    }
    const uint32_t sy = (uint32_t)V.n[0], sz = (uint32_t)V.n[0] * (uint32_t)V.n[1];

    const double diag = sqrt(V.s[0] * V.s[0] + V.s[1] * V.s[1] + V.s[2] * V.s[2]);
    float B = live ? (float)(fabs((double)y) * diag) : 0.0f;
    float Cs = live ? 1.0f : 0.0f;
    // the window starts zeroed here; each flush zeroes the entries it read, so
    // every chunk finds the entries it uses at zero (block_sum2 synchronises)
    for (int i = threadIdx.x; i < win_cap; i += kBlock) win[i] = 0;
    block_sum2(B, Cs, reinterpret_cast<float*>(red));
    if (Cs == 0.0f) return;                        // no ray of this tile contributes
    const bool fixed_ok = isfinite(B) && B > 0.0f;
    float scale = 0.0f, inv_scale = 0.0f;
    if (fixed_ok) {
        const int e = clampi((int)floor(log2(1073741824.0 / (double)B)), -126, 126);
        scale = ldexpf(1.0f, e);
        inv_scale = ldexpf(1.0f, -e);
    }
    const float ys = y * scale;

    double tc = live ? S.t0 : 0.0;
    const double h = live ? (S.t1 - S.t0) / (double)M : 0.0;
    int guard = V.n[0] + V.n[1] + V.n[2] + 3;
    int Sc = M;
    int k0 = 0;
    while (k0 < M) {
        Sc = min(Sc, M - k0);
        int ext[3], lo[3];
        long long vol;
        double tb = 0.0;
        for (;;) {
            int v[6] = {INT_MAX, INT_MAX, INT_MAX, INT_MAX, INT_MAX, INT_MAX};
            if (live) {
                tb = k0 + Sc >= M ? S.t1 : S.t0 + (double)(k0 + Sc) * h;
                const double ta = tc;
#pragma unroll
                for (int a = 0; a < 3; ++a) {
                    const double ua = (S.C[a] + ta * S.d[a] + V.half_e[a]) * V.inv_s[a];
                    const double ub = (S.C[a] + tb * S.d[a] + V.half_e[a]) * V.inv_s[a];
                    const double lo_u = fmax(floor(fmin(ua, ub)) - 1.0, 0.0);
                    const double hi_u = fmin(floor(fmax(ua, ub)) + 1.0, (double)(V.n[a] - 1));
                    v[a] = (int)lo_u;
                    v[3 + a] = -(int)fmax(hi_u, lo_u);
                }
            }
            block_min6(v, red, box);
            if (box[0] == INT_MAX) break;            // every ray of the tile has ended
            vol = 1;
#pragma unroll
            for (int a = 0; a < 3; ++a) {
                lo[a] = box[a];
                ext[a] = max(-box[3 + a] - box[a] + 1, 1);
                vol *= ext[a];
            }
            if (!fixed_ok || vol <= win_cap || Sc == 1) break;
            Sc = max(1, Sc >> 1);
        }
        if (box[0] == INT_MAX) break;
        const bool windowed = fixed_ok && vol <= win_cap;
        const int wy = ext[0], wz = ext[0] * ext[1];
        // walk this ray's pieces up to tb
        while (live) {
            const NextAxis m = next_axis(S);
            const double te = fmin(m.t, tb);
            const double len = te - tc;
            if (len > 0.0) {
                const float l = (float)len;
                const int wx_ = S.i[0] - lo[0], wy_ = S.i[1] - lo[1], wz_ = S.i[2] - lo[2];
                const bool in_win = windowed && (unsigned)wx_ < (unsigned)ext[0] &&
                                    (unsigned)wy_ < (unsigned)ext[1] &&
                                    (unsigned)wz_ < (unsigned)ext[2];
                if (in_win)
                    atomicAdd(&win[__mul24(wz_, wz) + __mul24(wy_, wy) + wx_],
                              __float2int_rn(l * ys));
                else
                    unsafeAtomicAdd(grad + (uint32_t)S.i[2] * sz + (uint32_t)S.i[1] * sy +
                                        (uint32_t)S.i[0],
                                    y * l);
            }
            tc = fmax(tc, te);
            if (!(m.t <= te)) break;                 // the chunk ends before the crossing
            if (!(m.t < S.t1) || --guard <= 0 || !advance(S, m, V)) live = false;
        }
        if (windowed) {
            __syncthreads();
            // the box lies inside the volume: the gradient offset steps with the walk
            BoxWalk bw(ext);
            BoxAddr ba(bw, lo, sy, sz);
            for (int i = threadIdx.x; i < (int)vol; i += kBlock) {
                const int val = win[i];
                if (val != 0) {
                    win[i] = 0;
                    unsafeAtomicAdd(grad + ba.addr, (float)val * inv_scale);
                }
                int cx, cy;
                bw.next(cx, cy);
                ba.next(cx, cy);
            }
            __syncthreads();
        }
        k0 += Sc;
        // a chunk that left room in the window: try a longer one next
        if (vol * 2 <= win_cap) Sc *= 2;
    }
}

// ----------------------------------------------------------------- launchers

// Pieces in flight per lane: eight, or twelve for fp32 volumes under four
// pieces per cell per view (16 views of 200^2 at 256^3: 0.430 -> 0.399 ms;
// twelve slowed bf16 there, 0.360 -> 0.384 ms, and the denser 1024^2 and helix
// launches by ~10%).
template <typename T, int G>
static void launch_siddon_march(const LaunchArgs& a, const T* v, uint32_t bytes, int tiles_x,
                                int tiles_per_view, int n_tiles, float* out, float* s_out,
                                hipStream_t stream)
{
    const dim3 grid(n_tiles), block(kBlock);
    if (a.mode == kBeerLambert)
        hipLaunchKernelGGL((drr_siddon_march_kernel<T, kBeerLambert, G>), grid, block, 0, stream,
                           v, bytes, a.V, a.K, a.poses, a.H, a.W, tiles_x, tiles_per_view, out,
                           s_out);
    else
        hipLaunchKernelGGL((drr_siddon_march_kernel<T, kLineIntegral, G>), grid, block, 0, stream,
                           v, bytes, a.V, a.K, a.poses, a.H, a.W, tiles_x, tiles_per_view, out,
                           s_out);
}

hipError_t launch_siddon_forward(const LaunchArgs& a, const void* vol, int dtype, float* out,
                                 float* s_out, hipStream_t stream)
{
    const int tiles_x = (a.W + kTile - 1) / kTile, tiles_y = (a.H + kTile - 1) / kTile;
    const int tiles_per_view = tiles_x * tiles_y, n_tiles = tiles_per_view * a.n_views;
    if (n_tiles == 0) return hipSuccess;
    const uint32_t bytes = a.V.total_bytes;
    // pieces one view puts per cell, with about nx + ny + nz pieces per ray
    const double cells = (double)a.V.n[0] * a.V.n[1] * a.V.n[2];
    const double reuse = (double)a.H * a.W * (a.V.n[0] + a.V.n[1] + a.V.n[2]) / cells;
    if (dtype == 0) {
        const float* v = static_cast<const float*>(vol);
        if (reuse < 4.0)
            launch_siddon_march<float, 12>(a, v, bytes, tiles_x, tiles_per_view, n_tiles, out,
                                           s_out, stream);
        else
            launch_siddon_march<float, 8>(a, v, bytes, tiles_x, tiles_per_view, n_tiles, out,
                                          s_out, stream);
    } else {
        launch_siddon_march<uint16_t, 8>(a, static_cast<const uint16_t*>(vol), bytes, tiles_x,
                                         tiles_per_view, n_tiles, out, s_out, stream);
    }
    return hipGetLastError();
}

hipError_t launch_siddon_backward(const LaunchArgs& a, const float* grad_out, const float* s_in,
                                  float* grad, hipStream_t stream)
{
    // chunks of the ray: about one voxel along the longest axis each
    const int M = max(a.V.n[0], max(a.V.n[1], a.V.n[2]));
    // pieces per ray ~ M: the same density measure as the trilinear scatter
    const double cells = (double)(a.V.n[0] + 1) * (a.V.n[1] + 1) * (a.V.n[2] + 1);
    const double view_reuse = (double)a.H * a.W * M / cells;
    // views sparse against the voxels: the brick-owned backward, which writes
    // every voxel itself (no fill, no global atomics)
    if (view_reuse < kBrickMaxViewReuse)
        return launch_siddon_brick_backward(a, grad_out, s_in, grad, stream);
    hipError_t e = launch_fill(grad, (size_t)a.V.n[0] * a.V.n[1] * a.V.n[2], stream);
    if (e != hipSuccess) return e;
    const int tiles_x = (a.W + kTile - 1) / kTile, tiles_y = (a.H + kTile - 1) / kTile;
    const int tiles_per_view = tiles_x * tiles_y, n_tiles = tiles_per_view * a.n_views;
    if (n_tiles == 0) return hipSuccess;
    const dim3 grid(n_tiles), block(kBlock);
    const int cap = window_cap(view_reuse, true);
    const size_t lds = (size_t)cap * sizeof(int);
    if (a.mode == kBeerLambert)
        hipLaunchKernelGGL((drr_siddon_scatter_kernel<kBeerLambert>), grid, block, lds, stream,
                           a.V, a.K, a.poses, a.H, a.W, M, tiles_x, tiles_per_view, grad_out,
                           s_in, grad, cap);
    else
        hipLaunchKernelGGL((drr_siddon_scatter_kernel<kLineIntegral>), grid, block, lds, stream,
                           a.V, a.K, a.poses, a.H, a.W, M, tiles_x, tiles_per_view, grad_out,
                           s_in, grad, cap);
    return hipGetLastError();
}

}  // namespace drr
