// drr_device.hpp -- device-side building blocks of the cone-beam DRR path for
// gfx950: per-view camera setup, per-ray generation and box clipping, exact
// fixed-point sample stepping, and the clamped trilinear cell of a sample.
// Shared by the forward march and the backward scatter so both see
// bit-identical sample positions.
//
// Method (source pages): nanodrr introduction (Hartley-Zisserman pinhole
// camera, P = K [R | t]); flashdrr.rendering VolumeRaycaster.set_fov
// (normalised per-pixel directions), __init__ (ray_samples, Beer-Lambert) and
// class text (trilinear grid_sample gathers, differentiable in the volume).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace drr {

constexpr int kTile = 16;          // a workgroup renders a 16 x 16 pixel tile
constexpr int kWaveTile = 8;       // each wave64 renders an 8 x 8 sub-tile
constexpr int kBlock = kTile * kTile;
constexpr int kNumXcd = 8;         // MI355X: 8 XCDs, each with its own L2

// Raw-buffer descriptor word 3 for the gfx9 family (untyped dword access).
constexpr int kBufferWord3 = 0x00020000;

struct Intrinsics {
    float k[9];                    // row-major 3x3 K
};

// Volume description.  Sample positions are continuous voxel indices q
// (voxel centres at integers, q = (p + E/2) / s - 1/2) kept in 32.32 fixed
// point: the high word is floor(q), the low word the trilinear weight of the
// upper corner in units of 2^-32.  Stepping along a ray is an exact 64-bit
// integer add, so the only position error is the rounding of the start and of
// the step to 2^-33 voxel (about 6e-8 voxel after 512 steps) -- far below the
// 1e-5 voxel an fp32 position carries at |q| ~ 128, which would move a
// low-signal ray's integral at a sharp air/tissue edge by more than 1e-5.
struct VolumeDesc {
    int n[3];                      // nx, ny, nz
    double s[3];                   // spacing (mm)
    double inv_s[3];               // 1 / spacing
    double half_e[3];              // box half extent n s / 2 (mm)
    double q_off[3];               // E / (2 s) - 1/2 = (n - 1) / 2
    uint32_t row_bytes;            // nx * element size
    uint32_t slice_bytes;          // nx * ny * element size
    uint32_t total_bytes;          // whole volume (buffer range)
    // corner-cell copy (when the forward uses one): (nx+1) x (ny+1) x (nz+1)
    // cells of 8 elements, cell (i, j, k) holding the clamped corners of the
    // trilinear cell whose low corner is voxel (i-1, j-1, k-1)
    uint32_t cell_row_bytes;
    uint32_t cell_slice_bytes;
    uint32_t cell_total_bytes;
};

// Several volumes and channels in one call (flashdrr API,
// VolumeRaycaster.forward: (B, C, D, H, W) volumes, N = B * views_per_vol
// views, view v rendering volume v / views_per_vol, output (N, C, H, W)).  A
// launch covers every (view, channel) pair; channel-volume (b, c) sits at
// element offset (b * C + c) * (one volume) of its array.  The density factor
// scales mu (optical depth f dz sum mu); margin widens the near/far range.
struct Batch {
    uint64_t src_stride;           // bytes from one channel-volume to the next (read side)
    uint32_t grad_stride;          // fp32 elements per gradient channel-volume
    int C;                         // channels
    int vpv;                       // views per volume
    float f;                       // density factor
    float margin;                  // near/far margin (mm)
};

// Per-view camera, fp64: world direction of image point (u, v, 1) is
// M (u, v, 1) with M = R^T K^-1; camera centre C = -R^T t.
struct ViewGeom {
    double M[9];
    double C[3];
};

// One clipped ray: sample k sits at q = q0 + k dq (32.32 fixed point), the
// midpoint rule t_k = t0 + (k + 1/2) dz.
struct MarchRay {
    int64_t q0[3];
    int64_t dq[3];
    float dz;                      // (t1 - t0) / N in mm
};

// K^-1 = adj(K) / det(K), fp64.
__device__ inline void intrinsics_inverse(const Intrinsics& K, double Ki[9])
{
    double k[9];
#pragma unroll
    for (int i = 0; i < 9; ++i) k[i] = (double)K.k[i];
    const double a00 = k[4] * k[8] - k[5] * k[7];
    const double a01 = k[2] * k[7] - k[1] * k[8];
    const double a02 = k[1] * k[5] - k[2] * k[4];
    const double a10 = k[5] * k[6] - k[3] * k[8];
    const double a11 = k[0] * k[8] - k[2] * k[6];
    const double a12 = k[2] * k[3] - k[0] * k[5];
    const double a20 = k[3] * k[7] - k[4] * k[6];
    const double a21 = k[1] * k[6] - k[0] * k[7];
    const double a22 = k[0] * k[4] - k[1] * k[3];
    const double inv_det = 1.0 / (k[0] * a00 + k[1] * a10 + k[2] * a20);
    Ki[0] = a00 * inv_det; Ki[1] = a01 * inv_det; Ki[2] = a02 * inv_det;
    Ki[3] = a10 * inv_det; Ki[4] = a11 * inv_det; Ki[5] = a12 * inv_det;
    Ki[6] = a20 * inv_det; Ki[7] = a21 * inv_det; Ki[8] = a22 * inv_det;
}

__device__ inline void view_setup(const float* __restrict__ pose, const Intrinsics& K,
                                  ViewGeom& G)
{
    double Ki[9];
    intrinsics_inverse(K, Ki);
    double R[9], t[3];
#pragma unroll
    for (int r = 0; r < 3; ++r) {
#pragma unroll
        for (int c = 0; c < 3; ++c) R[r * 3 + c] = (double)pose[r * 4 + c];
        t[r] = (double)pose[r * 4 + 3];
    }
#pragma unroll
    for (int a = 0; a < 3; ++a) {
#pragma unroll
        for (int b = 0; b < 3; ++b)
            G.M[a * 3 + b] = R[0 * 3 + a] * Ki[0 * 3 + b] + R[1 * 3 + a] * Ki[1 * 3 + b] +
                             R[2 * 3 + a] * Ki[2 * 3 + b];
        G.C[a] = -(R[0 * 3 + a] * t[0] + R[1 * 3 + a] * t[1] + R[2 * 3 + a] * t[2]);
    }
}

constexpr int64_t kFixedOne = int64_t(1) << 32;   // 1.0 in 32.32 fixed point

__device__ inline int64_t to_fixed(double x) { return __double2ll_rn(x * 4294967296.0); }

// Unit world direction of the ray through pixel (r, c), fp64.
__device__ inline void ray_direction(const ViewGeom& G, int r, int c, double d[3])
{
    const double u = (double)c + 0.5, v = (double)r + 0.5;
#pragma unroll
    for (int a = 0; a < 3; ++a) d[a] = G.M[a * 3 + 0] * u + G.M[a * 3 + 1] * v + G.M[a * 3 + 2];
    const double inv_len = 1.0 / sqrt(d[0] * d[0] + d[1] * d[1] + d[2] * d[2]);
#pragma unroll
    for (int a = 0; a < 3; ++a) d[a] *= inv_len;
}

// The N midpoint samples of [t0, t1] on the ray C + t d, in fixed point.
__device__ inline void march_from_range(const ViewGeom& G, const VolumeDesc& V, const double d[3],
                                        double t0, double t1, int N, MarchRay& R)
{
    const double dz = (t1 - t0) / (double)N;
    const double ts = t0 + 0.5 * dz;
#pragma unroll
    for (int a = 0; a < 3; ++a) {
        R.q0[a] = to_fixed((G.C[a] + ts * d[a]) * V.inv_s[a] + V.q_off[a]);
        R.dq[a] = to_fixed(dz * d[a] * V.inv_s[a]);
    }
    R.dz = (float)dz;
}

// Ray through pixel (r, c), clipped to the volume box by the slab method in
// fp64.  Returns false when the ray misses (t1 <= t0 with t0 = max(t_entry, 0)).
__device__ inline bool ray_setup(const ViewGeom& G, const VolumeDesc& V, int r, int c, int N,
                                 MarchRay& R)
{
    double d[3];
    ray_direction(G, r, c, d);
    double t_entry = -__builtin_inf(), t_exit = __builtin_inf();
    bool inside = true;
#pragma unroll
    for (int a = 0; a < 3; ++a) {
        const double lo = -V.half_e[a], hi = V.half_e[a];
        if (d[a] == 0.0) {
            inside = inside && !(G.C[a] < lo || G.C[a] > hi);
        } else {
            const double ta = (lo - G.C[a]) / d[a];
            const double tb = (hi - G.C[a]) / d[a];
            t_entry = fmax(t_entry, fmin(ta, tb));
            t_exit = fmin(t_exit, fmax(ta, tb));
        }
    }
    const double t0 = fmax(t_entry, 0.0);
    if (!inside || !(t_exit > t0)) return false;
    march_from_range(G, V, d, t0, t_exit, N, R);
    return true;
}

// Per-view clipping range of the near/far mode (flashdrr API,
// compute_clipping_distances: one near and one far distance per view, from the
// camera to the closest and to the farthest point of the volume, widened by a
// margin): the closest point of the box (distance 0 inside it) and its
// farthest corner; near is not allowed below 0.
__device__ inline void view_near_far(const ViewGeom& G, const VolumeDesc& V, float margin,
                                     double& t_near, double& t_far)
{
    double dn2 = 0.0, df2 = 0.0;
#pragma unroll
    for (int a = 0; a < 3; ++a) {
        const double h = V.half_e[a], c = G.C[a];
        const double dn = c < -h ? -h - c : (c > h ? c - h : 0.0);
        const double df = fabs(c) + h;
        dn2 += dn * dn;
        df2 += df * df;
    }
    t_near = fmax(sqrt(dn2) - (double)margin, 0.0);
    t_far = sqrt(df2) + (double)margin;
}

// Ray through pixel (r, c) sampled over the view's [t_near, t_far] (near/far
// mode: every ray of the view shares the range; samples outside the volume
// read zero padding).  Returns false when the range is empty.
__device__ inline bool ray_setup_range(const ViewGeom& G, const VolumeDesc& V, int r, int c, int N,
                                       double t_near, double t_far, MarchRay& R)
{
    if (!(t_far > t_near)) return false;
    double d[3];
    ray_direction(G, r, c, d);
    march_from_range(G, V, d, t_near, t_far, N, R);
    return true;
}

// Samples [k_lo, k_hi) of a near/far march whose continuous index lies in
// [-1, n) on every axis: the zero-padded trilinear support.  Every other sample
// reads only padding and adds exactly 0 (to the sum, the composite and the
// gradient), so the march can skip it.  The bounds come from the fixed-point
// start and step in fp64 and are widened by one sample each way.
__device__ inline void padded_support(const MarchRay& R, const VolumeDesc& V, int N, int& k_lo,
                                      int& k_hi)
{
    double lo = 0.0, hi = (double)N;
    bool none = false;             // an axis the ray does not move along, outside the support
#pragma unroll
    for (int a = 0; a < 3; ++a) {
        const double q0 = (double)R.q0[a] * 2.3283064365386963e-10;
        const double dq = (double)R.dq[a] * 2.3283064365386963e-10;
        const double b0 = -1.0, b1 = (double)V.n[a];
        if (dq == 0.0) {
            none = none || !(q0 >= b0 && q0 < b1);
        } else {
            const double k0 = (b0 - q0) / dq, k1 = (b1 - q0) / dq;
            lo = fmax(lo, fmin(k0, k1));
            hi = fmin(hi, fmax(k0, k1));
        }
    }
    lo = fmin(fmax(lo, 0.0), (double)N);
    hi = fmin(fmax(hi, 0.0), (double)N);
    k_lo = max((int)floor(lo) - 1, 0);
    k_hi = min((int)ceil(hi) + 1, N);
    if (none || k_hi < k_lo) k_hi = k_lo;
}

__device__ inline int fixed_floor(int64_t q) { return (int)(q >> 32); }

// 4 floor(q) + off in one instruction on the high word.  Left to itself the
// compiler folds the shift into a 64-bit funnel shift and a mask, then adds
// (three instructions for what v_lshl_add_u32 does in one).
__device__ inline uint32_t fixed_floor_x4_add(int64_t q, uint32_t off)
{
    uint32_t r;
    asm("v_lshl_add_u32 %0, %1, 2, %2" : "=v"(r) : "v"((uint32_t)(q >> 32)), "v"(off));
    return r;
}

// a b + c for a, b < 2^24 in one v_mad_u32_u24, with b a wave-uniform value
// (an SGPR operand).  Left to itself the compiler keeps a uniform c in an SGPR
// as well, which the instruction cannot take beside b, and spends a multiply
// and a three-way add instead.
__device__ inline uint32_t mad_u24(uint32_t a, uint32_t b, uint32_t c)
{
    uint32_t r;
    asm("v_mad_u32_u24 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(b), "v"(c));
    return r;
}

__device__ inline float fixed_frac(int64_t q)
{
    return (float)(uint32_t)q * 2.3283064365386963e-10f;  // 2^-32
}

__device__ inline int clampi(int i, int lo, int hi) { return min(max(i, lo), hi); }

// Keeps per-sample position updates a chain of single adds: without it the
// compiler rebuilds q + i dq for every unrolled sample from precomputed
// multiples, which costs more 64-bit adds than it saves.
__device__ inline void serial_step(int64_t& qx, int64_t& qy, int64_t& qz)
{
    asm("" : "+v"(qx), "+v"(qy), "+v"(qz));
}

// The same, placed where a sample's fractions have been taken from the
// positions: the position registers can then be updated in place.
__device__ inline void serial_step_after(int64_t& qx, int64_t& qy, int64_t& qz, float tx,
                                         float ty, float tz)
{
    asm("" : "+v"(qx), "+v"(qy), "+v"(qz) : "v"(tx), "v"(ty), "v"(tz));
}

// Clamped trilinear cell of a sample: both corner indices per axis clamped to
// [0, n-1] (clamp to edge) and the weights of the upper corners.
struct Cell {
    int x0, x1, y0, y1, z0, z1;
    float fx, fy, fz;
};

__device__ inline void cell_of(const VolumeDesc& V, int64_t qx, int64_t qy, int64_t qz, Cell& C)
{
    const int ix = fixed_floor(qx), iy = fixed_floor(qy), iz = fixed_floor(qz);
    C.fx = fixed_frac(qx);
    C.fy = fixed_frac(qy);
    C.fz = fixed_frac(qz);
    C.x0 = clampi(ix, 0, V.n[0] - 1);
    C.x1 = clampi(ix + 1, 0, V.n[0] - 1);
    C.y0 = clampi(iy, 0, V.n[1] - 1);
    C.y1 = clampi(iy + 1, 0, V.n[1] - 1);
    C.z0 = clampi(iz, 0, V.n[2] - 1);
    C.z1 = clampi(iz + 1, 0, V.n[2] - 1);
}

// Map a hardware workgroup id to a logical tile so that the workgroups one XCD
// receives (ids x, x + 8, x + 16, ...) own one contiguous run of tiles: every
// XCD's L2 then serves a compact part of the detector, and so of the volume.
// Inclusive prefix sum over a wave64 by DPP lane moves (no LDS round trips):
// shifts by 1, 2, 4 and 8 lanes within each row of 16 (Hillis-Steele), then
// the last lane of rows 0 and 2 added to rows 1 and 3, and lane 31 added to
// rows 2 and 3.  A lane the move has no source for adds 0.
__device__ inline int wave_inclusive_scan(int x)
{
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31
    return x;
}

// Minimum over a wave64, left in lane 63 (the same DPP moves; a lane without
// a source takes INT_MAX), then read from that lane.
__device__ inline int wave_min(int x)
{
    constexpr int kMax = 0x7fffffff;
    x = min(x, __builtin_amdgcn_update_dpp(kMax, x, 0x111, 0xf, 0xf, false));
    x = min(x, __builtin_amdgcn_update_dpp(kMax, x, 0x112, 0xf, 0xf, false));
    x = min(x, __builtin_amdgcn_update_dpp(kMax, x, 0x114, 0xf, 0xf, false));
    x = min(x, __builtin_amdgcn_update_dpp(kMax, x, 0x118, 0xf, 0xf, false));
    x = min(x, __builtin_amdgcn_update_dpp(kMax, x, 0x142, 0xa, 0xf, false));
    x = min(x, __builtin_amdgcn_update_dpp(kMax, x, 0x143, 0xc, 0xf, false));
    return __builtin_amdgcn_readlane(x, 63);
}

// Sum of a float over a wave64 the same way (a lane without a source adds 0).
template <int CTRL, int ROW_MASK>
__device__ inline float dpp_move(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf,
                                                      false));
}

__device__ inline float wave_sum(float x)
{
    x += dpp_move<0x111, 0xf>(x);
    x += dpp_move<0x112, 0xf>(x);
    x += dpp_move<0x114, 0xf>(x);
    x += dpp_move<0x118, 0xf>(x);
    x += dpp_move<0x142, 0xa>(x);
    x += dpp_move<0x143, 0xc>(x);
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}

__device__ inline int xcd_contiguous_tile(int bid, int nblocks)
{
    const int xcd = bid % kNumXcd, idx = bid / kNumXcd;
    const int per = nblocks / kNumXcd, rem = nblocks % kNumXcd;
    return xcd * per + min(xcd, rem) + idx;
}

// Pixel owned by this thread: 16 x 16 tiles, four 8 x 8 wave sub-tiles.
struct PixelCoord {
    int view, r, c;
};

__device__ inline PixelCoord tile_pixel(int tile, int tiles_x, int tiles_per_view)
{
    PixelCoord p;
    p.view = tile / tiles_per_view;
    const int t = tile - p.view * tiles_per_view;
    const int ty = t / tiles_x, tx = t - ty * tiles_x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    p.r = ty * kTile + (wave >> 1) * kWaveTile + (lane >> 3);
    p.c = tx * kTile + (wave & 1) * kWaveTile + (lane & 7);
    return p;
}

// The same 16 x 16 tile with each wave64 on a 16 x 4 strip of rows.  The march
// that gathers from a copy in global memory reads rows of 16 consecutive x
// per 128-byte line, so wider wave footprints touch fewer lines per load for
// views that look along z or y: measured on MI355X, 16 views of 200^2 over
// 256^3 from z-pairs 0.562 -> 0.543 ms (fp32), 0.445 -> 0.437 ms (bf16); the
// LDS-staged marches gain nothing from it (1024^2 compositing 0.590 -> 0.600 ms).
__device__ inline PixelCoord tile_pixel_rows(int tile, int tiles_x, int tiles_per_view)
{
    PixelCoord p;
    p.view = tile / tiles_per_view;
    const int t = tile - p.view * tiles_per_view;
    const int ty = t / tiles_x, tx = t - ty * tiles_x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    p.r = ty * kTile + wave * 4 + (lane >> 4);
    p.c = tx * kTile + (lane & 15);
    return p;
}

}  // namespace drr
