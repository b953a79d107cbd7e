// drr_window.hpp -- workgroup helpers of the backward scatters: the LDS window
// size, block-wide reductions, and the interleaved pixel layout of a tile.
//
// Method (source pages): flashdrr.rendering VolumeRaycaster class text --
// rendering is differentiable with respect to the volume; diffct 2.1.0
// Quickstart -- backproject() applies the matched adjoint.
#pragma once

#include <limits.h>

#include "drr_device.hpp"

namespace drr {

// LDS window of the backward scatters, sized per launch (dynamic LDS).  When
// one view's rays are dense against the voxels a tile's box is thin, chunks
// are long, and occupancy matters: 6144 int32 (24 KB) lets six workgroups
// share a CU (the scatter's registers allow six waves per SIMD).  When they
// are sparse (a voxel or more between neighbouring rays) the box is wide,
// chunks are short, and a larger window saves chunks: 16000 entries (62.5 KB,
// two workgroups per CU, under the 64 KB default dynamic-LDS limit).
// Measured on MI355X (1024^2 step / 360-view helix / 16-view 200^2 batch):
// 4096 entries 1.15 / 27.9 / - ms, 6144 1.12 / 19.9 / 7.37, 8192
// 1.19 / 21.4 / 4.96, 12288 1.28 / 23.8 / 3.08, 16384 - / - / 2.81,
// 24576 2.68 / 56.0 / 4.89.  With the later scatter (register sums started on
// the lane's own cell, uniform trip counts, flush reads ahead) views between
// 4 and 16 samples per cell run better on 7168 entries (five workgroups per
// CU): the helix (11.7 per view) 15.2 -> 12.1 ms, its cell-constant backward
// 11.9 -> 11.4 ms, the 1024^2 step (31.6) unchanged at 6144 (7168: 0.577 ->
// 0.591 ms; 8192 and 10240 slowed the 1024^2 cell-constant backward, 9.6
// pieces per cell: 0.60 -> 0.65 / 0.73 ms).  The trilinear scatter now takes
// the largest window that still lets five workgroups share a CU: 7936 entries
// (31 KB), helix 12.2 -> 11.3 ms (7424: 11.8, 7680: 11.4-11.5; 8128 and 8192,
// four per CU: 11.5; 10240: 12.9); the cell-constant scatter keeps 7168 (7680:
// 1024^2 0.593 -> 0.598 ms, helix 11.24 -> 11.11 ms; 8192: 0.638 / 12.1 ms).
constexpr int kWinCapDense = 6144;
constexpr int kWinCapMid = 7936;
constexpr int kWinCapMidSiddon = 7168;
constexpr int kWinCapSparse = 16000;

// Window entries for a launch whose views each put `view_reuse` samples per
// cell of the volume (trilinear), or ray-voxel pieces (cell-constant, SIDDON).
inline int window_cap(double view_reuse, bool siddon = false)
{
    const int mid = siddon ? kWinCapMidSiddon : kWinCapMid;
    return view_reuse >= 16.0 ? kWinCapDense : (view_reuse >= 4.0 ? mid : kWinCapSparse);
}

// Trilinear weights of one sample scaled by c: w[n] for corner n (bit 0 = x1,
// bit 1 = y1, bit 2 = z1), the same products as corner_weights without clamps.
// Add c times the eight trilinear weights of fractions (fx, fy, fz) to acc,
// corner order x fastest: acc[i] += c w_x(i & 1) w_y((i >> 1) & 1) w_z(i >> 2).
__device__ inline void add_weights8(float fx, float fy, float fz, float c, float acc[8])
{
    const float wz1 = c * fz, wz0 = c - wz1;
    const float w11 = wz1 * fy, w10 = wz1 - w11;
    const float w01 = wz0 * fy, w00 = wz0 - w01;
    const float fx0 = 1.0f - fx;
    acc[0] = fmaf(w00, fx0, acc[0]);
    acc[1] = fmaf(w00, fx, acc[1]);
    acc[2] = fmaf(w01, fx0, acc[2]);
    acc[3] = fmaf(w01, fx, acc[3]);
    acc[4] = fmaf(w10, fx0, acc[4]);
    acc[5] = fmaf(w10, fx, acc[5]);
    acc[6] = fmaf(w11, fx0, acc[6]);
    acc[7] = fmaf(w11, fx, acc[7]);
}

// The same from fractions times 2^32 (Fx = 2^32 fx, exactly the low word of a
// 32.32 position as a float: one conversion, no scaling per sample), with the
// coefficient passed as c 2^-96 and c 2^-64: every product then carries the
// scale it needs, the complements are 2^32 - F (rounded as 1 - f would be),
// and the eight additions equal c w_corner.  A coefficient below 2^-30 (in
// window units) may lose precision to subnormals, far below the window's unit.
__device__ inline void add_weights8_scaled(float Fx, float Fy, float Fz, float c96, float c64,
                                           float acc[8])
{
    constexpr float kTwo32 = 4294967296.0f;
    const float gx = kTwo32 - Fx, gy = kTwo32 - Fy;
    const float wz1 = c96 * Fz, wz0 = fmaf(-c96, Fz, c64);      // c fz 2^-64, c (1 - fz) 2^-64
    const float w11 = wz1 * Fy, w10 = wz1 * gy;                 // times 2^32 in y
    const float w01 = wz0 * Fy, w00 = wz0 * gy;
    acc[0] = fmaf(w00, gx, acc[0]);
    acc[1] = fmaf(w00, Fx, acc[1]);
    acc[2] = fmaf(w01, gx, acc[2]);
    acc[3] = fmaf(w01, Fx, acc[3]);
    acc[4] = fmaf(w10, gx, acc[4]);
    acc[5] = fmaf(w10, Fx, acc[5]);
    acc[6] = fmaf(w11, gx, acc[6]);
    acc[7] = fmaf(w11, Fx, acc[7]);
}

// Position (x, y, z) of entry i = threadIdx.x + n kBlock of a box of
// ext[0] x ext[1] x ... entries (x fastest), advanced kBlock entries per
// step with carries instead of divisions.
struct BoxWalk {
    int x, y, z;
    int sx, sy, sz, ex, ey;

    __device__ explicit BoxWalk(const int ext[3])
    {
        ex = ext[0];
        ey = ext[1];
        const int r = (int)threadIdx.x / ex, q = kBlock / ex;
        x = (int)threadIdx.x - r * ex;
        y = r % ey;
        z = r / ey;
        sx = kBlock - q * ex;
        sy = q % ey;
        sz = q / ey;
    }
    __device__ void next()
    {
        int cx, cy;
        next(cx, cy);
    }

    // The same, reporting the carries out of x and out of y (0 or 1).
    __device__ void next(int& cx, int& cy)
    {
        x += sx;                       // sx < ex: at most one carry
        cx = x >= ex ? 1 : 0;
        x -= cx * ex;
        y += sy + cx;                  // sy + cx <= ey: at most one carry
        cy = y >= ey ? 1 : 0;
        y -= cy * ey;
        z += sz + cy;
    }
};

// Element offset in a volume (row stride vy, slice stride vz elements) of the
// entries a BoxWalk visits, box corner lo, stepped with the walk's carries
// instead of multiplied out; valid for a box inside the volume.
struct BoxAddr {
    uint32_t addr;
    uint32_t step, carry_x, carry_y;

    __device__ BoxAddr(const BoxWalk& w, const int lo[3], uint32_t vy, uint32_t vz)
    {
        addr = (uint32_t)(lo[2] + w.z) * vz + (uint32_t)(lo[1] + w.y) * vy + (uint32_t)(lo[0] + w.x);
        step = (uint32_t)w.sx + (uint32_t)w.sy * vy + (uint32_t)w.sz * vz;
        carry_x = vy - (uint32_t)w.ex;                 // next row: back ex, on vy
        carry_y = vz - (uint32_t)w.ey * vy;            // next slice: back ey rows, on vz
    }
    __device__ void next(int cx, int cy)
    {
        addr += step + (cx ? carry_x : 0u) + (cy ? carry_y : 0u);
    }
};

// Workgroup-wide min of six ints (maxima are passed negated).
__device__ inline void block_min6(int v[6], int* red, int* out)
{
#pragma unroll
    for (int i = 0; i < 6; ++i) v[i] = wave_min(v[i]);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (lane == 0) {
#pragma unroll
        for (int i = 0; i < 6; ++i) red[wave * 6 + i] = v[i];
    }
    __syncthreads();
    if (threadIdx.x < 6) {
        int m = red[threadIdx.x];
        for (int w = 1; w < kBlock / 64; ++w) m = min(m, red[w * 6 + threadIdx.x]);
        out[threadIdx.x] = m;
    }
    __syncthreads();
}

// Workgroup-wide sums of two floats.
__device__ inline void block_sum2(float& a, float& b, float* red)
{
    a = wave_sum(a);
    b = wave_sum(b);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (lane == 0) {
        red[2 * wave] = a;
        red[2 * wave + 1] = b;
    }
    __syncthreads();
    a = 0.0f;
    b = 0.0f;
#pragma unroll
    for (int w = 0; w < kBlock / 64; ++w) {
        a += red[2 * w];
        b += red[2 * w + 1];
    }
    __syncthreads();
}

// Pixel owned by a thread of the backward: the 16 x 16 tile is split into four
// interleaved 8 x 8 lattices (stride 2), one per wave, so the 64 lanes of a
// wave sit two pixels apart and rarely target the same voxel in one LDS atomic
// instruction (same-address lanes serialise).  Measured on the 1024^2 step:
// 2.97 ms with 8 x 8 contiguous wave tiles, 1.56 ms interleaved.  (Wider
// lattices -- 32 x 32 tiles, four rays per thread -- cost registers and window
// room and were slower.)
__device__ inline PixelCoord scatter_pixel(int tile, int tiles_x, int tiles_per_view)
{
    PixelCoord p;
    p.view = tile / tiles_per_view;
    const int t = tile - p.view * tiles_per_view;
    const int ty = t / tiles_x, tx = t - ty * tiles_x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    p.r = ty * kTile + 2 * (lane >> 3) + (wave >> 1);
    p.c = tx * kTile + 2 * (lane & 7) + (wave & 1);
    return p;
}

}  // namespace drr
