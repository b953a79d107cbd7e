// drr_stage.hpp -- LDS staging of volume boxes, shared by the forward march and
// the pose-gradient march: the transfer function, the values a box holds, the
// chunk box of a tile's rays, the fill of the box and the eight corners of a
// sample read back from it.
//
// Method (source pages): flashdrr.rendering VolumeRaycaster class text --
// samples are trilinear (grid_sample) gathers of the volume, mapped per channel
// by the transfer function (np.interp of the knots) before the march.
#pragma once

#include <limits.h>

#include "drr_device.hpp"
#include "drr_internal.hpp"
#include "drr_sample.hpp"
#include "drr_window.hpp"

namespace drr {

// Value of one voxel as fp32 (bf16 widens exactly).
__device__ inline float widen(float x) { return x; }
__device__ inline float widen(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

// The transfer function of channel ch at x (segment search over uniform knots,
// so every knot is a scalar operand); slope receives the segment's slope.
__device__ inline float transfer_eval(const TransferFn& T, int ch, float x, float& slope)
{
    const int b = ch * T.knots;
    float x0 = T.xp[b], y0 = T.yp[b], m = T.m[b];
    for (int i = 1; i < T.knots - 1; ++i) {
        const bool up = x >= T.xp[b + i];
        x0 = up ? T.xp[b + i] : x0;
        y0 = up ? T.yp[b + i] : y0;
        m = up ? T.m[b + i] : m;
    }
    slope = m;
    return fmaf(m, x - x0, y0);
}

// fp32 entries of a staged box: 31 KB, the most that lets five workgroups of
// the forward march share a CU (measured on MI355X: 8192 entries, four per CU,
// against 7936: 1024^2 0.400 -> 0.390 ms, 2048^2 0.763 -> 0.731 ms, the
// 360-view helix 8.58 -> 8.25 ms; 7680: the same; 8064: four per CU again)
constexpr int kStageCap = 7936;

// The value a box entry holds for (unclamped) voxel index (x, y, z): the
// clamped voxel (clamp to edge) of the channel-volume behind `rs`, widened to
// fp32 and mapped by channel ch's transfer function when TF.
template <typename T, bool TF>
__device__ inline float staged_value(__amdgpu_buffer_rsrc_t rs, const VolumeDesc& V, int x,
                                     int y, int z, const TransferFn& tf, int ch)
{
    const uint32_t off = (uint32_t)clampi(z, 0, V.n[2] - 1) * (uint32_t)V.n[1] * (uint32_t)V.n[0] +
                         (uint32_t)clampi(y, 0, V.n[1] - 1) * (uint32_t)V.n[0] +
                         (uint32_t)clampi(x, 0, V.n[0] - 1);
    const float v = load_one<T>(rs, off * (uint32_t)sizeof(T));
    if constexpr (TF) {
        float m;
        return transfer_eval(tf, ch, v, m);
    } else {
        return v;
    }
}

// Box of the tile's chunk: every thread passes the floors bounding its ray's
// corners for the chunk (lo_f, hi_f per axis; INT_MAX when it has none), the
// workgroup reduces them (red: (kBlock / 64) * 6 ints, bb: 6 ints of LDS) and
// every thread gets the box corner lo, its extent ext (entries per axis, the
// high corner included) and its entry count.  Returns false when no thread has
// a ray in the chunk.
__device__ inline bool chunk_box(const int lo_f[3], const int hi_f[3], int* red, int* bb,
                                 int lo[3], int ext[3], long long& cells)
{
    int v[6];
#pragma unroll
    for (int a = 0; a < 3; ++a) {
        v[a] = lo_f[a];
        v[3 + a] = hi_f[a] == INT_MAX ? INT_MAX : -(hi_f[a] + 1);
    }
    block_min6(v, red, bb);
    if (bb[0] == INT_MAX) return false;
    cells = 1;
#pragma unroll
    for (int a = 0; a < 3; ++a) {
        lo[a] = bb[a];
        ext[a] = max(-bb[3 + a] - bb[a] + 1, 1);
        cells *= ext[a];
    }
    return true;
}

// Fill box[0, n) with the entries of the box at corner lo, extent ext (x
// fastest), eight loads in flight per thread before the first LDS write.  The
// caller synchronises afterwards.
template <typename T, bool TF>
__device__ inline void stage_fill(float* box, int n, __amdgpu_buffer_rsrc_t rs,
                                  const VolumeDesc& V, const int lo[3], const int ext[3],
                                  const TransferFn& tf, int ch)
{
    BoxWalk bw(ext);
    int i = threadIdx.x;
    constexpr int kFill = 8;
    bool interior = true;
#pragma unroll
    for (int a = 0; a < 3; ++a) interior = interior && lo[a] >= 0 && lo[a] + ext[a] <= V.n[a];
    if (interior) {
        // every entry is a voxel: no clamping, and the element offset steps
        // with the walk
        BoxAddr ba(bw, lo, (uint32_t)V.n[0], (uint32_t)V.n[0] * (uint32_t)V.n[1]);
        if constexpr (sizeof(T) == 4 && !TF) {
            // fp32 as it is: the loads write LDS themselves (buffer_load ...
            // lds puts lane l's dword at the wave's base + 4 l, and the
            // entries i of one wave and round are consecutive), so no value
            // passes through registers; they complete before the caller's
            // barrier
            for (; i < n; i += kBlock) {
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rs, (__attribute__((address_space(3))) void*)(box + (i & ~63)), 4,
                    ba.addr * 4u, 0, 0, 0);
                int cx, cy;
                bw.next(cx, cy);
                ba.next(cx, cy);
            }
            __builtin_amdgcn_s_waitcnt(0);
            return;
        }
        auto value = [&](uint32_t off) {
            const float v = load_one<T>(rs, off * (uint32_t)sizeof(T));
            if constexpr (TF) {
                float m;
                return transfer_eval(tf, ch, v, m);
            } else {
                return v;
            }
        };
        for (; i + (kFill - 1) * kBlock < n; i += kFill * kBlock) {
            float v[kFill];
#pragma unroll
            for (int u = 0; u < kFill; ++u) {
                v[u] = value(ba.addr);
                int cx, cy;
                bw.next(cx, cy);
                ba.next(cx, cy);
            }
#pragma unroll
            for (int u = 0; u < kFill; ++u) box[i + u * kBlock] = v[u];
        }
        for (; i < n; i += kBlock) {
            box[i] = value(ba.addr);
            int cx, cy;
            bw.next(cx, cy);
            ba.next(cx, cy);
        }
        return;
    }
    for (; i + (kFill - 1) * kBlock < n; i += kFill * kBlock) {
        float v[kFill];
#pragma unroll
        for (int u = 0; u < kFill; ++u, bw.next())
            v[u] = staged_value<T, TF>(rs, V, lo[0] + bw.x, lo[1] + bw.y, lo[2] + bw.z, tf, ch);
#pragma unroll
        for (int u = 0; u < kFill; ++u) box[i + u * kBlock] = v[u];
    }
    for (; i < n; i += kBlock, bw.next())
        box[i] = staged_value<T, TF>(rs, V, lo[0] + bw.x, lo[1] + bw.y, lo[2] + bw.z, tf, ch);
}

// The eight corners of a cell of the staged box at byte address p (row and
// slice strides sy, sz in bytes): four pairs adjacent in x.
__device__ inline void box_corners(const char* p, uint32_t sy, uint32_t sz, CornerVals& c)
{
    const float* p00 = reinterpret_cast<const float*>(p);
    const float* p10 = reinterpret_cast<const float*>(p + sy);
    const float* p01 = reinterpret_cast<const float*>(p + sz);
    const float* p11 = reinterpret_cast<const float*>(p + sz + sy);
    c.v[0] = p00[0]; c.v[1] = p00[1];
    c.v[2] = p10[0]; c.v[3] = p10[1];
    c.v[4] = p01[0]; c.v[5] = p01[1];
    c.v[6] = p11[0]; c.v[7] = p11[1];
}

// LDS byte offset of the cell at fixed-point position q (relative to the box
// corner) in a box of byte strides sy, sz.
__device__ inline uint32_t box_offset(int64_t qx, int64_t qy, int64_t qz, uint32_t sy,
                                      uint32_t sz)
{
    return fixed_floor_x4_add(qx, __umul24((uint32_t)fixed_floor(qz), sz) +
                                      __umul24((uint32_t)fixed_floor(qy), sy));
}

}  // namespace drr
