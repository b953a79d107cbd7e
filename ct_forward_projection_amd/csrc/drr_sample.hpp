// drr_sample.hpp -- how a march reads the eight trilinear corners of a sample
// (shared by the forward and the pose-gradient kernels): buffer loads of the
// volume as x-pairs or single elements, or of the corner-cell copy, and the
// trilinear interpolation (with its gradient) of the eight values.
//
// Method (source pages): flashdrr.rendering VolumeRaycaster class text --
// samples are trilinear (grid_sample) gathers of the volume.
#pragma once

#include "drr_device.hpp"

namespace drr {

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two x-neighbours (x, x+1) of one volume row starting at byte offset `off`.
template <typename T>
__device__ inline void load_pair(__amdgpu_buffer_rsrc_t rs, uint32_t off, float& a, float& b);

template <>
__device__ inline void load_pair<float>(__amdgpu_buffer_rsrc_t rs, uint32_t off, float& a,
                                        float& b)
{
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(rs, (int)off, 0, 0);
    a = __uint_as_float((uint32_t)v[0]);
    b = __uint_as_float((uint32_t)v[1]);
}

template <>
__device__ inline void load_pair<uint16_t>(__amdgpu_buffer_rsrc_t rs, uint32_t off, float& a,
                                           float& b)
{
    const uint32_t v = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)off, 0, 0);
    a = bf16_lo(v);
    b = bf16_hi(v);
}

template <typename T>
__device__ inline float load_one(__amdgpu_buffer_rsrc_t rs, uint32_t off);

template <>
__device__ inline float load_one<float>(__amdgpu_buffer_rsrc_t rs, uint32_t off)
{
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, (int)off, 0, 0));
}

template <>
__device__ inline float load_one<uint16_t>(__amdgpu_buffer_rsrc_t rs, uint32_t off)
{
    return __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, (int)off, 0, 0)
                           << 16);
}

// How the march reads the eight trilinear corners of a sample.
//   Pair   (nx >= 2): each of the four (y, z) rows is one x-pair load starting
//          at xp = clamp(ix, 0, nx - 2); at the clamped x edges the pair still
//          holds the right voxel and the weight is pinned to 0 (ix < 0) or 1
//          (ix > nx - 2), which is exactly clamp to edge.  4 loads per sample.
//   Single (nx == 1): the x corners are read one by one.  8 loads per sample.
//   Cell   (corner-cell copy): the 8 clamped corners are one 16-byte (bf16) or
//          two 16-byte (fp32) loads at cell (ix + 1, iy + 1, iz + 1); no clamp.
//   ZPair  (z-pair copy, nx >= 2 and nz >= 2): element (x, y, z) of the copy,
//          0 <= z <= nz - 2, holds the voxels (x, y, z) and (x, y, z + 1), so
//          the x-neighbours (xp, xp + 1) of one y row are four values in one
//          16-byte (fp32) or 8-byte (bf16) load: 2 loads per sample.  x and z
//          are pinned at the clamped edges as in Pair.  With zero padding the
//          copy has a border of zeros instead (pairs for x, y in [-1, n] and z
//          in [-1, nz - 1]) and nothing is pinned.
enum class Layout { Single, Pair, Cell, ZPair };

struct SampleAddr {
    uint32_t o, dy, dz;            // bytes: first row (+ x offset), row steps
    uint32_t x1;                   // Single: byte offset of the x1 corner minus x0
    float fx, fy, fz;
    float gxs;                     // Pair, ZPair: 0 where the x weight was pinned at a
                                   // clamped edge (the field is flat in x there), else 1
    float gzs;                     // ZPair: the same for z
    float ex, ey, ez;              // zero padding: 1 - fx, 1 - fy, 1 - fz, exact
};

// 1 - f for the fraction f of a 32.32 fixed-point position, taken from the
// integer so that it keeps full relative precision when f is close to 1.  With
// zero padding a voxel next to the volume's edge is weighed against a zero
// voxel by 1 - f alone, and 1 - (f rounded to fp32) would carry up to 3e-8
// absolute error into values that can be 1e-3 of the image's maximum.
__device__ inline float fixed_comp(int64_t q)
{
    const uint32_t fr = (uint32_t)q;
    return fr ? (float)(0u - fr) * 2.3283064365386963e-10f : 1.0f;
}

// Byte offset past the end of any corner-cell copy (those stay below
// 0xffffff00 bytes): buffer loads there return zeros.
constexpr uint32_t kOutOfRange = 0xffffff00u;

// ZP (zero padding, Cell and ZPair layouts): a sample whose cell lies outside
// the copy's grid reads 0; the copy itself holds 0 for corners outside the
// volume.
template <typename T, Layout L, bool ZP = false>
__device__ inline SampleAddr sample_addr(const VolumeDesc& V, int64_t qx, int64_t qy, int64_t qz)
{
    SampleAddr A;
    const int ix = fixed_floor(qx), iy = fixed_floor(qy), iz = fixed_floor(qz);
    A.fx = fixed_frac(qx);
    A.fy = fixed_frac(qy);
    A.fz = fixed_frac(qz);
    A.gxs = 1.0f;
    A.gzs = 1.0f;
    if constexpr (L == Layout::ZPair && ZP) {
        // zero-padded z-pairs: element (ix + 1, iy + 1, iz + 1) of a copy with a
        // border of zeros (rows nx + 2 long, ny + 2 rows, nz + 1 slices); a
        // sample whose cell lies outside it reads past the buffer's end (both
        // rows), where loads return 0
        A.ex = fixed_comp(qx);
        A.ey = fixed_comp(qy);
        A.ez = fixed_comp(qz);
        const bool in = (uint32_t)(ix + 1) <= (uint32_t)V.n[0] &&
                        (uint32_t)(iy + 1) <= (uint32_t)V.n[1] &&
                        (uint32_t)(iz + 1) <= (uint32_t)V.n[2];
        A.o = in ? (uint32_t)(iz + 1) * V.slice_bytes + __umul24((uint32_t)(iy + 1), V.row_bytes) +
                       (uint32_t)(ix + 1) * (uint32_t)(2 * sizeof(T))
                 : kOutOfRange;
        A.dy = in ? V.row_bytes : 0u;
        A.dz = A.x1 = 0;
        return A;
    }
    if constexpr (L == Layout::ZPair) {
        // row and slice strides of the z-pair copy (V.row_bytes, V.slice_bytes)
        const int y0 = clampi(iy, 0, V.n[1] - 1), y1 = clampi(iy + 1, 0, V.n[1] - 1);
        const int xp = clampi(ix, 0, V.n[0] - 2), zp = clampi(iz, 0, V.n[2] - 2);
        A.fx = __builtin_amdgcn_fmed3f(A.fx + (float)(ix - xp), 0.0f, 1.0f);
        A.fz = __builtin_amdgcn_fmed3f(A.fz + (float)(iz - zp), 0.0f, 1.0f);
        A.gxs = ix == xp ? 1.0f : 0.0f;
        A.gzs = iz == zp ? 1.0f : 0.0f;
        A.o = (uint32_t)zp * V.slice_bytes + __umul24((uint32_t)y0, V.row_bytes) +
              (uint32_t)xp * (uint32_t)(2 * sizeof(T));
        A.dy = y1 > y0 ? V.row_bytes : 0u;
        A.dz = A.x1 = 0;
        return A;
    }
    if constexpr (L == Layout::Cell) {
        // a sample inside the box has -1 <= floor(q) <= n - 1; anything else
        // would fall outside the buffer range and read zeros, never fault
        A.o = (uint32_t)(iz + 1) * V.cell_slice_bytes +
              __umul24((uint32_t)(iy + 1), V.cell_row_bytes) + (uint32_t)(ix + 1) * (8 * sizeof(T));
        if constexpr (ZP) {
            A.ex = fixed_comp(qx);
            A.ey = fixed_comp(qy);
            A.ez = fixed_comp(qz);
            const bool in = (uint32_t)(ix + 1) <= (uint32_t)V.n[0] &&
                            (uint32_t)(iy + 1) <= (uint32_t)V.n[1] &&
                            (uint32_t)(iz + 1) <= (uint32_t)V.n[2];
            if (!in) A.o = kOutOfRange;
        }
        A.dy = A.dz = A.x1 = 0;
        return A;
    } else {
        // (the padded z-pair case returned above)
        static_assert(!ZP || L == Layout::ZPair,
                      "zero padding reads the corner-cell or padded z-pair copy");
    }
    const int y0 = clampi(iy, 0, V.n[1] - 1), y1 = clampi(iy + 1, 0, V.n[1] - 1);
    const int z0 = clampi(iz, 0, V.n[2] - 1), z1 = clampi(iz + 1, 0, V.n[2] - 1);
    const uint32_t r00 = (uint32_t)z0 * V.slice_bytes + __umul24((uint32_t)y0, V.row_bytes);
    A.dy = y1 > y0 ? V.row_bytes : 0u;
    A.dz = z1 > z0 ? V.slice_bytes : 0u;
    if constexpr (L == Layout::Pair) {
        const int xp = clampi(ix, 0, V.n[0] - 2);
        A.fx = __builtin_amdgcn_fmed3f(A.fx + (float)(ix - xp), 0.0f, 1.0f);
        A.gxs = ix == xp ? 1.0f : 0.0f;
        A.o = r00 + (uint32_t)xp * (uint32_t)sizeof(T);
        A.x1 = 0;
    } else {
        const int x0 = clampi(ix, 0, V.n[0] - 1), x1 = clampi(ix + 1, 0, V.n[0] - 1);
        A.o = r00 + (uint32_t)x0 * (uint32_t)sizeof(T);
        A.x1 = (uint32_t)(x1 - x0) * (uint32_t)sizeof(T);
    }
    return A;
}

// The eight corner values (x0, x1) of rows (y0,z0) (y1,z0) (y0,z1) (y1,z1).
struct CornerVals {
    float v[8];
};

template <typename T>
__device__ inline void load_cell(__amdgpu_buffer_rsrc_t rs, uint32_t off, CornerVals& c);

template <>
__device__ inline void load_cell<float>(__amdgpu_buffer_rsrc_t rs, uint32_t off, CornerVals& c)
{
    const auto a = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, 0);
    const auto b = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(off + 16), 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        c.v[i] = __uint_as_float(a[i]);
        c.v[4 + i] = __uint_as_float(b[i]);
    }
}

template <>
__device__ inline void load_cell<uint16_t>(__amdgpu_buffer_rsrc_t rs, uint32_t off, CornerVals& c)
{
    const auto a = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        c.v[2 * i] = bf16_lo(a[i]);
        c.v[2 * i + 1] = bf16_hi(a[i]);
    }
}

// One y row of the z-pair copy at byte offset `off`: corners (x0, x1) x (z0, z1)
// into c.v[base], c.v[base + 1] (z0) and c.v[base + 4], c.v[base + 5] (z1).
template <typename T>
__device__ inline void load_zpair_row(__amdgpu_buffer_rsrc_t rs, uint32_t off, CornerVals& c,
                                      int base);

template <>
__device__ inline void load_zpair_row<float>(__amdgpu_buffer_rsrc_t rs, uint32_t off,
                                             CornerVals& c, int base)
{
    const auto a = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, 0);
    c.v[base] = __uint_as_float(a[0]);
    c.v[base + 4] = __uint_as_float(a[1]);
    c.v[base + 1] = __uint_as_float(a[2]);
    c.v[base + 5] = __uint_as_float(a[3]);
}

template <>
__device__ inline void load_zpair_row<uint16_t>(__amdgpu_buffer_rsrc_t rs, uint32_t off,
                                                CornerVals& c, int base)
{
    const auto a = __builtin_amdgcn_raw_buffer_load_b64(rs, (int)off, 0, 0);
    c.v[base] = bf16_lo((uint32_t)a[0]);
    c.v[base + 4] = bf16_hi((uint32_t)a[0]);
    c.v[base + 1] = bf16_lo((uint32_t)a[1]);
    c.v[base + 5] = bf16_hi((uint32_t)a[1]);
}

template <typename T, Layout L>
__device__ inline void gather(__amdgpu_buffer_rsrc_t rs, const SampleAddr& A, CornerVals& c)
{
    if constexpr (L == Layout::Cell) {
        load_cell<T>(rs, A.o, c);
        return;
    }
    if constexpr (L == Layout::ZPair) {
        load_zpair_row<T>(rs, A.o, c, 0);
        load_zpair_row<T>(rs, A.o + A.dy, c, 2);
        return;
    }
    const uint32_t rows[4] = {A.o, A.o + A.dy, A.o + A.dz, A.o + A.dz + A.dy};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        if constexpr (L == Layout::Pair) {
            load_pair<T>(rs, rows[r], c.v[2 * r], c.v[2 * r + 1]);
        } else {
            c.v[2 * r] = load_one<T>(rs, rows[r]);
            c.v[2 * r + 1] = load_one<T>(rs, rows[r] + A.x1);
        }
    }
}

__device__ inline float interpolate(const SampleAddr& A, const CornerVals& c)
{
    const float c00 = fmaf(A.fx, c.v[1] - c.v[0], c.v[0]);
    const float c10 = fmaf(A.fx, c.v[3] - c.v[2], c.v[2]);
    const float c01 = fmaf(A.fx, c.v[5] - c.v[4], c.v[4]);
    const float c11 = fmaf(A.fx, c.v[7] - c.v[6], c.v[6]);
    const float c0 = fmaf(A.fy, c10 - c00, c00);
    const float c1 = fmaf(A.fy, c11 - c01, c01);
    return fmaf(A.fz, c1 - c0, c0);
}

// The same trilinear value as weighted sums with the exact complements (zero
// padding): every corner's weight keeps full relative precision.
__device__ inline float interpolate_exact(const SampleAddr& A, const CornerVals& c)
{
    const float c00 = fmaf(A.fx, c.v[1], A.ex * c.v[0]);
    const float c10 = fmaf(A.fx, c.v[3], A.ex * c.v[2]);
    const float c01 = fmaf(A.fx, c.v[5], A.ex * c.v[4]);
    const float c11 = fmaf(A.fx, c.v[7], A.ex * c.v[6]);
    const float c0 = fmaf(A.fy, c10, A.ey * c00);
    const float c1 = fmaf(A.fy, c11, A.ey * c01);
    return fmaf(A.fz, c1, A.ez * c0);
}

// Trilinear value and its gradient with respect to the continuous index q
// (per voxel); with clamped corners the differences along a clamped axis vanish.
__device__ inline float interpolate_grad(const SampleAddr& A, const CornerVals& c, float g[3])
{
    const float dx00 = c.v[1] - c.v[0], dx10 = c.v[3] - c.v[2];
    const float dx01 = c.v[5] - c.v[4], dx11 = c.v[7] - c.v[6];
    const float c00 = fmaf(A.fx, dx00, c.v[0]), c10 = fmaf(A.fx, dx10, c.v[2]);
    const float c01 = fmaf(A.fx, dx01, c.v[4]), c11 = fmaf(A.fx, dx11, c.v[6]);
    const float dy0 = c10 - c00, dy1 = c11 - c01;
    const float c0 = fmaf(A.fy, dy0, c00), c1 = fmaf(A.fy, dy1, c01);
    const float gx0 = fmaf(A.fy, dx10 - dx00, dx00), gx1 = fmaf(A.fy, dx11 - dx01, dx01);
    g[0] = A.gxs * fmaf(A.fz, gx1 - gx0, gx0);
    g[1] = fmaf(A.fz, dy1 - dy0, dy0);
    const float dz = c1 - c0;
    g[2] = A.gzs * dz;
    return fmaf(A.fz, dz, c0);
}

}  // namespace drr
