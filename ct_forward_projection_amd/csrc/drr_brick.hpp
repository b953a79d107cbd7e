// drr_brick.hpp -- index arithmetic of the brick-owned volume backward:
// which cells a brick's samples lie in, which detector pixels can reach them,
// which samples of a ray do, and where a sample's corners sit in the brick's
// LDS copy.  Every function is __host__ __device__ so a CPU build can replay
// the same arithmetic with bounds checks (tests/cpu_checks).
//
// Method (source pages): flashdrr.rendering VolumeRaycaster class text --
// rendering is differentiable with respect to the volume; diffct 2.1.0
// Quickstart -- backproject() applies the matched adjoint A^T, i.e. every
// sample of every ray adds y dz w_corner to its eight trilinear corners.
//
// The gradient is split into bricks of at most B x B x B voxels, and one
// workgroup owns each brick: it adds, in LDS, every sample whose trilinear
// cell touches one of its voxels, then writes its voxels once (no global
// atomics, no zero fill).  A sample whose continuous index lies in
// [lo - 1, lo + e) on every axis (lo the brick's first voxel, e its extent)
// has its cell in [lo - 1, lo + e - 1] and its corners in [lo - 1, lo + e];
// the LDS copy holds those e + 2 voxels per axis (a one-voxel apron).  Apron
// entries at -1 or n stand for the clamped edge voxel (clamp to edge) and are
// folded into it before the brick is written; other apron entries belong to
// the neighbouring brick, which adds the same samples itself.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace drr {

// One ray of the backward, as the ray-record pass writes it (64 bytes): the
// forward's fixed-point start and step (bit-identical sample positions), the
// coefficient c = y dz every sample adds (times its weights), and |c| m with
// m the most samples the ray can put in one cell, which bounds what one cell's
// register sum can reach.  n = 0 marks a ray that adds nothing (a miss, or
// c = 0).
struct RayRecord {
    int64_t q0[3];
    int64_t dq[3];
    float coef;
    int n;
    float cell_bound;
    int pad;
};
static_assert(sizeof(RayRecord) == 64, "ray records are 64 bytes");

// Samples one ray can put in one cell: consecutive samples advance by |dq|_inf
// voxels along some axis, so at most floor(1 / |dq|_inf) + 1 share a cell.
__host__ __device__ inline int samples_per_cell_bound(const int64_t dq[3], int N)
{
    int64_t m = 0;
    for (int a = 0; a < 3; ++a) {
        const int64_t v = dq[a] < 0 ? -dq[a] : dq[a];
        m = v > m ? v : m;
    }
    if (m == 0) return N;
    const int64_t per = ((int64_t)1 << 32) / m + 1;
    return per < (int64_t)N ? (int)per : N;
}

// The brick of index (bx, by, bz): first voxel lo and extent e (<= B) per axis.
struct BrickBox {
    int lo[3];
    int e[3];
};

__host__ __device__ inline BrickBox brick_box(const int n[3], int B, int bx, int by, int bz)
{
    BrickBox b;
    const int idx[3] = {bx, by, bz};
    for (int a = 0; a < 3; ++a) {
        b.lo[a] = idx[a] * B;
        const int rest = n[a] - b.lo[a];
        b.e[a] = rest < B ? rest : B;
    }
    return b;
}

// Pitch of a brick's LDS copy along each axis (B + 2: the apron on both sides).
__host__ __device__ constexpr int brick_pitch(int B) { return B + 2; }

// LDS entry of copy coordinates (x, y, z), each in [0, e + 1] (voxel lo - 1 + x).
__host__ __device__ inline int brick_entry(int B, int x, int y, int z)
{
    const int P = brick_pitch(B);
    return x + P * (y + P * z);
}

// LDS entry of the cell (x, y, z) in copy coordinates (its low corner), the
// first of its eight corner entries.
__host__ __device__ inline int brick_cell_entry(int B, int x, int y, int z)
{
    return brick_entry(B, x, y, z);
}

// Offset of corner n (bit 0: x + 1, bit 1: y + 1, bit 2: z + 1) from its
// cell's entry.
__host__ __device__ inline int brick_corner_offset(int B, int n)
{
    const int P = brick_pitch(B);
    return (n & 1) + P * ((n >> 1) & 1) + P * P * (n >> 2);
}

// Folding the apron along axis a (clamp to edge): line i in [0, P^2) of the
// copy runs along axis a through the entries base + j step, j in [0, P), with
// the other two coordinates (u, w) = (i % P, i / P).  At the volume's low face
// entry j = 0 (voxel -1) adds into j = 1 (voxel 0); at its high face entry
// j = e + 1 (voxel n) adds into j = e (voxel n - 1).
__host__ __device__ inline int brick_line_base(int B, int a, int i, int& step)
{
    const int P = brick_pitch(B);
    const int u = i % P, w = i / P;
    if (a == 0) {
        step = 1;
        return P * (u + P * w);
    }
    if (a == 1) {
        step = P;
        return u + P * P * w;
    }
    step = P * P;
    return u + P * w;
}

// Detector pixels whose rays can carry a sample into the brick's cells, as an
// inclusive rectangle [r0, r1] x [c0, c1] (empty when r1 < r0 or c1 < c0).
// The region those samples lie in is the box of continuous indices
// [lo - 1, lo + e) per axis, cut to the volume [-1/2, n - 1/2]; a ray through
// pixel centre (c + 1/2, r + 1/2) meets it only if that centre lies in the
// region's projection, inside the bounding rectangle of its eight projected
// corners.  A sample at distance t on the ray through image point
// m = (u, v, 1) projects to P X = t m / |K^-1 m|, whose third component is
// > 0: a region with no corner in front of the camera ((P X)_2 > 0) is
// unreachable (empty rectangle).  The projection runs in fp32 (its rounding
// is a few 1e-7 of the coordinates): the rectangle is widened by 1/16 pixel
// plus 2^-12 of the largest projected coordinate, and a region with a corner
// at or behind the camera plane, or nearer to it than 2^-10 of the farthest
// corner's depth, gets the whole detector.
//   P: K [R | t] as 3 x 4 (fp32); g: the region (brick_region).
struct PixelRect {
    int r0, r1, c0, c1;
};

// The brick region in world coordinates (mm): continuous indices
// [lo - 1, lo + e) per axis cut to [-1/2, n - 1/2], at (q - q_off) s.
struct BrickRegion {
    float lo[3], hi[3];
};

__host__ __device__ inline BrickRegion brick_region(const int n[3], const double s[3],
                                                    const double q_off[3], const BrickBox& b)
{
    BrickRegion g;
    for (int a = 0; a < 3; ++a) {
        const double ql = fmax((double)(b.lo[a] - 1), -0.5);
        const double qh = fmin((double)(b.lo[a] + b.e[a]), (double)n[a] - 0.5);
        g.lo[a] = (float)((ql - q_off[a]) * s[a]);
        g.hi[a] = (float)((qh - q_off[a]) * s[a]);
    }
    return g;
}

__host__ __device__ inline PixelRect brick_pixel_rect(const float P[12], const BrickRegion& g,
                                                      int H, int W)
{
    PixelRect R{0, H - 1, 0, W - 1};
    const float* lo = g.lo;
    const float* hi = g.hi;
    float umin = 3e38f, umax = -3e38f, vmin = 3e38f, vmax = -3e38f;
    float wmin = 3e38f, wmax = -3e38f;
    for (int k = 0; k < 8; ++k) {
        const float x = (k & 1) ? hi[0] : lo[0];
        const float y = (k & 2) ? hi[1] : lo[1];
        const float z = (k & 4) ? hi[2] : lo[2];
        const float w = P[8] * x + P[9] * y + P[10] * z + P[11];
        const float iw = 1.0f / w;
        const float u = (P[0] * x + P[1] * y + P[2] * z + P[3]) * iw;
        const float v = (P[4] * x + P[5] * y + P[6] * z + P[7]) * iw;
        wmin = fminf(wmin, w); wmax = fmaxf(wmax, w);
        umin = fminf(umin, u); umax = fmaxf(umax, u);
        vmin = fminf(vmin, v); vmax = fmaxf(vmax, v);
    }
    if (!(wmax > 0.0f)) {                         // behind the camera: no ray reaches it
        R.r1 = R.r0 - 1;
        R.c1 = R.c0 - 1;
        return R;
    }
    if (!(wmin > wmax * 0.0009765625f)) return R; // at or near the camera plane
    const float big = fmaxf(fmaxf(fabsf(umin), fabsf(umax)), fmaxf(fabsf(vmin), fabsf(vmax)));
    const float m = 0.0625f + big * 0.000244140625f;
    if (!(big < 1e9f)) return R;
    // pixel centres c + 1/2 in [umin - m, umax + m]
    const float c0 = ceilf(umin - m - 0.5f), c1 = floorf(umax + m - 0.5f);
    const float r0 = ceilf(vmin - m - 0.5f), r1 = floorf(vmax + m - 0.5f);
    R.c0 = (int)fmaxf(c0, 0.0f);
    R.c1 = (int)fminf(c1, (float)(W - 1));
    R.r0 = (int)fmaxf(r0, 0.0f);
    R.r1 = (int)fminf(r1, (float)(H - 1));
    if (c1 < 0.0f || c0 > (float)(W - 1)) R.c1 = R.c0 - 1;
    if (r1 < 0.0f || r0 > (float)(H - 1)) R.r1 = R.r0 - 1;
    return R;
}

// What the brick kernel needs of a view: its projection K [R | t] as 3 x 4,
// fp32 (from the fp64 camera).
struct BrickView {
    float P[12];
};

// The region's eight corners projected into the image, for the per-row spans
// below: u, v of corner k (x, y, z bits as in brick_pixel_rect) and that
// function's margin m.  `narrow` when every corner lies in front of the
// camera (depth above 2^-10 of the farthest): the region's projection is then
// the convex hull of the projected corners (a perspective projection keeps a
// convex set in front of the camera convex).  Otherwise the caller uses whole
// rows of the rectangle.
struct BrickHull {
    float u[8], v[8];
    float m;
    bool narrow;
};

__host__ __device__ inline BrickHull brick_hull(const float P[12], const BrickRegion& g)
{
    BrickHull h;
    float wmin = 3e38f, wmax = -3e38f, big = 0.0f;
    for (int k = 0; k < 8; ++k) {
        const float x = (k & 1) ? g.hi[0] : g.lo[0];
        const float y = (k & 2) ? g.hi[1] : g.lo[1];
        const float z = (k & 4) ? g.hi[2] : g.lo[2];
        const float w = P[8] * x + P[9] * y + P[10] * z + P[11];
        const float iw = 1.0f / w;
        h.u[k] = (P[0] * x + P[1] * y + P[2] * z + P[3]) * iw;
        h.v[k] = (P[4] * x + P[5] * y + P[6] * z + P[7]) * iw;
        wmin = fminf(wmin, w);
        wmax = fmaxf(wmax, w);
        big = fmaxf(big, fmaxf(fabsf(h.u[k]), fabsf(h.v[k])));
    }
    h.m = 0.0625f + big * 0.000244140625f;
    h.narrow = wmax > 0.0f && wmin > wmax * 0.0009765625f && big < 1e9f;
    return h;
}

// Columns [c0, c1] of detector row r whose pixel centres can lie in the
// region's projection: the hull's extent along the row over the band
// |v - (r + 1/2)| <= m (its corners inside the band and the crossings of the
// band's two edges with the twelve projected box edges -- the hull's outline
// runs along some of them), widened by m and cut to [c_lo, c_hi].  A hull
// that does not touch the band gives c1 < c0; one that is not narrow gives
// [c_lo, c_hi].  Crossings are clamped between their edge's end points, so a
// nearly horizontal edge cannot throw one far off.
__host__ __device__ inline void brick_row_span(const BrickHull& h, int r, int c_lo, int c_hi,
                                               int& c0, int& c1)
{
    c0 = c_lo;
    c1 = c_hi;
    if (!h.narrow) return;
    const float vc = (float)r + 0.5f, b0 = vc - h.m, b1 = vc + h.m;
    float umin = 3e38f, umax = -3e38f;
    for (int k = 0; k < 8; ++k) {
        if (h.v[k] >= b0 && h.v[k] <= b1) {
            umin = fminf(umin, h.u[k]);
            umax = fmaxf(umax, h.u[k]);
        }
    }
    for (int a = 0; a < 3; ++a) {
        const int bit = 1 << a;
        for (int k = 0; k < 8; ++k) {
            if (k & bit) continue;
            const int l = k | bit;                     // the edge (k, l) along axis a
            const float va = h.v[k], vb = h.v[l], ua = h.u[k], ub = h.u[l];
            for (int e = 0; e < 2; ++e) {
                const float yb = e ? b1 : b0;
                if ((va - yb) * (vb - yb) < 0.0f) {
                    const float x = ua + (yb - va) * (ub - ua) / (vb - va);
                    const float xc = fminf(fmaxf(x, fminf(ua, ub)), fmaxf(ua, ub));
                    umin = fminf(umin, xc);
                    umax = fmaxf(umax, xc);
                }
            }
        }
    }
    if (!(umin <= umax)) {
        c1 = c0 - 1;
        return;
    }
    const float f0 = ceilf(umin - h.m - 0.5f), f1 = floorf(umax + h.m - 0.5f);
    if (f1 < (float)c_lo || f0 > (float)c_hi) {
        c1 = c0 - 1;
        return;
    }
    c0 = f0 > (float)c_lo ? (int)f0 : c_lo;
    c1 = f1 < (float)c_hi ? (int)f1 : c_hi;
}

// fp32 value of a 64-bit integer from its two words: the high word's
// conversion carries the scale 2^32, the low word's is exact to 2^-24
// relative, so the result is within 2^-23 of x relative.
__host__ __device__ inline float int64_to_float(int64_t x)
{
    return (float)(int32_t)(x >> 32) * 4294967296.0f + (float)(uint32_t)(x & 0xffffffffu);
}

// A range [k_lo, k_hi) of a ray's samples that contains every sample whose
// continuous index lies in the brick region [lo - 1, lo + e) on every axis (it
// may hold a few more).  The bounds are estimated in fp32 from the exact
// fixed-point differences to the region's faces and widened by one sample
// plus 2^-20 of their size, which covers the fp32 rounding of the estimate
// (relative error below 2^-21) for any n <= 2^24.
__host__ __device__ inline void brick_sample_range(const RayRecord& r, const BrickBox& b,
                                                   int& k_lo, int& k_hi)
{
    float lo = 0.0f, hi = (float)r.n;
    bool none = false;
    for (int a = 0; a < 3; ++a) {
        const int64_t L = (int64_t)(b.lo[a] - 1) * ((int64_t)1 << 32);
        const int64_t U = (int64_t)(b.lo[a] + b.e[a]) * ((int64_t)1 << 32);
        const int64_t d = r.dq[a];
        if (d == 0) {
            none = none || r.q0[a] < L || r.q0[a] >= U;
        } else {
            const float inv = 1.0f / int64_to_float(d);
            const float k0 = int64_to_float(L - r.q0[a]) * inv;
            const float k1 = int64_to_float(U - r.q0[a]) * inv;
            lo = fmaxf(lo, fminf(k0, k1));
            hi = fminf(hi, fmaxf(k0, k1));
        }
    }
    if (none || !(hi >= lo - 4.0f)) {
        k_lo = k_hi = 0;
        return;
    }
    const float wl = 1.0f + fabsf(lo) * 9.5367431640625e-07f;   // 2^-20
    const float wh = 1.0f + fabsf(hi) * 9.5367431640625e-07f;
    const float fl = floorf(lo - wl), fh = ceilf(hi + wh);
    k_lo = fl <= 0.0f ? 0 : (fl >= (float)r.n ? r.n : (int)fl);
    k_hi = fh <= 0.0f ? 0 : (fh >= (float)r.n ? r.n : (int)fh);
    if (k_hi < k_lo) k_hi = k_lo;
}

// Whether a position relative to the brick copy's origin (voxel lo - 1 at 0,
// fixed point) lies in a cell of the region: [0, e] on every axis.
__host__ __device__ inline bool brick_rel_inside(const int64_t q[3], const BrickBox& b)
{
    bool in = true;
    for (int a = 0; a < 3; ++a) in = in && (uint32_t)(int32_t)(q[a] >> 32) <= (uint32_t)b.e[a];
    return in;
}

// Whether sample k of the ray lies in the brick region: its cell, in copy
// coordinates (voxel lo - 1 at 0), in [0, e] on every axis.
__host__ __device__ inline bool brick_sample_inside(const RayRecord& r, const BrickBox& b, int k)
{
    int64_t q[3];
    for (int a = 0; a < 3; ++a)
        q[a] = r.q0[a] + (int64_t)k * r.dq[a] - (int64_t)(b.lo[a] - 1) * ((int64_t)1 << 32);
    return brick_rel_inside(q, b);
}

// The exact range [k_lo, k_hi) of the ray's samples in the brick region, and
// the position of sample k_lo relative to the copy's origin (q_rel): the
// estimate of brick_sample_range shrunk at both ends by the exact cell test,
// stepping the fixed-point position by dq.  Positions are linear in k and the
// region is a box, so the samples inside it are one run: every sample of the
// result is inside, and no other sample is.
__host__ __device__ inline void brick_exact_range(const RayRecord& r, const BrickBox& b, int& k_lo,
                                                  int& k_hi, int64_t q_rel[3])
{
    brick_sample_range(r, b, k_lo, k_hi);
    if (k_lo >= k_hi) return;
    int64_t* q = q_rel;
    for (int a = 0; a < 3; ++a)
        q[a] = r.q0[a] - (int64_t)(b.lo[a] - 1) * ((int64_t)1 << 32) + (int64_t)k_lo * r.dq[a];
    while (k_lo < k_hi && !brick_rel_inside(q, b)) {
        ++k_lo;
        for (int a = 0; a < 3; ++a) q[a] += r.dq[a];
    }
    if (k_lo >= k_hi) return;
    int64_t qe[3];
    for (int a = 0; a < 3; ++a) qe[a] = q[a] + (int64_t)(k_hi - 1 - k_lo) * r.dq[a];
    while (k_hi > k_lo && !brick_rel_inside(qe, b)) {
        --k_hi;
        for (int a = 0; a < 3; ++a) qe[a] -= r.dq[a];
    }
}

}  // namespace drr
