// drr_siddon.hpp -- the walk of one ray through the voxels of the
// cell-constant (Siddon) model, shared by its projector, its tile scatter and
// its brick-owned backward.
//
// diffct 2.1.0, "Why diffct" feature list: project() and backproject() form an
// exact adjoint pair for the cell-constant Siddon model: a ray's line integral
// is sum_v mu_v l_v with l_v the exact length of the clipped ray inside voxel v.
// The ray is C + t d (unit d, t in mm).  Axis a's voxel planes sit at
// p s_a - E_a / 2 for plane index p in [0, n_a] (voxel i between planes i and
// i + 1), crossed at t = p k_a + b_a with k_a = s_a / d_a and
// b_a = (-E_a / 2 - C_a) / d_a.  That fp64 expression (plane_crossing) is the
// only way any kernel evaluates a crossing, so all of them see the same ones.
#pragma once

#include "drr_brick.hpp"
#include "drr_device.hpp"

namespace drr {

// Walk state of one ray.  Axis a's next plane crossing is tn[a] =
// p[a] k[a] + b[a]; i is the current voxel.
struct SiddonRay {
    double C[3], d[3];
    double k[3], b[3];
    double t0, t1;
    double tn[3];
    int p[3], i[3], step[3];
};

__host__ __device__ inline double plane_crossing(const SiddonRay& S, int a, int p)
{
    return fma((double)p, S.k[a], S.b[a]);
}

// Ray through pixel (r, c) (unit direction as in ray_setup), clipped to the box
// by the same plane expression the walk uses: C, d, k, b, t0, t1 and the step
// of each axis (0 for an axis the ray runs parallel to).  False on a miss.
__host__ __device__ inline bool siddon_clip(const ViewGeom& G, const VolumeDesc& V, int r,
                                            int c, SiddonRay& S)
{
    const double u = (double)c + 0.5, v = (double)r + 0.5;
    double w[3];
#pragma unroll
    for (int a = 0; a < 3; ++a) w[a] = G.M[a * 3 + 0] * u + G.M[a * 3 + 1] * v + G.M[a * 3 + 2];
    const double inv_len = 1.0 / sqrt(w[0] * w[0] + w[1] * w[1] + w[2] * w[2]);
    double t_entry = -__builtin_inf(), t_exit = __builtin_inf();
    bool inside = true;
#pragma unroll
    for (int a = 0; a < 3; ++a) {
        S.C[a] = G.C[a];
        S.d[a] = w[a] * inv_len;
        if (S.d[a] == 0.0) {
            S.k[a] = 0.0;
            S.b[a] = __builtin_inf();
            S.step[a] = 0;
            inside = inside && !(G.C[a] < -V.half_e[a] || G.C[a] > V.half_e[a]);
        } else {
            const double inv = 1.0 / S.d[a];
            S.k[a] = V.s[a] * inv;
            S.b[a] = (-V.half_e[a] - G.C[a]) * inv;
            S.step[a] = S.d[a] > 0.0 ? 1 : -1;
            const double t_lo = S.b[a];
            const double t_hi = plane_crossing(S, a, V.n[a]);
            t_entry = fmax(t_entry, fmin(t_lo, t_hi));
            t_exit = fmin(t_exit, fmax(t_lo, t_hi));
        }
    }
    S.t0 = fmax(t_entry, 0.0);
    S.t1 = t_exit;
    return inside && S.t1 > S.t0;
}

// Axis a's index of the voxel holding the ray's point at t, clamped to
// [lo, hi] (so a point on a face belongs to the boundary voxel).
__host__ __device__ inline int siddon_voxel_at(const SiddonRay& S, const VolumeDesc& V, int a,
                                               double t, int lo, int hi)
{
    const double ua = (S.C[a] + t * S.d[a] + V.half_e[a]) * V.inv_s[a];
    return (int)fmin(fmax(floor(ua), (double)lo), (double)hi);
}

// siddon_clip and the walk's start: the voxel holding the entry point and each
// axis' first crossing ahead.
__host__ __device__ inline bool siddon_setup(const ViewGeom& G, const VolumeDesc& V, int r,
                                             int c, SiddonRay& S)
{
    if (!siddon_clip(G, V, r, c, S)) return false;
#pragma unroll
    for (int a = 0; a < 3; ++a) {
        S.i[a] = siddon_voxel_at(S, V, a, S.t0, 0, V.n[a] - 1);
        S.p[a] = S.step[a] > 0 ? S.i[a] + 1 : S.i[a];
        S.tn[a] = S.step[a] != 0 ? plane_crossing(S, a, S.p[a]) : __builtin_inf();
        if (S.step[a] == 0) S.p[a] = 0;
    }
    return true;
}

// The axis whose crossing comes first (x before y before z on ties).
struct NextAxis {
    bool x, y;          // z when neither
    double t;
};

__host__ __device__ inline NextAxis next_axis(const SiddonRay& S)
{
    NextAxis m;
    m.x = S.tn[0] <= S.tn[1] && S.tn[0] <= S.tn[2];
    m.y = !m.x && S.tn[1] <= S.tn[2];
    m.t = m.x ? S.tn[0] : (m.y ? S.tn[1] : S.tn[2]);
    return m;
}

// Cross the plane of the chosen axis: the voxel index and that axis' next
// crossing move on.  Returns false when the walk leaves the volume.
__host__ __device__ inline bool advance(SiddonRay& S, const NextAxis& m, const VolumeDesc& V)
{
    const bool z = !m.x && !m.y;
    const bool sel[3] = {m.x, m.y, z};
    bool in = true;
#pragma unroll
    for (int a = 0; a < 3; ++a) {
        if (sel[a]) {
            S.i[a] += S.step[a];
            S.p[a] += S.step[a];
            S.tn[a] = plane_crossing(S, a, S.p[a]);
            in = (unsigned)S.i[a] < (unsigned)V.n[a];
        }
    }
    return in;
}

// ------------------------------------------------ the walk inside a brick
//
// For the brick-owned backward (drr_brick.hip): the pieces of a ray inside one
// brick of voxels [lo, lo + e) per axis.  The walk starts at t_in, the later of
// the ray's entry into the volume and into the brick's box, in the voxel past
// every plane crossed at or before t_in, and ends at t_out; all crossings come
// from plane_crossing, so these are the forward's pieces between the same
// crossings, and every piece of positive length falls in exactly one brick.
// Host and device: the CPU checks replay them against the whole walk.

// The brick's voxel box as world coordinates of its bounding planes.
__host__ __device__ inline BrickRegion siddon_brick_region(const VolumeDesc& V, const BrickBox& b)
{
    BrickRegion g;
#pragma unroll
    for (int a = 0; a < 3; ++a) {
        g.lo[a] = (float)((double)b.lo[a] * V.s[a] - V.half_e[a]);
        g.hi[a] = (float)((double)(b.lo[a] + b.e[a]) * V.s[a] - V.half_e[a]);
    }
    return g;
}

// The ray's range [t_in, t_out) inside the brick's box (and the volume's);
// false when it has none.  An axis the ray runs parallel to keeps the voxel
// the forward's walk gives it (the one holding the entry point).
__host__ __device__ inline bool siddon_brick_range(SiddonRay& S, const VolumeDesc& V,
                                                   const BrickBox& b, double& t_in,
                                                   double& t_out)
{
    t_in = S.t0;
    t_out = S.t1;
#pragma unroll
    for (int a = 0; a < 3; ++a) {
        if (S.step[a] == 0) {
            S.i[a] = siddon_voxel_at(S, V, a, S.t0, 0, V.n[a] - 1);
            if (S.i[a] < b.lo[a] || S.i[a] >= b.lo[a] + b.e[a]) return false;
        } else {
            const double tl = plane_crossing(S, a, b.lo[a]);
            const double th = plane_crossing(S, a, b.lo[a] + b.e[a]);
            t_in = fmax(t_in, fmin(tl, th));
            t_out = fmin(t_out, fmax(tl, th));
        }
    }
    return t_out > t_in;
}

// The walk's state at t_in: on each axis the voxel past every plane crossed at
// or before t_in, and the next plane ahead (none, at infinity, for an axis the
// ray runs parallel to: its voxel is siddon_brick_range's).  The voxel holding
// the point at t_in is off by at most one from that (the point and the
// crossings round differently only within a few ulps of a plane), so one test
// of the planes on either side settles it.
__host__ __device__ inline void siddon_brick_start(SiddonRay& S, const VolumeDesc& V,
                                                   const BrickBox& b, double t_in)
{
#pragma unroll
    for (int a = 0; a < 3; ++a) {
        if (S.step[a] == 0) {
            S.p[a] = 0;
            S.tn[a] = __builtin_inf();
            continue;
        }
        const int lo = b.lo[a], hi = b.lo[a] + b.e[a] - 1;
        int i = siddon_voxel_at(S, V, a, t_in, lo, hi);
        const bool below = plane_crossing(S, a, i) <= t_in;       // plane i crossed
        const bool above = plane_crossing(S, a, i + 1) <= t_in;   // plane i + 1 crossed
        if (S.step[a] > 0) {
            i += (above && i < hi) ? 1 : ((!below && i > lo) ? -1 : 0);
            S.p[a] = i + 1;
        } else {
            i += (below && i > lo) ? -1 : ((!above && i < hi) ? 1 : 0);
            S.p[a] = i;
        }
        S.i[a] = i;
        S.tn[a] = plane_crossing(S, a, S.p[a]);
    }
}

// Walks ray S from t_in to t_out through the brick, handing each piece (its
// voxel's entry in the brick copy, its length; zero for a tie of crossings,
// which adds nothing) to `add`.  Every crossing before t_out is of a plane
// inside the brick (t_out is at or before each axis' exit plane, and the
// crossings of one axis come in plane order), so the voxel stays in the brick;
// the walk takes no branch per piece: all three next crossings are made and
// the nearest one's kept.
template <int B, typename Add>
__host__ __device__ inline void siddon_brick_walk(const SiddonRay& S, const BrickBox& b,
                                                  double t_in, double t_out, Add add)
{
    double tn0 = S.tn[0], tn1 = S.tn[1], tn2 = S.tn[2];
    int p0 = S.p[0], p1 = S.p[1], p2 = S.p[2];
    int e = (S.i[0] - b.lo[0]) + B * ((S.i[1] - b.lo[1]) + B * (S.i[2] - b.lo[2]));
    const int ex = S.step[0], ey = B * S.step[1], ez = B * B * S.step[2];
    double tc = t_in;
    int guard = b.e[0] + b.e[1] + b.e[2] + 3;
    for (;;) {
        // the nearest crossing, x before y before z on ties (as the forward)
        const bool sx = tn0 <= tn1 && tn0 <= tn2;
        const bool sy = !sx && tn1 <= tn2;
        const double mt = sx ? tn0 : (sy ? tn1 : tn2);
        const double te = mt < t_out ? mt : t_out;
        const double len = te - tc;
        add(e, len > 0.0 ? len : 0.0);
        tc = te > tc ? te : tc;
        if (!(mt < t_out) || --guard <= 0) break;
        const int q0 = p0 + S.step[0], q1 = p1 + S.step[1], q2 = p2 + S.step[2];
        const double n0 = plane_crossing(S, 0, q0), n1 = plane_crossing(S, 1, q1);
        const double n2 = plane_crossing(S, 2, q2);
        const bool sz = !sx && !sy;
        p0 = sx ? q0 : p0;
        p1 = sy ? q1 : p1;
        p2 = sz ? q2 : p2;
        tn0 = sx ? n0 : tn0;
        tn1 = sy ? n1 : tn1;
        tn2 = sz ? n2 : tn2;
        e += sx ? ex : (sy ? ey : ez);
    }
}

}  // namespace drr
