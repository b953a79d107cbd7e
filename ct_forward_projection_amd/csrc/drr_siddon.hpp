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

__device__ inline double plane_crossing(const SiddonRay& S, int a, int p)
{
    return fma((double)p, S.k[a], S.b[a]);
}

// Ray through pixel (r, c) (unit direction as in ray_setup), clipped to the box
// by the same plane expression the walk uses: C, d, k, b, t0, t1 and the step
// of each axis (0 for an axis the ray runs parallel to).  False on a miss.
__device__ inline bool siddon_clip(const ViewGeom& G, const VolumeDesc& V, int r, int c,
                                   SiddonRay& S)
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
__device__ inline int siddon_voxel_at(const SiddonRay& S, const VolumeDesc& V, int a, double t,
                                      int lo, int hi)
{
    const double ua = (S.C[a] + t * S.d[a] + V.half_e[a]) * V.inv_s[a];
    return (int)fmin(fmax(floor(ua), (double)lo), (double)hi);
}

// siddon_clip and the walk's start: the voxel holding the entry point and each
// axis' first crossing ahead.
__device__ inline bool siddon_setup(const ViewGeom& G, const VolumeDesc& V, int r, int c,
                                    SiddonRay& S)
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

__device__ inline NextAxis next_axis(const SiddonRay& S)
{
    NextAxis m;
    m.x = S.tn[0] <= S.tn[1] && S.tn[0] <= S.tn[2];
    m.y = !m.x && S.tn[1] <= S.tn[2];
    m.t = m.x ? S.tn[0] : (m.y ? S.tn[1] : S.tn[2]);
    return m;
}

// Cross the plane of the chosen axis: the voxel index and that axis' next
// crossing move on.  Returns false when the walk leaves the volume.
__device__ inline bool advance(SiddonRay& S, const NextAxis& m, const VolumeDesc& V)
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

}  // namespace drr
