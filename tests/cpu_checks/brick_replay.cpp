// CPU replay of the brick-owned backward's index arithmetic (the library's
// drr_brick.hpp, compiled for the host), on pinhole cameras of its own:
//   - every sample whose cell touches a brick comes from a pixel inside
//     brick_pixel_rect and inside its row's brick_row_span, and a sample index
//     inside brick_sample_range;
//   - every corner the kernel adds lands inside the brick's LDS copy;
//   - the brick copies, folded at the volume faces (clamp to edge) and read
//     back at their own voxels, equal a direct scatter of every sample to its
//     eight clamped corners (fp64 both ways).
// Exit status 0 when every check holds; the first failure is printed.
//
// The rays come from this file's own fp64 camera: direction R^T K^-1
// (c + 1/2, r + 1/2, 1) normalised, slab clip to the box, N midpoint samples,
// positions as 32.32 fixed-point continuous voxel indices -- the arithmetic
// the library's ray setup performs, restated so the replay stands alone.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <random>
#include <vector>

#include "../../ct_forward_projection_amd/csrc/drr_brick.hpp"

using drr::BrickBox;
using drr::PixelRect;
using drr::RayRecord;

static int g_fail = 0;
#define CHECK(cond, ...)                                             \
    do {                                                             \
        if (!(cond)) {                                               \
            if (g_fail++ < 5) {                                      \
                fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
                fprintf(stderr, __VA_ARGS__);                        \
                fprintf(stderr, "\n");                               \
            }                                                        \
        }                                                            \
    } while (0)

struct Case {
    int n[3];          // nx, ny, nz
    double s[3];       // spacing
    int H, W, N, views, B;
    double dist, fov_scale, rot;
    bool inside;       // cameras near the centre (inside the box)
    unsigned seed;
};

static void mat3_mul(const double A[9], const double B[9], double C[9])
{
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 3; ++j)
            C[i * 3 + j] = A[i * 3] * B[j] + A[i * 3 + 1] * B[3 + j] + A[i * 3 + 2] * B[6 + j];
}

static void rot_xyz(double ax, double ay, double az, double R[9])
{
    const double cx = cos(ax), sx = sin(ax), cy = cos(ay), sy = sin(ay);
    const double cz = cos(az), sz = sin(az);
    const double Rx[9] = {1, 0, 0, 0, cx, -sx, 0, sx, cx};
    const double Ry[9] = {cy, 0, sy, 0, 1, 0, -sy, 0, cy};
    const double Rz[9] = {cz, -sz, 0, sz, cz, 0, 0, 0, 1};
    double T[9];
    mat3_mul(Rz, Ry, T);
    mat3_mul(T, Rx, R);
}

static int64_t to_fixed(double x) { return (int64_t)llrint(x * 4294967296.0); }

int run_case(const Case& cs)
{
    std::mt19937_64 rng(cs.seed);
    std::uniform_real_distribution<double> U(-1.0, 1.0);
    const int nx = cs.n[0], ny = cs.n[1], nz = cs.n[2];
    double half[3], q_off[3];
    for (int a = 0; a < 3; ++a) {
        half[a] = 0.5 * cs.n[a] * cs.s[a];
        q_off[a] = 0.5 * (cs.n[a] - 1);
    }
    const double ext = fmax(fmax(2 * half[0], 2 * half[1]), 2 * half[2]);
    const double f = cs.fov_scale * fmax(cs.H, cs.W) * cs.dist / ext;
    const double K[9] = {f, 0, 0.5 * cs.W + 0.3, 0, f, 0.5 * cs.H - 0.2, 0, 0, 1};
    const double Ki[9] = {1 / f, 0, -K[2] / f, 0, 1 / f, -K[5] / f, 0, 0, 1};
    const size_t n_vox = (size_t)nx * ny * nz;
    std::vector<double> direct(n_vox, 0.0), bricked(n_vox, 0.0);
    long long n_samples_total = 0, n_candidates = 0, n_rejected = 0;

    for (int v = 0; v < cs.views; ++v) {
        // camera-to-world rotation Rc, centre C; world-to-camera R = Rc^T, t = -R C
        double Rc[9];
        rot_xyz(cs.rot * U(rng), cs.rot * U(rng), cs.rot * U(rng), Rc);
        double C[3];
        const double back[3] = {0, 0, cs.inside ? 0.0 : -cs.dist};
        for (int a = 0; a < 3; ++a)
            C[a] = Rc[a * 3] * back[0] + Rc[a * 3 + 1] * back[1] + Rc[a * 3 + 2] * back[2] +
                   (cs.inside ? 0.3 * half[a] * U(rng) : 0.05 * ext * U(rng));
        double R[9], t[3];
        for (int i = 0; i < 3; ++i)
            for (int j = 0; j < 3; ++j) R[i * 3 + j] = Rc[j * 3 + i];
        for (int i = 0; i < 3; ++i) t[i] = -(R[i * 3] * C[0] + R[i * 3 + 1] * C[1] + R[i * 3 + 2] * C[2]);
        // P = K [R | t] in fp32 from the fp32 K and pose the library receives
        float Kf[9], Rf[9], tf[3], Pm[12];
        for (int i = 0; i < 9; ++i) Kf[i] = (float)K[i];
        for (int i = 0; i < 9; ++i) Rf[i] = (float)R[i];
        for (int i = 0; i < 3; ++i) tf[i] = (float)t[i];
        for (int i = 0; i < 3; ++i)
            for (int j = 0; j < 4; ++j)
                Pm[i * 4 + j] = Kf[i * 3] * (j < 3 ? Rf[j] : tf[0]) +
                                Kf[i * 3 + 1] * (j < 3 ? Rf[3 + j] : tf[1]) +
                                Kf[i * 3 + 2] * (j < 3 ? Rf[6 + j] : tf[2]);
        // M = R^T K^-1
        double M[9];
        for (int a = 0; a < 3; ++a)
            for (int b = 0; b < 3; ++b)
                M[a * 3 + b] = R[a] * Ki[b] + R[3 + a] * Ki[3 + b] + R[6 + a] * Ki[6 + b];


        // ray records of the view
        std::vector<RayRecord> rec((size_t)cs.H * cs.W);
        for (int r = 0; r < cs.H; ++r)
            for (int c = 0; c < cs.W; ++c) {
                RayRecord& o = rec[(size_t)r * cs.W + c];
                o = RayRecord{};
                double d[3];
                for (int a = 0; a < 3; ++a) d[a] = M[a * 3] * (c + 0.5) + M[a * 3 + 1] * (r + 0.5) + M[a * 3 + 2];
                const double inv = 1.0 / sqrt(d[0] * d[0] + d[1] * d[1] + d[2] * d[2]);
                for (int a = 0; a < 3; ++a) d[a] *= inv;
                double te = -INFINITY, tx = INFINITY;
                bool in = true;
                for (int a = 0; a < 3; ++a) {
                    if (d[a] == 0.0) {
                        in = in && !(C[a] < -half[a] || C[a] > half[a]);
                    } else {
                        const double ta = (-half[a] - C[a]) / d[a], tb = (half[a] - C[a]) / d[a];
                        te = fmax(te, fmin(ta, tb));
                        tx = fmin(tx, fmax(ta, tb));
                    }
                }
                const double t0 = fmax(te, 0.0);
                if (!in || !(tx > t0)) continue;
                const double dz = (tx - t0) / cs.N, ts = t0 + 0.5 * dz;
                for (int a = 0; a < 3; ++a) {
                    o.q0[a] = to_fixed((C[a] + ts * d[a]) / cs.s[a] + q_off[a]);
                    o.dq[a] = to_fixed(dz * d[a] / cs.s[a]);
                }
                o.n = cs.N;
                o.coef = (float)(dz * (0.5 + 0.5 * U(rng)));
                o.cell_bound = fabsf(o.coef) * (float)drr::samples_per_cell_bound(o.dq, cs.N);
            }

        // the direct scatter: every sample to its eight clamped corners
        for (const RayRecord& o : rec) {
            if (o.n == 0) continue;
            for (int k = 0; k < o.n; ++k) {
                int cl[3];
                double fr[3];
                for (int a = 0; a < 3; ++a) {
                    const int64_t q = o.q0[a] + (int64_t)k * o.dq[a];
                    cl[a] = (int)(q >> 32);
                    fr[a] = (double)(uint32_t)q * 2.3283064365386963e-10;
                    CHECK(cl[a] >= -1 && cl[a] <= cs.n[a] - 1, "sample cell %d outside [-1, %d]",
                          cl[a], cs.n[a] - 1);
                }
                ++n_samples_total;
                for (int m = 0; m < 8; ++m) {
                    double w = o.coef;
                    int g[3];
                    for (int a = 0; a < 3; ++a) {
                        const int bit = (m >> a) & 1;
                        w *= bit ? fr[a] : 1.0 - fr[a];
                        g[a] = cl[a] + bit;
                        g[a] = g[a] < 0 ? 0 : (g[a] > cs.n[a] - 1 ? cs.n[a] - 1 : g[a]);
                    }
                    direct[((size_t)g[2] * ny + g[1]) * nx + g[0]] += w;
                }
            }
        }

        // the bricks
        const int B = cs.B, P = drr::brick_pitch(B), NE = P * P * P;
        const int nbx = (nx + B - 1) / B, nby = (ny + B - 1) / B, nbz = (nz + B - 1) / B;
        for (int bz = 0; bz < nbz; ++bz)
            for (int by = 0; by < nby; ++by)
                for (int bx = 0; bx < nbx; ++bx) {
                    const BrickBox b = drr::brick_box(cs.n, B, bx, by, bz);
                    for (int a = 0; a < 3; ++a) CHECK(b.e[a] >= 1 && b.e[a] <= B, "extent %d", b.e[a]);
                    const drr::BrickRegion reg = drr::brick_region(cs.n, cs.s, q_off, b);
                    const PixelRect pr = drr::brick_pixel_rect(Pm, reg, cs.H, cs.W);
                    const drr::BrickHull hull = drr::brick_hull(Pm, reg);
                    std::vector<int> span0(cs.H, 0), span1(cs.H, -1);
                    for (int r = pr.r0; r <= pr.r1; ++r) {
                        drr::brick_row_span(hull, r, pr.c0, pr.c1, span0[r], span1[r]);
                        CHECK(span1[r] < span0[r] || (span0[r] >= pr.c0 && span1[r] <= pr.c1),
                              "row span [%d, %d] outside the rectangle", span0[r], span1[r]);
                    }
                    std::vector<double> acc(NE, 0.0);
                    for (int r = 0; r < cs.H; ++r)
                        for (int c = 0; c < cs.W; ++c) {
                            const RayRecord& o = rec[(size_t)r * cs.W + c];
                            if (o.n == 0) continue;
                            const bool in_rect =
                                r >= pr.r0 && r <= pr.r1 && c >= pr.c0 && c <= pr.c1;
                            const bool cand = in_rect && c >= span0[r] && c <= span1[r];
                            int k_lo = 0, k_hi = 0, x_lo = 0, x_hi = 0;
                            if (in_rect && !cand) ++n_rejected;
                            if (cand) {
                                ++n_candidates;
                                drr::brick_sample_range(o, b, k_lo, k_hi);
                                CHECK(k_lo >= 0 && k_lo <= k_hi && k_hi <= o.n,
                                      "range [%d, %d) of %d", k_lo, k_hi, o.n);
                                int64_t q_rel[3];
                                drr::brick_exact_range(o, b, x_lo, x_hi, q_rel);
                                CHECK(x_lo >= k_lo && x_hi <= k_hi && x_lo <= x_hi,
                                      "exact range [%d, %d) outside [%d, %d)", x_lo, x_hi, k_lo, k_hi);
                                if (x_hi > x_lo)
                                    for (int a = 0; a < 3; ++a)
                                        CHECK(q_rel[a] == o.q0[a] + (int64_t)x_lo * o.dq[a] -
                                                              (int64_t)(b.lo[a] - 1) * ((int64_t)1 << 32),
                                              "relative start position");
                                for (int k = x_lo; k < x_hi; ++k)
                                    CHECK(drr::brick_sample_inside(o, b, k),
                                          "sample %d of the exact range is outside", k);
                            }
                            for (int k = 0; k < o.n; ++k) {
                                int cl[3];
                                double fr[3];
                                bool in = true;
                                for (int a = 0; a < 3; ++a) {
                                    const int64_t q = o.q0[a] + (int64_t)k * o.dq[a] -
                                                      ((int64_t)(b.lo[a] - 1) * ((int64_t)1 << 32));
                                    cl[a] = (int)(q >> 32);
                                    fr[a] = (double)(uint32_t)q * 2.3283064365386963e-10;
                                    in = in && (uint32_t)cl[a] <= (uint32_t)b.e[a];
                                }
                                if (!in) continue;
                                CHECK(in_rect, "brick (%d,%d,%d) misses pixel (%d,%d) of view %d",
                                      bx, by, bz, r, c, v);
                                CHECK(cand, "row span drops pixel (%d,%d) of view %d", r, c, v);
                                CHECK(k >= k_lo && k < k_hi,
                                      "sample %d outside [%d, %d) (brick %d,%d,%d)", k, k_lo,
                                      k_hi, bx, by, bz);
                                CHECK(k >= x_lo && k < x_hi,
                                      "sample %d outside the exact range [%d, %d)", k, x_lo, x_hi);
                                const int e0 = drr::brick_cell_entry(B, cl[0], cl[1], cl[2]);
                                for (int m = 0; m < 8; ++m) {
                                    const int e = e0 + drr::brick_corner_offset(B, m);
                                    CHECK(e >= 0 && e < NE, "entry %d outside [0, %d)", e, NE);
                                    if (e < 0 || e >= NE) continue;
                                    double w = o.coef;
                                    for (int a = 0; a < 3; ++a)
                                        w *= ((m >> a) & 1) ? fr[a] : 1.0 - fr[a];
                                    acc[e] += w;
                                }
                            }
                        }
                    // fold, axis by axis, as the kernel does
                    for (int a = 0; a < 3; ++a) {
                        const bool low = b.lo[a] == 0, high = b.lo[a] + b.e[a] == cs.n[a];
                        for (int i = 0; i < P * P; ++i) {
                            int step;
                            const int base = drr::brick_line_base(B, a, i, step);
                            CHECK(base >= 0 && base + (b.e[a] + 1) * step < NE, "fold line");
                            if (low) acc[base + step] += acc[base];
                            if (high) acc[base + b.e[a] * step] += acc[base + (b.e[a] + 1) * step];
                        }
                    }
                    for (int z = 0; z < b.e[2]; ++z)
                        for (int y = 0; y < b.e[1]; ++y)
                            for (int x = 0; x < b.e[0]; ++x)
                                bricked[((size_t)(b.lo[2] + z) * ny + b.lo[1] + y) * nx + b.lo[0] + x] +=
                                    acc[drr::brick_entry(B, x + 1, y + 1, z + 1)];
                }
    }
    double worst = 0.0, scale = 0.0;
    for (size_t i = 0; i < n_vox; ++i) {
        worst = fmax(worst, fabs(direct[i] - bricked[i]));
        scale = fmax(scale, fabs(direct[i]));
    }
    CHECK(worst <= 1e-12 * fmax(scale, 1e-300), "bricked vs direct: %g of %g", worst, scale);
    printf("case n=(%d,%d,%d) B=%d views=%d det=%dx%d N=%d%s: %lld samples, %lld candidates "
           "(%lld more in the rectangles), max |bricked - direct| %.3g (scale %.3g)\n",
           nx, ny, nz, cs.B, cs.views, cs.H, cs.W, cs.N, cs.inside ? " inside" : "",
           n_samples_total, n_candidates, n_rejected, worst, scale);
    return g_fail;
}

int main()
{
    const Case cases[] = {
        // ragged volume, anisotropic voxels, oblique cameras
        {{11, 9, 7}, {1.0, 1.25, 0.8}, 13, 17, 37, 3, 4, 60.0, 1.2, 0.7, false, 1},
        // bricks larger than the volume on one axis; volume one voxel thick
        {{20, 20, 1}, {1.0, 1.0, 1.0}, 9, 50, 9, 2, 16, 60.0, 1.2, 0.7, false, 2},
        {{1, 12, 12}, {1.0, 1.0, 1.0}, 17, 33, 5, 2, 4, 60.0, 1.2, 0.7, false, 3},
        // several bricks per axis with a ragged last one, dense sampling
        {{35, 33, 31}, {1.0, 1.0, 1.0}, 40, 44, 203, 2, 16, 80.0, 1.5, 0.5, false, 4},
        {{26, 30, 22}, {0.9, 1.1, 1.0}, 30, 30, 64, 3, 12, 70.0, 1.3, 0.6, false, 5},
        // cameras inside the box (regions straddle or sit behind the camera)
        {{20, 20, 20}, {1.0, 1.0, 1.0}, 21, 21, 50, 2, 8, 3.0, 0.4, 3.1, true, 6},
        // many samples, axis-near rays
        {{10, 12, 14}, {1.0, 1.0, 1.0}, 8, 8, 5000, 1, 4, 60.0, 1.2, 0.0, false, 7},
        // a distant camera with a narrow field of view (dense rays), B = 16
        {{40, 36, 44}, {1.0, 1.0, 1.0}, 96, 96, 128, 2, 16, 1000.0, 2.5, 0.2, false, 8},
        // a close camera with a wide field of view (diverging rays)
        {{30, 30, 30}, {0.7, 0.7, 0.7}, 64, 64, 96, 3, 12, 25.0, 0.3, 0.5, false, 9},
    };
    for (const Case& c : cases)
        if (run_case(c) != 0) break;
    if (g_fail) {
        fprintf(stderr, "%d check(s) failed\n", g_fail);
        return 1;
    }
    printf("all brick index checks passed\n");
    return 0;
}
