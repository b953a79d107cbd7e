// CPU replay of the brick-owned Siddon backward's walk (the library's
// drr_siddon.hpp and drr_brick.hpp, compiled for the host):
//   - for every ray, the pieces of positive length that the whole walk gives
//     (the projector's loop: nearest crossing, piece, advance) are exactly the
//     union over bricks of the pieces the brick walks give -- same voxels,
//     bit-identical fp64 lengths, each piece in one brick only;
//   - every entry a brick walk hands out lies inside that brick;
//   - every brick with a piece of the ray finds the ray's pixel among its
//     candidates (brick_pixel_rect and brick_row_span of the brick's region).
// Bricks of 16 (the kernel's) and of 5 and 7 voxels (many bricks in small
// volumes), random cameras including sources inside the volume, anisotropic
// voxels, volumes whose sides are not multiples of the brick, and rays parallel
// to voxel planes.  Exit status 0 when every check holds; the first failures
// are printed.
//
// The cameras are this file's own: M = R^T K^-1 and C = -R^T t in fp64 (the
// library's view setup, restated), so that both walks share one ray.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdio.h>

#include <algorithm>
#include <random>
#include <vector>

#include "../../ct_forward_projection_amd/csrc/drr_siddon.hpp"

using drr::BrickBox;
using drr::SiddonRay;
using drr::ViewGeom;
using drr::VolumeDesc;

static int g_fail = 0;
#define CHECK(cond, ...)                                             \
    do {                                                             \
        if (!(cond)) {                                               \
            if (g_fail++ < 8) {                                      \
                fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
                fprintf(stderr, __VA_ARGS__);                        \
                fprintf(stderr, "\n");                               \
            }                                                        \
        }                                                            \
    } while (0)

struct Piece {
    int x, y, z;
    double len;
    bool operator<(const Piece& o) const
    {
        if (z != o.z) return z < o.z;
        if (y != o.y) return y < o.y;
        if (x != o.x) return x < o.x;
        return len < o.len;
    }
};

struct Camera {
    double K[9], R[9], t[3];
};

static VolumeDesc volume(int nx, int ny, int nz, const double s[3])
{
    VolumeDesc V{};
    const int n[3] = {nx, ny, nz};
    for (int a = 0; a < 3; ++a) {
        V.n[a] = n[a];
        V.s[a] = s[a];
        V.inv_s[a] = 1.0 / s[a];
        V.half_e[a] = 0.5 * n[a] * s[a];
        V.q_off[a] = 0.5 * (n[a] - 1);
    }
    return V;
}

static void inverse3(const double m[9], double r[9])
{
    const double d = m[0] * (m[4] * m[8] - m[5] * m[7]) - m[1] * (m[3] * m[8] - m[5] * m[6]) +
                     m[2] * (m[3] * m[7] - m[4] * m[6]);
    r[0] = (m[4] * m[8] - m[5] * m[7]) / d;
    r[1] = (m[2] * m[7] - m[1] * m[8]) / d;
    r[2] = (m[1] * m[5] - m[2] * m[4]) / d;
    r[3] = (m[5] * m[6] - m[3] * m[8]) / d;
    r[4] = (m[0] * m[8] - m[2] * m[6]) / d;
    r[5] = (m[2] * m[3] - m[0] * m[5]) / d;
    r[6] = (m[3] * m[7] - m[4] * m[6]) / d;
    r[7] = (m[1] * m[6] - m[0] * m[7]) / d;
    r[8] = (m[0] * m[4] - m[1] * m[3]) / d;
}

static ViewGeom geometry(const Camera& cam)
{
    double Ki[9];
    inverse3(cam.K, Ki);
    ViewGeom G;
    for (int a = 0; a < 3; ++a) {
        for (int b = 0; b < 3; ++b)
            G.M[a * 3 + b] = cam.R[0 * 3 + a] * Ki[0 * 3 + b] + cam.R[1 * 3 + a] * Ki[1 * 3 + b] +
                             cam.R[2 * 3 + a] * Ki[2 * 3 + b];
        G.C[a] = -(cam.R[0 * 3 + a] * cam.t[0] + cam.R[1 * 3 + a] * cam.t[1] +
                   cam.R[2 * 3 + a] * cam.t[2]);
    }
    return G;
}

// The fp32 projection K [R | t] the brick search works with.
static void projection(const Camera& cam, float P[12])
{
    for (int r = 0; r < 3; ++r)
        for (int c = 0; c < 4; ++c) {
            double v = 0.0;
            for (int k = 0; k < 3; ++k) v += cam.K[r * 3 + k] * (c < 3 ? cam.R[k * 3 + c] : cam.t[k]);
            P[r * 4 + c] = (float)v;
        }
}

// Rotation from three angles (radians) and a camera centre Cw: t = -R Cw.
static Camera camera(double f, double cx, double cy, double ax, double ay, double az,
                     const double Cw[3])
{
    Camera cam{};
    const double K[9] = {f, 0.0, cx, 0.0, f, cy, 0.0, 0.0, 1.0};
    for (int i = 0; i < 9; ++i) cam.K[i] = K[i];
    const double sx = sin(ax), cxa = cos(ax), sy = sin(ay), cya = cos(ay), sz = sin(az),
                 cza = cos(az);
    const double Rx[9] = {1, 0, 0, 0, cxa, -sx, 0, sx, cxa};
    const double Ry[9] = {cya, 0, sy, 0, 1, 0, -sy, 0, cya};
    const double Rz[9] = {cza, -sz, 0, sz, cza, 0, 0, 0, 1};
    double T[9];
    for (int r = 0; r < 3; ++r)
        for (int c = 0; c < 3; ++c) {
            T[r * 3 + c] = 0.0;
            for (int k = 0; k < 3; ++k) T[r * 3 + c] += Ry[r * 3 + k] * Rx[k * 3 + c];
        }
    for (int r = 0; r < 3; ++r)
        for (int c = 0; c < 3; ++c) {
            cam.R[r * 3 + c] = 0.0;
            for (int k = 0; k < 3; ++k) cam.R[r * 3 + c] += Rz[r * 3 + k] * T[k * 3 + c];
        }
    for (int r = 0; r < 3; ++r)
        cam.t[r] = -(cam.R[r * 3 + 0] * Cw[0] + cam.R[r * 3 + 1] * Cw[1] + cam.R[r * 3 + 2] * Cw[2]);
    return cam;
}

// The whole walk of the ray through pixel (r, c): the projector's loop.
static bool whole_walk(const ViewGeom& G, const VolumeDesc& V, int r, int c,
                       std::vector<Piece>& out)
{
    SiddonRay S;
    if (!drr::siddon_setup(G, V, r, c, S)) return false;
    double tc = S.t0;
    int guard = V.n[0] + V.n[1] + V.n[2] + 3;
    for (;;) {
        const drr::NextAxis m = drr::next_axis(S);
        const double te = fmin(m.t, S.t1);
        const double len = te - tc;
        if (len > 0.0) out.push_back({S.i[0], S.i[1], S.i[2], len});
        tc = fmax(tc, te);
        if (!(m.t < S.t1) || --guard <= 0 || !drr::advance(S, m, V)) break;
    }
    return true;
}

static long long g_rays = 0, g_pieces = 0, g_brick_walks = 0;

template <int B>
static void replay(const VolumeDesc& V, const Camera& cam, int H, int W)
{
    const ViewGeom G = geometry(cam);
    float P[12];
    projection(cam, P);
    const int nb[3] = {(V.n[0] + B - 1) / B, (V.n[1] + B - 1) / B, (V.n[2] + B - 1) / B};
    for (int r = 0; r < H; ++r)
        for (int c = 0; c < W; ++c) {
            std::vector<Piece> whole, bricks;
            const bool hit = whole_walk(G, V, r, c, whole);
            SiddonRay S0;
            CHECK(drr::siddon_clip(G, V, r, c, S0) == hit, "clip and setup disagree at (%d, %d)",
                  r, c);
            if (!hit) continue;
            ++g_rays;
            g_pieces += (long long)whole.size();
            for (int bz = 0; bz < nb[2]; ++bz)
                for (int by = 0; by < nb[1]; ++by)
                    for (int bx = 0; bx < nb[0]; ++bx) {
                        const BrickBox b = drr::brick_box(V.n, B, bx, by, bz);
                        SiddonRay S;
                        drr::siddon_clip(G, V, r, c, S);
                        double t_in, t_out;
                        if (!drr::siddon_brick_range(S, V, b, t_in, t_out)) continue;
                        ++g_brick_walks;
                        drr::siddon_brick_start(S, V, b, t_in);
                        size_t before = bricks.size();
                        drr::siddon_brick_walk<B>(S, b, t_in, t_out, [&](int e, double len) {
                            const int x = e % B, y = (e / B) % B, z = e / (B * B);
                            const bool in = e >= 0 && e < B * B * B && x < b.e[0] &&
                                            y < b.e[1] && z < b.e[2];
                            CHECK(in, "entry %d outside brick (%d %d %d) of extent %d %d %d", e,
                                  bx, by, bz, b.e[0], b.e[1], b.e[2]);
                            if (in && len > 0.0)
                                bricks.push_back({b.lo[0] + x, b.lo[1] + y, b.lo[2] + z, len});
                        });
                        if (bricks.size() == before) continue;
                        // the brick's candidate search finds this pixel
                        const drr::BrickRegion g = drr::siddon_brick_region(V, b);
                        const drr::PixelRect R = drr::brick_pixel_rect(P, g, H, W);
                        const bool in_rect = r >= R.r0 && r <= R.r1 && c >= R.c0 && c <= R.c1;
                        CHECK(in_rect, "pixel (%d, %d) outside the rectangle of brick (%d %d %d)",
                              r, c, bx, by, bz);
                        if (in_rect) {
                            int c0, c1;
                            drr::brick_row_span(drr::brick_hull(P, g), r, R.c0, R.c1, c0, c1);
                            CHECK(c >= c0 && c <= c1,
                                  "pixel (%d, %d) outside row span [%d, %d] of brick (%d %d %d)",
                                  r, c, c0, c1, bx, by, bz);
                        }
                    }
            std::sort(whole.begin(), whole.end());
            std::sort(bricks.begin(), bricks.end());
            bool same = whole.size() == bricks.size();
            for (size_t i = 0; same && i < whole.size(); ++i)
                same = whole[i].x == bricks[i].x && whole[i].y == bricks[i].y &&
                       whole[i].z == bricks[i].z && whole[i].len == bricks[i].len;
            CHECK(same, "ray (%d, %d): %zu pieces whole, %zu from bricks of %d", r, c,
                  whole.size(), bricks.size(), B);
        }
}

int main()
{
    std::mt19937_64 rng(20261203);
    std::uniform_real_distribution<double> U(0.0, 1.0);
    int cases = 0;
    for (int k = 0; k < 24; ++k) {
        const int nx = 5 + (int)(U(rng) * 36), ny = 5 + (int)(U(rng) * 36),
                  nz = 5 + (int)(U(rng) * 36);
        const double s[3] = {0.6 + U(rng), 0.6 + U(rng), 0.6 + U(rng)};
        const VolumeDesc V = volume(nx, ny, nz, s);
        const double ext = fmax(fmax(nx * s[0], ny * s[1]), nz * s[2]);
        // every fourth camera inside the volume, the others outside
        const bool inside = k % 4 == 3;
        const double dist = inside ? 0.2 * ext : (1.5 + 2.0 * U(rng)) * ext;
        const double ax = (U(rng) - 0.5) * 2.0, ay = (U(rng) - 0.5) * 2.0,
                     az = (U(rng) - 0.5) * 2.0;
        // centre on the camera's optical axis behind the volume's centre
        const double origin[3] = {0.0, 0.0, 0.0};
        const Camera probe = camera(1.0, 0.0, 0.0, ax, ay, az, origin);
        double Cw[3];
        for (int a = 0; a < 3; ++a)
            Cw[a] = -dist * probe.R[2 * 3 + a] + (U(rng) - 0.5) * 0.3 * ext * (inside ? 0.0 : 1.0);
        const int H = 9 + (int)(U(rng) * 10), W = 9 + (int)(U(rng) * 10);
        const double f = inside ? 0.6 * W : 1.1 * W * dist / ext;
        const Camera cam = camera(f, 0.5 * W + 0.25, 0.5 * H - 0.25, ax, ay, az, Cw);
        replay<16>(V, cam, H, W);
        replay<7>(V, cam, H, W);
        replay<5>(V, cam, H, W);
        ++cases;
    }
    // rays parallel to voxel planes: an axis-aligned camera whose principal
    // ray runs along z, one pixel column exactly in a plane x = const
    {
        const double s[3] = {1.0, 1.0, 1.0};
        const VolumeDesc V = volume(13, 11, 17, s);
        const double Cw[3] = {0.5, 0.3, -60.0};
        const Camera cam = camera(64.0, 3.5, 2.5, 0.0, 0.0, 0.0, Cw);
        replay<16>(V, cam, 7, 9);
        replay<5>(V, cam, 7, 9);
        ++cases;
    }
    // rays through voxel edges: a camera turned 45 degrees about z, centred on
    // the diagonal x = y of a cube of equal voxels, whose middle detector row
    // holds rays with d_x = d_y -- they cross x and y planes together (exactly
    // or within a few ulps), at brick faces and inside bricks
    {
        const double s[3] = {1.0, 1.0, 0.8};
        const VolumeDesc V = volume(23, 23, 19, s);
        const double a = 0.70710678118654757;
        Camera cam{};
        const double K[9] = {12.0, 0.0, 8.5, 0.0, 12.0, 4.5, 0.0, 0.0, 1.0};
        const double R[9] = {a, -a, 0.0, 0.0, 0.0, -1.0, a, a, 0.0};
        const double Cw[3] = {-40.0, -40.0, 0.35};
        for (int i = 0; i < 9; ++i) cam.K[i] = K[i], cam.R[i] = R[i];
        for (int r = 0; r < 3; ++r)
            cam.t[r] = -(R[r * 3 + 0] * Cw[0] + R[r * 3 + 1] * Cw[1] + R[r * 3 + 2] * Cw[2]);
        replay<16>(V, cam, 9, 17);
        replay<7>(V, cam, 9, 17);
        replay<5>(V, cam, 9, 17);
        ++cases;
    }
    printf("%d cameras, %lld rays, %lld pieces, %lld brick walks\n", cases, g_rays, g_pieces,
           g_brick_walks);
    if (g_fail) {
        printf("%d Siddon brick checks failed\n", g_fail);
        return 1;
    }
    printf("all Siddon brick checks passed\n");
    return 0;
}
