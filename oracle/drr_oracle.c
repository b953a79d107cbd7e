/*
 * drr_oracle.c -- CPU oracle for differentiable cone-beam DRR ray casting.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the package smoke check and
 * the benchmark's CPU-baseline leg may load this library.  It shares no source,
 * header, table or helper with the HIP library: it reads the same seeded input
 * arrays and nothing else.
 *
 * Plain, slow and meant to be checked by eye: scalar double arithmetic, no SIMD,
 * no fast-math, no FMA contraction, OpenMP only across rays.  Every function
 * names the passage of the source pages it follows:
 *
 *   [nanodrr]   "nanodrr" project page, introduction: projective geometry uses
 *               the Hartley-Zisserman pinhole camera (P = K [R | t]).
 *   [fd-init]   flashdrr.rendering API, VolumeRaycaster.__init__: ray_samples
 *               samples per ray; use_beer_lambert returns 1 - exp(-int mu dz).
 *   [fd-fov]    flashdrr.rendering API, VolumeRaycaster.set_fov: per-pixel ray
 *               directions are built in the image plane and normalised.
 *   [fd-class]  flashdrr.rendering API, VolumeRaycaster class text: samples
 *               along each ray are trilinear (grid_sample) gathers of the volume;
 *               rendering is differentiable with respect to the volume.
 *   [diffct-qs] diffct 2.1.0, Quickstart: project() gives line integrals,
 *               backproject() the matched adjoint A^T, and for
 *               0.5 ||A x - y||^2 the gradient is A^T (A x - y).
 *   [tt-adj]    torchtomo, "Discrete Adjoint and Learned Primal-Dual": the
 *               adjoint satisfies <A x, y> = <x, A^T y>.
 *   [diffct-ft] diffct 2.1.0, "Why diffct" feature list: project() and
 *               backproject() are an exact adjoint pair for the cell-constant
 *               Siddon model (each voxel a constant, each ray weighted by its
 *               exact length inside the voxel).
 *
 * Readings taken where the pages are silent (each is restated at the code that
 * implements it):
 *   - world units are mm, mu is 1/mm, ray directions are unit vectors so the
 *     ray parameter t is a distance in mm;
 *   - the volume vol[k][j][i] (x fastest) fills the axis-aligned box
 *     [-E/2, E/2] with E = (nx sx, ny sy, nz sz); voxel (i,j,k) is centred at
 *     ((i+1/2) sx - Ex/2, (j+1/2) sy - Ey/2, (k+1/2) sz - Ez/2);
 *   - pixel (r, c) is the homogeneous image point (c + 1/2, r + 1/2, 1);
 *   - each ray is clipped to the box (slab test), t0 = max(t_entry, 0),
 *     t1 = t_exit, and it misses when t1 <= t0 (output 0, no gradient);
 *   - the N samples sit at the midpoints t0 + (k + 1/2) dz, dz = (t1 - t0) / N;
 *   - trilinear interpolation at the continuous index q = (p + E/2) / s - 1/2
 *     with both corner indices of every axis clamped to [0, n-1];
 *   - the Beer-Lambert output is evaluated as -expm1(-s), equal to 1 - exp(-s).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_BEER_LAMBERT 0
#define ORACLE_LINE_INTEGRAL 1

/* ------------------------------------------------------------------ geometry */

/* Camera centre of a world-to-camera pose [R | t] ([nanodrr]): x_cam = R x + t,
 * so the centre (x_cam = 0) is C = -R^T t.  pose is 3x4 row-major. */
static void camera_centre(const double *pose, double C[3])
{
    for (int a = 0; a < 3; ++a) {
        C[a] = -(pose[0 * 4 + a] * pose[0 * 4 + 3] +
                 pose[1 * 4 + a] * pose[1 * 4 + 3] +
                 pose[2 * 4 + a] * pose[2 * 4 + 3]);
    }
}

static double det3(const double m[9])
{
    return m[0] * (m[4] * m[8] - m[5] * m[7])
         - m[1] * (m[3] * m[8] - m[5] * m[6])
         + m[2] * (m[3] * m[7] - m[4] * m[6]);
}

/* Solve K x = b by Cramer's rule (K row-major).  Returns 0 if K is singular. */
static int solve3(const double K[9], const double b[3], double x[3])
{
    double D = det3(K);
    if (D == 0.0) return 0;
    for (int col = 0; col < 3; ++col) {
        double M[9];
        memcpy(M, K, sizeof(M));
        for (int row = 0; row < 3; ++row) M[row * 3 + col] = b[row];
        x[col] = det3(M) / D;
    }
    return 1;
}

/* Unit world direction of the ray through pixel (r, c) ([nanodrr], [fd-fov]):
 * back-project the homogeneous pixel centre m = (c + 1/2, r + 1/2, 1) through
 * K^-1 into camera coordinates, rotate to world with R^T, normalise. */
static int pixel_direction(const double K[9], const double *pose, int r, int c, double d[3])
{
    double m[3] = { c + 0.5, r + 0.5, 1.0 };
    double dc[3];
    if (!solve3(K, m, dc)) return 0;
    for (int a = 0; a < 3; ++a)
        d[a] = pose[0 * 4 + a] * dc[0] + pose[1 * 4 + a] * dc[1] + pose[2 * 4 + a] * dc[2];
    double len = sqrt(d[0] * d[0] + d[1] * d[1] + d[2] * d[2]);
    if (!(len > 0.0)) return 0;
    for (int a = 0; a < 3; ++a) d[a] /= len;
    return 1;
}

/* Slab test of the ray C + t d against the box [-E/2, E/2].  An axis with
 * d_a == 0 constrains nothing if C_a lies inside the slab and misses otherwise.
 * Returns 1 and the clipped range [t0, t1] (t0 = max(t_entry, 0)) on a hit. */
static int clip_to_box(const double C[3], const double d[3], const double E[3],
                       double *t0, double *t1)
{
    double t_entry = -INFINITY, t_exit = INFINITY;
    for (int a = 0; a < 3; ++a) {
        double lo = -0.5 * E[a], hi = 0.5 * E[a];
        if (d[a] == 0.0) {
            if (C[a] < lo || C[a] > hi) return 0;
            continue;
        }
        double ta = (lo - C[a]) / d[a];
        double tb = (hi - C[a]) / d[a];
        double tmin = ta < tb ? ta : tb;
        double tmax = ta < tb ? tb : ta;
        if (tmin > t_entry) t_entry = tmin;
        if (tmax < t_exit) t_exit = tmax;
    }
    double start = t_entry > 0.0 ? t_entry : 0.0;
    if (!(t_exit > start)) return 0;
    *t0 = start;
    *t1 = t_exit;
    return 1;
}

typedef struct {
    double C[3], d[3];
    double t0, t1;
    int hit;
} oracle_ray_t;

/* Steps 1-2 of the forward: ray generation and clipping for pixel (r, c). */
static void make_ray(const double K[9], const double *pose, const double E[3],
                     int r, int c, oracle_ray_t *ray)
{
    camera_centre(pose, ray->C);
    ray->hit = 0;
    ray->t0 = 0.0;
    ray->t1 = 0.0;
    ray->d[0] = ray->d[1] = ray->d[2] = 0.0;
    if (!pixel_direction(K, pose, r, c, ray->d)) return;
    ray->hit = clip_to_box(ray->C, ray->d, E, &ray->t0, &ray->t1);
}

/* ------------------------------------------------------------------ volume */

typedef struct {
    const float *vol;  /* vol[(k * ny + j) * nx + i] */
    long n[3];         /* nx, ny, nz */
    double s[3];       /* voxel spacing sx, sy, sz (mm) */
    double E[3];       /* box extent n_a * s_a (mm) */
} oracle_volume_t;

static void volume_init(oracle_volume_t *V, const float *vol, int nz, int ny, int nx,
                        const double *spacing)
{
    V->vol = vol;
    V->n[0] = nx;
    V->n[1] = ny;
    V->n[2] = nz;
    for (int a = 0; a < 3; ++a) {
        V->s[a] = spacing[a];
        V->E[a] = (double)V->n[a] * spacing[a];
    }
}

/* Continuous voxel index of a world point: voxel centres sit at integers. */
static void world_to_index(const oracle_volume_t *V, const double p[3], double q[3])
{
    for (int a = 0; a < 3; ++a) q[a] = (p[a] + 0.5 * V->E[a]) / V->s[a] - 0.5;
}

static long clamp_index(long i, long n)
{
    if (i < 0) return 0;
    if (i > n - 1) return n - 1;
    return i;
}

/* The eight trilinear corners of q ([fd-class] grid_sample, trilinear): corner
 * c (bit 0 = x, bit 1 = y, bit 2 = z) has linear offset off[c] and weight w[c];
 * corner indices are clamped to the volume (clamp to edge), so near a face two
 * corners may share one voxel and their weights then add up. */
static void trilinear_corners(const oracle_volume_t *V, const double q[3], long off[8], double w[8])
{
    long lo[3], hi[3];
    double f[3];
    for (int a = 0; a < 3; ++a) {
        double fl = floor(q[a]);
        f[a] = q[a] - fl;
        lo[a] = clamp_index((long)fl, V->n[a]);
        hi[a] = clamp_index((long)fl + 1, V->n[a]);
    }
    for (int c = 0; c < 8; ++c) {
        long i = (c & 1) ? hi[0] : lo[0];
        long j = (c & 2) ? hi[1] : lo[1];
        long k = (c & 4) ? hi[2] : lo[2];
        double wx = (c & 1) ? f[0] : 1.0 - f[0];
        double wy = (c & 2) ? f[1] : 1.0 - f[1];
        double wz = (c & 4) ? f[2] : 1.0 - f[2];
        off[c] = (k * V->n[1] + j) * V->n[0] + i;
        w[c] = wx * wy * wz;
    }
}

static double trilinear(const oracle_volume_t *V, const double q[3])
{
    long off[8];
    double w[8];
    trilinear_corners(V, q, off, w);
    double val = 0.0;
    for (int c = 0; c < 8; ++c) val += w[c] * (double)V->vol[off[c]];
    return val;
}

/* Sample k of N on a clipped ray, as a continuous voxel index: midpoint rule,
 * t_k = t0 + (k + 1/2) dz with dz = (t1 - t0) / N. */
static void sample_index(const oracle_volume_t *V, const oracle_ray_t *ray, double dz, int k,
                         double q[3])
{
    double t = ray->t0 + ((double)k + 0.5) * dz;
    double p[3];
    for (int a = 0; a < 3; ++a) p[a] = ray->C[a] + t * ray->d[a];
    world_to_index(V, p, q);
}

/* s = sum_k mu(t_k) dz over the N samples of one ray ([fd-init] ray_samples,
 * Beer-Lambert integrand mu dz).  A ray that misses the box integrates to 0. */
static double ray_line_integral(const oracle_volume_t *V, const oracle_ray_t *ray, int N)
{
    if (!ray->hit) return 0.0;
    double dz = (ray->t1 - ray->t0) / (double)N;
    double acc = 0.0;
    for (int k = 0; k < N; ++k) {
        double q[3];
        sample_index(V, ray, dz, k, q);
        acc += trilinear(V, q);
    }
    return acc * dz;
}

/* Output stage: Beer-Lambert image 1 - exp(-s) ([fd-init] use_beer_lambert,
 * evaluated as -expm1(-s)) or the raw line integral ([diffct-qs] project). */
static double output_value(double s, int mode)
{
    return mode == ORACLE_BEER_LAMBERT ? -expm1(-s) : s;
}

static int check_common(int nz, int ny, int nx, const double *spacing, int n_views, int H,
                        int W, int n_samples, int mode)
{
    if (nz < 1 || ny < 1 || nx < 1) return -1;
    if (n_views < 0 || H < 0 || W < 0) return -1;
    if (n_samples < 1) return -1;
    if (mode != ORACLE_BEER_LAMBERT && mode != ORACLE_LINE_INTEGRAL) return -1;
    for (int a = 0; a < 3; ++a)
        if (!(spacing[a] > 0.0)) return -1;
    return 0;
}

static void set_threads(int n_threads)
{
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
}

/* ------------------------------------------------------------------ exports */

/* Forward DRR for every pixel of every view.  out[(v*H + r)*W + c] receives the
 * Beer-Lambert image or the line integral; line_integral (nullable) receives s.
 * Returns 0, or -1 on invalid arguments. */
int oracle_forward(const float *vol, int nz, int ny, int nx, const double *spacing,
                   const double *K, const double *poses, int n_views, int H, int W,
                   int n_samples, int mode, double *out, double *line_integral, int n_threads)
{
    if (check_common(nz, ny, nx, spacing, n_views, H, W, n_samples, mode)) return -1;
    oracle_volume_t V;
    volume_init(&V, vol, nz, ny, nx, spacing);
    long n_rays = (long)n_views * H * W;
    set_threads(n_threads);
#pragma omp parallel for schedule(dynamic, 64)
    for (long ray_id = 0; ray_id < n_rays; ++ray_id) {
        int v = (int)(ray_id / ((long)H * W));
        int r = (int)((ray_id / W) % H);
        int c = (int)(ray_id % W);
        oracle_ray_t ray;
        make_ray(K, poses + 12L * v, V.E, r, c, &ray);
        double s = ray_line_integral(&V, &ray, n_samples);
        out[ray_id] = output_value(s, mode);
        if (line_integral) line_integral[ray_id] = s;
    }
    return 0;
}

/* Adjoint / volume gradient ([diffct-qs] backproject and x.grad; [fd-class]
 * differentiable with respect to the volume).  For upstream g = dL/dI:
 *   y_p = g_p exp(-s_p)   (Beer-Lambert, dI/ds = exp(-s))
 *   y_p = g_p             (line integral)
 * and for every sample and trilinear corner grad[corner] += y_p dz w_corner.
 * The weights depend on geometry only, so for the line integral this is exactly
 * A^T.  vol is needed only for Beer-Lambert (to evaluate s) and may be NULL for
 * the line integral.  grad (nz*ny*nx doubles) is overwritten.  Threads get
 * private gradient buffers while (threads - 1) buffers fit in max_buffer_bytes;
 * otherwise the scatter runs on one thread.  Returns the thread count used, or
 * -1 on invalid arguments. */
int oracle_adjoint(const float *vol, int nz, int ny, int nx, const double *spacing,
                   const double *K, const double *poses, int n_views, int H, int W,
                   int n_samples, int mode, const double *g, double *grad, int n_threads,
                   long long max_buffer_bytes)
{
    if (check_common(nz, ny, nx, spacing, n_views, H, W, n_samples, mode)) return -1;
    if (mode == ORACLE_BEER_LAMBERT && vol == NULL) return -1;
    oracle_volume_t V;
    volume_init(&V, vol, nz, ny, nx, spacing);
    long n_vox = (long)nx * ny * nz;
    long n_rays = (long)n_views * H * W;
    memset(grad, 0, sizeof(double) * (size_t)n_vox);

    int T = n_threads > 0 ? n_threads : 1;
#ifndef _OPENMP
    T = 1;
#endif
    while (T > 1 && (long long)(T - 1) * n_vox * (long long)sizeof(double) > max_buffer_bytes) --T;
    double **bufs = (double **)calloc((size_t)T, sizeof(double *));
    if (!bufs) return -1;
    bufs[0] = grad;
    for (int i = 1; i < T; ++i) {
        bufs[i] = (double *)calloc((size_t)n_vox, sizeof(double));
        if (!bufs[i]) {
            for (int j = 1; j < i; ++j) free(bufs[j]);
            free(bufs);
            return -1;
        }
    }
    set_threads(T);
#pragma omp parallel for schedule(dynamic, 64) num_threads(T)
    for (long ray_id = 0; ray_id < n_rays; ++ray_id) {
#ifdef _OPENMP
        double *acc = bufs[omp_get_thread_num()];
#else
        double *acc = bufs[0];
#endif
        int v = (int)(ray_id / ((long)H * W));
        int r = (int)((ray_id / W) % H);
        int c = (int)(ray_id % W);
        oracle_ray_t ray;
        make_ray(K, poses + 12L * v, V.E, r, c, &ray);
        if (!ray.hit) continue;
        double y = g[ray_id];
        if (mode == ORACLE_BEER_LAMBERT) y *= exp(-ray_line_integral(&V, &ray, n_samples));
        double dz = (ray.t1 - ray.t0) / (double)n_samples;
        for (int k = 0; k < n_samples; ++k) {
            double q[3];
            long off[8];
            double w[8];
            sample_index(&V, &ray, dz, k, q);
            trilinear_corners(&V, q, off, w);
            for (int cn = 0; cn < 8; ++cn) acc[off[cn]] += y * dz * w[cn];
        }
    }
    for (int i = 1; i < T; ++i) {
        for (long x = 0; x < n_vox; ++x) grad[x] += bufs[i][x];
        free(bufs[i]);
    }
    free(bufs);
    return T;
}

/* Geometry of one ray, for pins: out = (C[3], d[3], t0, t1).  Returns 1 on a
 * hit, 0 on a miss (t0 = t1 = 0), -1 if K is singular. */
int oracle_ray(const double *K, const double *pose, const double *extent, int r, int c,
               double *out)
{
    oracle_ray_t ray;
    double d[3];
    if (!pixel_direction(K, pose, r, c, d)) return -1;
    make_ray(K, pose, extent, r, c, &ray);
    for (int a = 0; a < 3; ++a) {
        out[a] = ray.C[a];
        out[3 + a] = ray.d[a];
    }
    out[6] = ray.t0;
    out[7] = ray.t1;
    return ray.hit;
}

/* Clipped chord length t1 - t0 of every ray (0 for a miss): which rays the
 * forward integrates at all.  Pinned by the constant-box chords. */
int oracle_chords(const double *extent, const double *K, const double *poses, int n_views,
                  int H, int W, double *chord, int n_threads)
{
    if (n_views < 0 || H < 0 || W < 0) return -1;
    long n_rays = (long)n_views * H * W;
    set_threads(n_threads);
#pragma omp parallel for schedule(dynamic, 256)
    for (long ray_id = 0; ray_id < n_rays; ++ray_id) {
        int v = (int)(ray_id / ((long)H * W));
        int r = (int)((ray_id / W) % H);
        int c = (int)(ray_id % W);
        oracle_ray_t ray;
        make_ray(K, poses + 12L * v, extent, r, c, &ray);
        chord[ray_id] = ray.hit ? ray.t1 - ray.t0 : 0.0;
    }
    return 0;
}

/* The same forward with an analytic density in place of the trilinear volume:
 * a sum of uniform balls, spheres[5 m .. 5 m + 4] = (cx, cy, cz, radius, mu).
 * The box (extent, centred at the origin) still clips the rays.  Used to pin
 * the geometry against the chord of a ball, 2 mu sqrt(r^2 - d^2). */
int oracle_forward_spheres(const double *spheres, int n_spheres, const double *extent,
                           const double *K, const double *poses, int n_views, int H, int W,
                           int n_samples, int mode, double *out, int n_threads)
{
    if (n_views < 0 || H < 0 || W < 0 || n_samples < 1) return -1;
    long n_rays = (long)n_views * H * W;
    set_threads(n_threads);
#pragma omp parallel for schedule(dynamic, 64)
    for (long ray_id = 0; ray_id < n_rays; ++ray_id) {
        int v = (int)(ray_id / ((long)H * W));
        int r = (int)((ray_id / W) % H);
        int c = (int)(ray_id % W);
        oracle_ray_t ray;
        make_ray(K, poses + 12L * v, extent, r, c, &ray);
        double s = 0.0;
        if (ray.hit) {
            double dz = (ray.t1 - ray.t0) / (double)n_samples;
            double acc = 0.0;
            for (int k = 0; k < n_samples; ++k) {
                double t = ray.t0 + ((double)k + 0.5) * dz;
                double p[3];
                for (int a = 0; a < 3; ++a) p[a] = ray.C[a] + t * ray.d[a];
                for (int b = 0; b < n_spheres; ++b) {
                    const double *sp = spheres + 5L * b;
                    double r2 = 0.0;
                    for (int a = 0; a < 3; ++a) r2 += (p[a] - sp[a]) * (p[a] - sp[a]);
                    if (r2 <= sp[3] * sp[3]) acc += sp[4];
                }
            }
            s = acc * dz;
        }
        out[ray_id] = output_value(s, mode);
    }
    return 0;
}

static int cmp_double(const void *a, const void *b)
{
    double x = *(const double *)a, y = *(const double *)b;
    return (x > y) - (x < y);
}

/* The N -> infinity limit of the sampled line integral: the exact integral of
 * the clamped trilinear field over [t0, t1].  The ray is cut wherever a
 * continuous index q_a(t) crosses an integer in [0, n_a - 1]; on each piece
 * every axis is either inside one cell (weight affine in t) or clamped
 * (constant), so the field is a cubic polynomial in t and 2-point
 * Gauss-Legendre integrates it exactly. */
int oracle_exact_line_integral(const float *vol, int nz, int ny, int nx, const double *spacing,
                               const double *K, const double *poses, int n_views, int H, int W,
                               double *s_out, int n_threads)
{
    if (check_common(nz, ny, nx, spacing, n_views, H, W, 1, ORACLE_LINE_INTEGRAL)) return -1;
    oracle_volume_t V;
    volume_init(&V, vol, nz, ny, nx, spacing);
    long n_rays = (long)n_views * H * W;
    long max_breaks = (long)nx + ny + nz + 2;
    const double gl = 0.5 / sqrt(3.0);
    set_threads(n_threads);
#pragma omp parallel
    {
        double *tb = (double *)malloc(sizeof(double) * (size_t)max_breaks);
#pragma omp for schedule(dynamic, 16)
        for (long ray_id = 0; ray_id < n_rays; ++ray_id) {
            int v = (int)(ray_id / ((long)H * W));
            int r = (int)((ray_id / W) % H);
            int c = (int)(ray_id % W);
            oracle_ray_t ray;
            make_ray(K, poses + 12L * v, V.E, r, c, &ray);
            if (!ray.hit || !tb) {
                s_out[ray_id] = 0.0;
                continue;
            }
            long nb = 0;
            tb[nb++] = ray.t0;
            for (int a = 0; a < 3; ++a) {
                if (ray.d[a] == 0.0) continue;
                for (long m = 0; m < V.n[a]; ++m) {
                    /* q_a(t) = m  <=>  C_a + t d_a = (m + 1/2) s_a - E_a / 2 */
                    double t = (((double)m + 0.5) * V.s[a] - 0.5 * V.E[a] - ray.C[a]) / ray.d[a];
                    if (t > ray.t0 && t < ray.t1) tb[nb++] = t;
                }
            }
            tb[nb++] = ray.t1;
            qsort(tb, (size_t)nb, sizeof(double), cmp_double);
            double s = 0.0;
            for (long b = 0; b + 1 < nb; ++b) {
                double len = tb[b + 1] - tb[b];
                if (!(len > 0.0)) continue;
                double mid = 0.5 * (tb[b] + tb[b + 1]);
                double nodes[2] = { mid - gl * len, mid + gl * len };
                for (int e = 0; e < 2; ++e) {
                    double p[3], q[3];
                    for (int a = 0; a < 3; ++a) p[a] = ray.C[a] + nodes[e] * ray.d[a];
                    world_to_index(&V, p, q);
                    s += 0.5 * len * trilinear(&V, q);
                }
            }
            s_out[ray_id] = s;
        }
        free(tb);
    }
    return 0;
}

/* ------------------------------------------------------------ pose gradient */

/* Value and gradient with respect to q of the clamped trilinear field at q.
 * With both corners of an axis clamped to one voxel the field is constant
 * along that axis and the formula gives 0 there, as it should. */
static double trilinear_grad(const oracle_volume_t *V, const double q[3], double gq[3])
{
    long off[8];
    double w[8];
    trilinear_corners(V, q, off, w);
    double f[3];
    for (int a = 0; a < 3; ++a) f[a] = q[a] - floor(q[a]);
    double val = 0.0;
    gq[0] = gq[1] = gq[2] = 0.0;
    for (int c = 0; c < 8; ++c) {
        double v = (double)V->vol[off[c]];
        val += w[c] * v;
        for (int a = 0; a < 3; ++a) {
            /* d w_c / d q_a: the factor of axis a becomes +1 (upper corner) or
             * -1 (lower corner), the other two factors stay */
            double dw = ((c >> a) & 1) ? 1.0 : -1.0;
            for (int b = 0; b < 3; ++b) {
                if (b == a) continue;
                dw *= ((c >> b) & 1) ? f[b] : 1.0 - f[b];
            }
            gq[a] += dw * v;
        }
    }
    return val;
}

/* Gradient of L = sum_p g_p I_p with respect to each view's pose entries
 * (flashdrr API, VolumeRaycaster class text: rendering is differentiable with
 * respect to the view matrices; flashdrr README Features: gradients through the
 * camera parameters).  grad_pose[12 v + j] receives dL/dP_v[j] for the 3x4
 * row-major [R | t] entries treated as independent.
 *
 * Plain forward-mode differentiation of the forward, one pose entry theta at a
 * time: dC = -dR^T t - R^T dt, dw = dR^T K^-1 m for the unnormalised direction
 * w, dd = (dw - d (d . dw)) / |w|; the clipped range moves with the plane that
 * bounds it, dt = -(dC_a + t dd_a) / d_a for the entry (exit) axis a (0 if the
 * range starts at the source), ddz = (dt1 - dt0) / N, and each sample
 * p_k = C + t_k d moves by dp_k = dC + dt_k d + t_k dd with
 * dt_k = dt0 + (k + 1/2) ddz; ds = ddz sum mu_k + dz sum grad mu(p_k) . dp_k,
 * dI = exp(-s) ds (Beer-Lambert) or ds.  Rays that miss contribute nothing.
 * Returns 0, or -1 on invalid arguments. */
int oracle_pose_gradient(const float *vol, int nz, int ny, int nx, const double *spacing,
                         const double *K, const double *poses, int n_views, int H, int W,
                         int n_samples, int mode, const double *g, double *grad_pose,
                         int n_threads)
{
    if (check_common(nz, ny, nx, spacing, n_views, H, W, n_samples, mode)) return -1;
    oracle_volume_t V;
    volume_init(&V, vol, nz, ny, nx, spacing);
    memset(grad_pose, 0, sizeof(double) * 12 * (size_t)n_views);
    set_threads(n_threads);
    for (int v = 0; v < n_views; ++v) {
        const double *pose = poses + 12L * v;
        double acc[12] = {0};
#pragma omp parallel
        {
            double mine[12] = {0};
#pragma omp for schedule(dynamic, 16)
            for (long pix = 0; pix < (long)H * W; ++pix) {
                int r = (int)(pix / W), c = (int)(pix % W);
                double gp = g[(long)v * H * W + pix];
                oracle_ray_t ray;
                make_ray(K, pose, V.E, r, c, &ray);
                if (!ray.hit || gp == 0.0) continue;
                /* unnormalised direction w = R^T K^-1 m and its length */
                double m[3] = { c + 0.5, r + 0.5, 1.0 }, u[3], w[3];
                solve3(K, m, u);
                for (int a = 0; a < 3; ++a)
                    w[a] = pose[0 * 4 + a] * u[0] + pose[1 * 4 + a] * u[1] + pose[2 * 4 + a] * u[2];
                double len = sqrt(w[0] * w[0] + w[1] * w[1] + w[2] * w[2]);
                /* which planes bound the clipped range */
                int a_in = -1, a_out = -1;
                double t_entry = -INFINITY, t_exit = INFINITY;
                for (int a = 0; a < 3; ++a) {
                    if (ray.d[a] == 0.0) continue;
                    double ta = (-0.5 * V.E[a] - ray.C[a]) / ray.d[a];
                    double tb = (0.5 * V.E[a] - ray.C[a]) / ray.d[a];
                    double tmin = ta < tb ? ta : tb, tmax = ta < tb ? tb : ta;
                    if (tmin > t_entry) { t_entry = tmin; a_in = a; }
                    if (tmax < t_exit) { t_exit = tmax; a_out = a; }
                }
                int entry_moves = t_entry > 0.0;
                double dz = (ray.t1 - ray.t0) / (double)n_samples;
                /* s and its 12 directional derivatives */
                double s = 0.0, ds[12] = {0};
                double dC[12][3], dd[12][3], dt0[12], ddz[12];
                for (int j = 0; j < 12; ++j) {
                    double dR[9] = {0}, dtv[3] = {0}, dw[3];
                    if (j < 9) dR[j] = 1.0; else dtv[j - 9] = 1.0;
                    for (int a = 0; a < 3; ++a) {
                        dC[j][a] = -(dR[0 * 3 + a] * pose[0 * 4 + 3] + dR[1 * 3 + a] * pose[1 * 4 + 3] +
                                     dR[2 * 3 + a] * pose[2 * 4 + 3])
                                   - (pose[0 * 4 + a] * dtv[0] + pose[1 * 4 + a] * dtv[1] +
                                      pose[2 * 4 + a] * dtv[2]);
                        dw[a] = dR[0 * 3 + a] * u[0] + dR[1 * 3 + a] * u[1] + dR[2 * 3 + a] * u[2];
                    }
                    double ddw = ray.d[0] * dw[0] + ray.d[1] * dw[1] + ray.d[2] * dw[2];
                    for (int a = 0; a < 3; ++a) dd[j][a] = (dw[a] - ray.d[a] * ddw) / len;
                    dt0[j] = entry_moves ? -(dC[j][a_in] + ray.t0 * dd[j][a_in]) / ray.d[a_in] : 0.0;
                    double dt1 = -(dC[j][a_out] + ray.t1 * dd[j][a_out]) / ray.d[a_out];
                    ddz[j] = (dt1 - dt0[j]) / (double)n_samples;
                }
                double sum_mu = 0.0, sum_dmu[12] = {0};
                for (int k = 0; k < n_samples; ++k) {
                    double tk = ray.t0 + ((double)k + 0.5) * dz, p[3], q[3], gq[3];
                    for (int a = 0; a < 3; ++a) p[a] = ray.C[a] + tk * ray.d[a];
                    world_to_index(&V, p, q);
                    sum_mu += trilinear_grad(&V, q, gq);
                    for (int j = 0; j < 12; ++j) {
                        double dtk = dt0[j] + ((double)k + 0.5) * ddz[j];
                        for (int a = 0; a < 3; ++a) {
                            double dp = dC[j][a] + dtk * ray.d[a] + tk * dd[j][a];
                            sum_dmu[j] += gq[a] * dp / V.s[a];
                        }
                    }
                }
                s = dz * sum_mu;
                double dI = mode == ORACLE_BEER_LAMBERT ? exp(-s) : 1.0;
                for (int j = 0; j < 12; ++j) {
                    ds[j] = ddz[j] * sum_mu + dz * sum_dmu[j];
                    mine[j] += gp * dI * ds[j];
                }
            }
#pragma omp critical
            for (int j = 0; j < 12; ++j) acc[j] += mine[j];
        }
        /* 3x4 row-major output: R[r][c] at r*4 + c, t[r] at r*4 + 3 */
        for (int rr = 0; rr < 3; ++rr) {
            for (int cc = 0; cc < 3; ++cc) grad_pose[12L * v + rr * 4 + cc] = acc[rr * 3 + cc];
            grad_pose[12L * v + rr * 4 + 3] = acc[9 + rr];
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ Siddon */

static int compare_double(const void *a, const void *b)
{
    double x = *(const double *)a, y = *(const double *)b;
    return (x > y) - (x < y);
}

/* Cell-constant (Siddon) model of one clipped ray ([diffct-ft]): the volume is
 * constant inside each voxel box [i s - E/2, (i + 1) s - E/2] per axis, and
 * the ray's line integral is sum_v mu_v l_v with l_v the length of the ray
 * inside voxel v.  Plain merged-crossing method: list t0, t1 and every voxel
 * plane crossing strictly between them, sort, and give each gap of positive
 * length to the voxel that holds its midpoint (index floor((p + E/2) / s),
 * clamped to the volume).  tbuf holds n_x + n_y + n_z + 5 doubles.  Writes the
 * voxel offsets and lengths of the pieces; returns their count. */
static int siddon_segments(const oracle_volume_t *V, const oracle_ray_t *ray, double *tbuf,
                           long *off, double *len)
{
    if (!ray->hit) return 0;
    int m = 0;
    tbuf[m++] = ray->t0;
    tbuf[m++] = ray->t1;
    for (int a = 0; a < 3; ++a) {
        if (ray->d[a] == 0.0) continue;
        for (long i = 0; i <= V->n[a]; ++i) {
            double plane = (double)i * V->s[a] - 0.5 * V->E[a];
            double t = (plane - ray->C[a]) / ray->d[a];
            if (t > ray->t0 && t < ray->t1) tbuf[m++] = t;
        }
    }
    qsort(tbuf, (size_t)m, sizeof(double), compare_double);
    int n = 0;
    for (int k = 0; k + 1 < m; ++k) {
        double ta = tbuf[k], tb = tbuf[k + 1];
        if (!(tb > ta)) continue;
        double tm = 0.5 * (ta + tb);
        long idx[3];
        for (int a = 0; a < 3; ++a) {
            double p = ray->C[a] + tm * ray->d[a];
            idx[a] = clamp_index((long)floor((p + 0.5 * V->E[a]) / V->s[a]), V->n[a]);
        }
        off[n] = (idx[2] * V->n[1] + idx[1]) * V->n[0] + idx[0];
        len[n] = tb - ta;
        ++n;
    }
    return n;
}

static long siddon_max_pieces(const oracle_volume_t *V) { return V->n[0] + V->n[1] + V->n[2] + 5; }

/* Siddon line integral of one ray: s = sum over pieces of mu_v l_v. */
static double siddon_line_integral(const oracle_volume_t *V, const oracle_ray_t *ray,
                                   double *tbuf, long *off, double *len)
{
    int n = siddon_segments(V, ray, tbuf, off, len);
    double s = 0.0;
    for (int k = 0; k < n; ++k) s += (double)V->vol[off[k]] * len[k];
    return s;
}

/* Forward DRR in the cell-constant model ([diffct-ft]; [diffct-qs] project for
 * the line integral, [fd-init] Beer-Lambert for the image); same cameras and
 * box clip as oracle_forward.  Returns 0, or -1 on invalid arguments or when
 * scratch memory cannot be allocated. */
int oracle_siddon_forward(const float *vol, int nz, int ny, int nx, const double *spacing,
                          const double *K, const double *poses, int n_views, int H, int W,
                          int mode, double *out, double *line_integral, int n_threads)
{
    if (check_common(nz, ny, nx, spacing, n_views, H, W, 1, mode)) return -1;
    oracle_volume_t V;
    volume_init(&V, vol, nz, ny, nx, spacing);
    long n_rays = (long)n_views * H * W;
    long cap = siddon_max_pieces(&V);
    int failed = 0;
    set_threads(n_threads);
#pragma omp parallel
    {
        double *tbuf = (double *)malloc(sizeof(double) * (size_t)cap);
        long *off = (long *)malloc(sizeof(long) * (size_t)cap);
        double *len = (double *)malloc(sizeof(double) * (size_t)cap);
        if (!tbuf || !off || !len) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 64)
        for (long ray_id = 0; ray_id < n_rays; ++ray_id) {
            if (!tbuf || !off || !len) continue;
            int v = (int)(ray_id / ((long)H * W));
            int r = (int)((ray_id / W) % H);
            int c = (int)(ray_id % W);
            oracle_ray_t ray;
            make_ray(K, poses + 12L * v, V.E, r, c, &ray);
            double s = siddon_line_integral(&V, &ray, tbuf, off, len);
            out[ray_id] = output_value(s, mode);
            if (line_integral) line_integral[ray_id] = s;
        }
        free(tbuf);
        free(off);
        free(len);
    }
    return failed ? -1 : 0;
}

/* Matched adjoint of the cell-constant forward ([diffct-ft], [diffct-qs]
 * backproject; [tt-adj]): grad[v] += y_p l_v for every piece of every ray, with
 * y_p = g_p exp(-s_p) (Beer-Lambert) or g_p (line integral, exactly A^T g).
 * vol is needed only for Beer-Lambert.  grad (nz*ny*nx doubles) is
 * overwritten; threads get private buffers while they fit in max_buffer_bytes.
 * Returns the thread count used, or -1 on invalid arguments or allocation
 * failure. */
int oracle_siddon_adjoint(const float *vol, int nz, int ny, int nx, const double *spacing,
                          const double *K, const double *poses, int n_views, int H, int W,
                          int mode, const double *g, double *grad, int n_threads,
                          long long max_buffer_bytes)
{
    if (check_common(nz, ny, nx, spacing, n_views, H, W, 1, mode)) return -1;
    if (mode == ORACLE_BEER_LAMBERT && vol == NULL) return -1;
    oracle_volume_t V;
    volume_init(&V, vol, nz, ny, nx, spacing);
    long n_vox = (long)nx * ny * nz;
    long n_rays = (long)n_views * H * W;
    long cap = siddon_max_pieces(&V);
    memset(grad, 0, sizeof(double) * (size_t)n_vox);

    int T = n_threads > 0 ? n_threads : 1;
#ifndef _OPENMP
    T = 1;
#endif
    while (T > 1 && (long long)(T - 1) * n_vox * (long long)sizeof(double) > max_buffer_bytes) --T;
    double **bufs = (double **)calloc((size_t)T, sizeof(double *));
    if (!bufs) return -1;
    bufs[0] = grad;
    for (int i = 1; i < T; ++i) {
        bufs[i] = (double *)calloc((size_t)n_vox, sizeof(double));
        if (!bufs[i]) {
            for (int j = 1; j < i; ++j) free(bufs[j]);
            free(bufs);
            return -1;
        }
    }
    int failed = 0;
    set_threads(T);
#pragma omp parallel num_threads(T)
    {
#ifdef _OPENMP
        double *acc = bufs[omp_get_thread_num()];
#else
        double *acc = bufs[0];
#endif
        double *tbuf = (double *)malloc(sizeof(double) * (size_t)cap);
        long *off = (long *)malloc(sizeof(long) * (size_t)cap);
        double *len = (double *)malloc(sizeof(double) * (size_t)cap);
        if (!tbuf || !off || !len) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 64)
        for (long ray_id = 0; ray_id < n_rays; ++ray_id) {
            if (!tbuf || !off || !len) continue;
            int v = (int)(ray_id / ((long)H * W));
            int r = (int)((ray_id / W) % H);
            int c = (int)(ray_id % W);
            oracle_ray_t ray;
            make_ray(K, poses + 12L * v, V.E, r, c, &ray);
            if (!ray.hit) continue;
            int n = siddon_segments(&V, &ray, tbuf, off, len);
            double y = g[ray_id];
            if (mode == ORACLE_BEER_LAMBERT) {
                double s = 0.0;
                for (int k = 0; k < n; ++k) s += (double)V.vol[off[k]] * len[k];
                y *= exp(-s);
            }
            for (int k = 0; k < n; ++k) acc[off[k]] += y * len[k];
        }
        free(tbuf);
        free(off);
        free(len);
    }
    for (int i = 1; i < T; ++i) {
        for (long x = 0; x < n_vox; ++x) grad[x] += bufs[i][x];
        free(bufs[i]);
    }
    free(bufs);
    return failed ? -1 : T;
}

/* ------------------------------------------------- render: the flashdrr front end */

/* The VolumeRaycaster options of the flashdrr pages on top of the same rays:
 *   [fd-fwd]    flashdrr.rendering API, VolumeRaycaster.forward: vol is
 *               (B, C, D, H, W); N = B * views_per_vol view matrices, view v
 *               rendering volume v / views_per_vol; output (N, C, H, W).
 *   [fd-init]   __init__: density_factor multiplies the volume intensities
 *               before integration; use_beer_lambert = False selects
 *               front-to-back alpha compositing (the "over" operator).
 *   [fd-clip]   compute_clipping_distances: one near / far distance per view,
 *               from the camera to the closest / farthest volume point, widened
 *               by a margin (30 mm by default).
 *   [fd-tf]     Transfer functions, piecewise_linear_channelwise: a per-channel
 *               piecewise-linear map over sorted knots (xp, yp) that extends
 *               its first and last segments, applied to the volume before ray
 *               casting.
 * Readings (the pages give no formulas for these):
 *   - the density factor f scales mu: the optical depth of a ray is
 *     tau = f dz sum_k mu_k; Beer-Lambert gives 1 - exp(-tau), the line
 *     integral gives tau;
 *   - alpha compositing treats each sample as a slab of thickness dz that
 *     emits its own value mu_k and absorbs with density f mu_k:
 *     alpha_k = 1 - exp(-f mu_k dz), T_k = prod_{j<k} (1 - alpha_j), and the
 *     front-to-back over operator accumulates I = sum_k T_k alpha_k mu_k;
 *   - the transfer function acts on voxels (mu_v = tf_c(x_v)), then the
 *     volume of mu is sampled trilinearly as everywhere else;
 *   - the near/far mode uses the box's closest point and farthest corner
 *     (near not below 0), samples the midpoints of [near, far] on every ray of
 *     the view, and reads 0 outside the volume (grid_sample's zero padding:
 *     a trilinear corner outside [0, n-1] holds 0); with far <= near a ray
 *     renders 0. */

#define ORACLE_ALPHA_COMPOSITE 2
#define ORACLE_CLIP_BOX 0
#define ORACLE_CLIP_NEAR_FAR 1

/* [fd-tf] the piecewise-linear map of one channel.  Segment i spans
 * [xp[i], xp[i+1]); below xp[1] segment 0 applies and from xp[K-2] on segment
 * K-2, which extends both end segments.  *slope receives the segment's slope
 * (one-sided at a knot: the segment on the right). */
static double transfer(const double *xp, const double *yp, int K, double x, double *slope)
{
    int i = 0;
    while (i < K - 2 && x >= xp[i + 1]) ++i;
    double m = (yp[i + 1] - yp[i]) / (xp[i + 1] - xp[i]);
    if (slope) *slope = m;
    return yp[i] + m * (x - xp[i]);
}

/* [fd-clip] near / far distances of a camera centre C from the box
 * [-E/2, E/2]: the closest point of the box (0 inside it) and the farthest
 * corner, then the margin. */
static void near_far(const double C[3], const double E[3], double margin, double *t_near,
                     double *t_far)
{
    double dn2 = 0.0, df2 = 0.0;
    for (int a = 0; a < 3; ++a) {
        double h = 0.5 * E[a];
        double dn = 0.0;
        if (C[a] < -h) dn = -h - C[a];
        if (C[a] > h) dn = C[a] - h;
        double df = fabs(C[a]) + h;
        dn2 += dn * dn;
        df2 += df * df;
    }
    double tn = sqrt(dn2) - margin;
    *t_near = tn > 0.0 ? tn : 0.0;
    *t_far = sqrt(df2) + margin;
}

/* The eight trilinear corners of q in a volume of n voxels: clamp to edge
 * (zero_pad = 0) as in the forward above, or zero padding (zero_pad = 1), where
 * a corner outside [0, n-1] holds 0 and its weight is dropped. */
static void render_corners(const long n[3], const double q[3], int zero_pad, long off[8],
                           double w[8])
{
    long lo[3];
    double f[3];
    for (int a = 0; a < 3; ++a) {
        double fl = floor(q[a]);
        f[a] = q[a] - fl;
        lo[a] = (long)fl;
    }
    for (int c = 0; c < 8; ++c) {
        long idx[3];
        double wt = 1.0;
        int outside = 0;
        for (int a = 0; a < 3; ++a) {
            int up = (c >> a) & 1;
            long i = lo[a] + up;
            wt *= up ? f[a] : 1.0 - f[a];
            if (i < 0 || i > n[a] - 1) outside = 1;
            idx[a] = clamp_index(i, n[a]);
        }
        off[c] = (idx[2] * n[1] + idx[1]) * n[0] + idx[0];
        w[c] = (zero_pad && outside) ? 0.0 : wt;
    }
}

typedef struct {
    long n[3];
    double s[3], E[3];
    int n_samples, mode, clip, zero_pad;
    double f, margin;
} render_params_t;

/* Sample range of one ray: [t0, t1] of the box clip, or the view's near/far.
 * Returns 0 when the ray renders nothing. */
static int render_range(const render_params_t *P, const oracle_ray_t *ray, double *t0,
                        double *t1)
{
    if (P->clip == ORACLE_CLIP_BOX) {
        *t0 = ray->t0;
        *t1 = ray->t1;
        return ray->hit;
    }
    near_far(ray->C, P->E, P->margin, t0, t1);
    return *t1 > *t0;
}

/* Sample values mu_k (k = 0..N-1) of one ray at t0 + (k + 1/2) dz, and, when
 * off/w are given, their corners and weights (8 per sample). */
static void render_samples(const render_params_t *P, const double *mu, const oracle_ray_t *ray,
                           double t0, double dz, double *vals, long *off, double *w)
{
    for (int k = 0; k < P->n_samples; ++k) {
        double t = t0 + ((double)k + 0.5) * dz;
        double q[3];
        for (int a = 0; a < 3; ++a)
            q[a] = (ray->C[a] + t * ray->d[a] + 0.5 * P->E[a]) / P->s[a] - 0.5;
        long o[8];
        double wt[8];
        render_corners(P->n, q, P->zero_pad, o, wt);
        double v = 0.0;
        for (int c = 0; c < 8; ++c) v += wt[c] * mu[o[c]];
        vals[k] = v;
        if (off) {
            memcpy(off + 8L * k, o, sizeof(o));
            memcpy(w + 8L * k, wt, sizeof(wt));
        }
    }
}

/* Output of one ray from its samples; *tau receives the optical depth. */
static double render_output(const render_params_t *P, const double *vals, double dz,
                            double *tau)
{
    double sum = 0.0;
    for (int k = 0; k < P->n_samples; ++k) sum += vals[k];
    *tau = P->f * dz * sum;
    if (P->mode == ORACLE_BEER_LAMBERT) return -expm1(-*tau);
    if (P->mode == ORACLE_LINE_INTEGRAL) return *tau;
    /* front-to-back over operator */
    double I = 0.0, T = 1.0;
    for (int k = 0; k < P->n_samples; ++k) {
        double a = P->f * vals[k] * dz;
        double alpha = -expm1(-a);
        I += T * alpha * vals[k];
        T *= exp(-a);
    }
    return I;
}

/* mu volumes of all B * C channels in fp64: the input widened, or the
 * channel's transfer function applied voxel by voxel ([fd-tf]); slopes
 * (nullable) receives the transfer function's slope per voxel. */
static double *render_mu(const float *vol, long n_chvol, int C, long n_vox, const double *tf_xp,
                         const double *tf_yp, int tf_knots, double *slopes)
{
    double *mu = (double *)malloc(sizeof(double) * (size_t)(n_chvol * n_vox));
    if (!mu) return NULL;
    for (long cv = 0; cv < n_chvol; ++cv) {
        int ch = (int)(cv % C);
        for (long x = 0; x < n_vox; ++x) {
            long i = cv * n_vox + x;
            if (tf_xp) {
                double m;
                mu[i] = transfer(tf_xp + (long)ch * tf_knots, tf_yp + (long)ch * tf_knots,
                                 tf_knots, (double)vol[i], &m);
                if (slopes) slopes[i] = m;
            } else {
                mu[i] = (double)vol[i];
                if (slopes) slopes[i] = 1.0;
            }
        }
    }
    return mu;
}

static int render_check(int B, int C, int nz, int ny, int nx, const double *spacing,
                        int n_views, int H, int W, int n_samples, int mode, double f, int clip,
                        double margin, const double *tf_xp, const double *tf_yp, int tf_knots)
{
    if (B < 1 || C < 1 || nz < 1 || ny < 1 || nx < 1 || n_views < 0 || H < 0 || W < 0) return -1;
    if (n_views % B) return -1;
    if (n_samples < 1) return -1;
    if (mode != ORACLE_BEER_LAMBERT && mode != ORACLE_LINE_INTEGRAL &&
        mode != ORACLE_ALPHA_COMPOSITE)
        return -1;
    if (clip != ORACLE_CLIP_BOX && clip != ORACLE_CLIP_NEAR_FAR) return -1;
    if (!isfinite(f) || !isfinite(margin)) return -1;
    for (int a = 0; a < 3; ++a)
        if (!(spacing[a] > 0.0)) return -1;
    if (tf_xp || tf_yp) {
        if (!tf_xp || !tf_yp || tf_knots < 2) return -1;
        for (int c = 0; c < C; ++c)
            for (int k = 0; k + 1 < tf_knots; ++k)
                if (!(tf_xp[c * tf_knots + k + 1] > tf_xp[c * tf_knots + k])) return -1;
    }
    return 0;
}

static void render_init(render_params_t *P, int nz, int ny, int nx, const double *spacing,
                        int n_samples, int mode, double f, int clip, double margin)
{
    P->n[0] = nx;
    P->n[1] = ny;
    P->n[2] = nz;
    for (int a = 0; a < 3; ++a) {
        P->s[a] = spacing[a];
        P->E[a] = (double)P->n[a] * spacing[a];
    }
    P->n_samples = n_samples;
    P->mode = mode;
    P->f = f;
    P->clip = clip;
    P->zero_pad = clip == ORACLE_CLIP_NEAR_FAR;
    P->margin = margin;
}

/* Render B volumes of C channels ([fd-fwd]): vol is (B, C, nz, ny, nx) fp32,
 * poses n_views x 12 with n_views a multiple of B, out and tau (nullable) are
 * (n_views, C, H, W).  tf_xp / tf_yp (C x tf_knots, nullable) give a transfer
 * function per channel.  Returns 0, or -1 on invalid arguments or no memory. */
int oracle_render(const float *vol, int B, int C, int nz, int ny, int nx, const double *spacing,
                  const double *K, const double *poses, int n_views, int H, int W, int n_samples,
                  int mode, double f, int clip, double margin, const double *tf_xp,
                  const double *tf_yp, int tf_knots, double *out, double *tau, int n_threads)
{
    if (render_check(B, C, nz, ny, nx, spacing, n_views, H, W, n_samples, mode, f, clip, margin,
                     tf_xp, tf_yp, tf_knots))
        return -1;
    render_params_t P;
    render_init(&P, nz, ny, nx, spacing, n_samples, mode, f, clip, margin);
    long n_vox = (long)nx * ny * nz;
    double *mu = render_mu(vol, (long)B * C, C, n_vox, tf_xp, tf_yp, tf_knots, NULL);
    if (!mu) return -1;
    int views_per_vol = n_views / B;
    long n_out = (long)n_views * C * H * W;
    int failed = 0;
    set_threads(n_threads);
#pragma omp parallel
    {
        double *vals = (double *)malloc(sizeof(double) * (size_t)n_samples);
        if (!vals) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 64)
        for (long id = 0; id < n_out; ++id) {
            if (!vals) continue;
            int v = (int)(id / ((long)C * H * W));
            int ch = (int)((id / ((long)H * W)) % C);
            int r = (int)((id / W) % H);
            int c = (int)(id % W);
            const double *m = mu + ((long)(v / views_per_vol) * C + ch) * n_vox;
            oracle_ray_t ray;
            make_ray(K, poses + 12L * v, P.E, r, c, &ray);
            double t0, t1, t = 0.0, I = 0.0;
            if (render_range(&P, &ray, &t0, &t1)) {
                double dz = (t1 - t0) / (double)n_samples;
                render_samples(&P, m, &ray, t0, dz, vals, NULL, NULL);
                I = render_output(&P, vals, dz, &t);
            }
            out[id] = I;
            if (tau) tau[id] = t;
        }
        free(vals);
    }
    free(mu);
    return failed ? -1 : 0;
}

/* Volume gradient of oracle_render for upstream g = dL/dI (n_views, C, H, W),
 * with respect to the input volume x (B, C, nz, ny, nx):
 *   dL/dmu_v = sum over rays and samples of c_k w_corner, with
 *     Beer-Lambert      c_k = g f dz exp(-tau)
 *     line integral     c_k = g f dz
 *     alpha compositing c_k = g (T_k (alpha_k + f dz (1 - alpha_k) mu_k)
 *                                - f dz sum_{j>k} T_j alpha_j mu_j)
 *   (the last: d/dmu_k of sum_j T_j alpha_j mu_j, where mu_k enters its own
 *   alpha and emission and the transmittance of every later sample);
 *   dL/dx_v = dL/dmu_v tf'(x_v) (1 without a transfer function).
 * grad (B * C * nz * ny * nx doubles) is overwritten.  Threads get private
 * gradient buffers while (threads - 1) buffers fit in max_buffer_bytes.
 * Returns the thread count used, or -1. */
int oracle_render_adjoint(const float *vol, int B, int C, int nz, int ny, int nx,
                          const double *spacing, const double *K, const double *poses,
                          int n_views, int H, int W, int n_samples, int mode, double f, int clip,
                          double margin, const double *tf_xp, const double *tf_yp, int tf_knots,
                          const double *g, double *grad, int n_threads,
                          long long max_buffer_bytes)
{
    if (render_check(B, C, nz, ny, nx, spacing, n_views, H, W, n_samples, mode, f, clip, margin,
                     tf_xp, tf_yp, tf_knots))
        return -1;
    render_params_t P;
    render_init(&P, nz, ny, nx, spacing, n_samples, mode, f, clip, margin);
    long n_vox = (long)nx * ny * nz;
    long n_all = (long)B * C * n_vox;
    double *slopes = (double *)malloc(sizeof(double) * (size_t)n_all);
    double *mu = slopes ? render_mu(vol, (long)B * C, C, n_vox, tf_xp, tf_yp, tf_knots, slopes)
                        : NULL;
    if (!mu) {
        free(slopes);
        return -1;
    }
    memset(grad, 0, sizeof(double) * (size_t)n_all);
    int T = n_threads > 0 ? n_threads : 1;
#ifndef _OPENMP
    T = 1;
#endif
    while (T > 1 && (long long)(T - 1) * n_all * (long long)sizeof(double) > max_buffer_bytes) --T;
    double **bufs = (double **)calloc((size_t)T, sizeof(double *));
    int failed = bufs == NULL;
    if (bufs) {
        bufs[0] = grad;
        for (int i = 1; i < T; ++i) {
            bufs[i] = (double *)calloc((size_t)n_all, sizeof(double));
            if (!bufs[i]) failed = 1;
        }
    }
    int views_per_vol = B > 0 ? n_views / B : 1;
    long n_out = (long)n_views * C * H * W;
    if (!failed) {
        set_threads(T);
#pragma omp parallel num_threads(T)
        {
#ifdef _OPENMP
            double *acc = bufs[omp_get_thread_num()];
#else
            double *acc = bufs[0];
#endif
            double *vals = (double *)malloc(sizeof(double) * (size_t)n_samples);
            double *coef = (double *)malloc(sizeof(double) * (size_t)n_samples);
            long *off = (long *)malloc(sizeof(long) * 8 * (size_t)n_samples);
            double *w = (double *)malloc(sizeof(double) * 8 * (size_t)n_samples);
            int ok = vals && coef && off && w;
            if (!ok) {
#pragma omp atomic write
                failed = 1;
            }
#pragma omp for schedule(dynamic, 64)
            for (long id = 0; id < n_out; ++id) {
                if (!ok) continue;
                int v = (int)(id / ((long)C * H * W));
                int ch = (int)((id / ((long)H * W)) % C);
                int r = (int)((id / W) % H);
                int c = (int)(id % W);
                long base = ((long)(v / views_per_vol) * C + ch) * n_vox;
                oracle_ray_t ray;
                make_ray(K, poses + 12L * v, P.E, r, c, &ray);
                double t0, t1, tau;
                if (!render_range(&P, &ray, &t0, &t1)) continue;
                double dz = (t1 - t0) / (double)n_samples;
                render_samples(&P, mu + base, &ray, t0, dz, vals, off, w);
                render_output(&P, vals, dz, &tau);
                if (P.mode == ORACLE_BEER_LAMBERT) {
                    for (int k = 0; k < n_samples; ++k) coef[k] = g[id] * f * dz * exp(-tau);
                } else if (P.mode == ORACLE_LINE_INTEGRAL) {
                    for (int k = 0; k < n_samples; ++k) coef[k] = g[id] * f * dz;
                } else {
                    /* transmittance in front of each sample, then the later
                     * samples' emission summed back to front */
                    double Tk = 1.0;
                    for (int k = 0; k < n_samples; ++k) {
                        double a = f * vals[k] * dz;
                        coef[k] = Tk;          /* T_k for now */
                        Tk *= exp(-a);
                    }
                    double later = 0.0;
                    for (int k = n_samples - 1; k >= 0; --k) {
                        double a = f * vals[k] * dz;
                        double alpha = -expm1(-a);
                        double Tf = coef[k];
                        coef[k] = g[id] * (Tf * (alpha + f * dz * (1.0 - alpha) * vals[k]) -
                                           f * dz * later);
                        later += Tf * alpha * vals[k];
                    }
                }
                for (int k = 0; k < n_samples; ++k)
                    for (int cn = 0; cn < 8; ++cn)
                        acc[base + off[8L * k + cn]] += coef[k] * w[8L * k + cn];
            }
            free(vals);
            free(coef);
            free(off);
            free(w);
        }
    }
    if (bufs) {
        for (int i = 1; i < T; ++i) {
            if (bufs[i] && !failed)
                for (long x = 0; x < n_all; ++x) grad[x] += bufs[i][x];
            free(bufs[i]);
        }
        free(bufs);
    }
    if (!failed)
        for (long x = 0; x < n_all; ++x) grad[x] *= slopes[x];
    free(mu);
    free(slopes);
    return failed ? -1 : T;
}

/* Value and q-gradient of the render field (clamp to edge, or zero padding in
 * the near/far mode) at q: the corner values are those render_corners reads
 * (0 for a corner outside the volume with zero padding), the value is their
 * trilinear blend and each gradient component the derivative of the corner
 * weights along that axis times the corner values. */
static double render_value_grad(const render_params_t *P, const double *mu, const double q[3],
                                double gq[3])
{
    long lo[3];
    double f[3];
    for (int a = 0; a < 3; ++a) {
        double fl = floor(q[a]);
        f[a] = q[a] - fl;
        lo[a] = (long)fl;
    }
    double val = 0.0;
    gq[0] = gq[1] = gq[2] = 0.0;
    for (int c = 0; c < 8; ++c) {
        long idx[3];
        int outside = 0;
        double w = 1.0;
        for (int a = 0; a < 3; ++a) {
            int up = (c >> a) & 1;
            long i = lo[a] + up;
            if (i < 0 || i > P->n[a] - 1) outside = 1;
            idx[a] = clamp_index(i, P->n[a]);
            w *= up ? f[a] : 1.0 - f[a];
        }
        double v = (P->zero_pad && outside) ? 0.0 : mu[(idx[2] * P->n[1] + idx[1]) * P->n[0] + idx[0]];
        val += w * v;
        for (int a = 0; a < 3; ++a) {
            double dw = ((c >> a) & 1) ? 1.0 : -1.0;
            for (int b = 0; b < 3; ++b) {
                if (b == a) continue;
                dw *= ((c >> b) & 1) ? f[b] : 1.0 - f[b];
            }
            gq[a] += dw * v;
        }
    }
    return val;
}

/* Pose gradient of oracle_render in every mode and both clips: for
 * L = sum_p g_p out_p, grad_pose[12 v + e] receives dL/dP_v[e] for view v's
 * 3x4 row-major [R | t], summed over its channels (flashdrr API,
 * VolumeRaycaster class text: rendering is differentiable with respect to the
 * view matrices, in either integration mode of __init__).
 *
 * Plain forward-mode differentiation of oracle_render, one pose entry theta at
 * a time, as oracle_pose_gradient does for the plain forward: the tangents of
 * the camera centre dC = -dR^T t - R^T dt and of the unit direction
 * dd = (dw - d (d . dw)) / |w| (w = R^T K^-1 m); of the range ends -- with the
 * box clip the bounding planes move them, dt = -(dC_a + t dd_a) / d_a for the
 * entry (exit) axis a (the start stays 0 at the source); in the near/far mode
 * near = |e| - margin with e the offset of C from the box's closest point and
 * far = |(|C_a| + E_a/2)_a| + margin move with C alone, d near = e . dC / |e|
 * (0 while near is held at 0), d far = sum_a (|C_a| + E_a/2) sign(C_a) dC_a /
 * (far - margin) --; of dz and of each sample position
 * dp_k = dC + dt_k d + t_k dd, and of each sample value
 * dv_k = grad v(q_k) . dp_k / s.  Then through the output:
 *   Beer-Lambert and line integral: tau = f dz sum v_k,
 *     dtau = f (ddz sum v_k + dz sum dv_k), dout = exp(-tau) dtau or dtau;
 *   compositing, a_k = f v_k dz: da_k = f (dv_k dz + v_k ddz),
 *     alpha_k = 1 - exp(-a_k), dalpha_k = exp(-a_k) da_k,
 *     T_k = exp(-sum_{j<k} a_j), dT_k = -T_k sum_{j<k} da_j,
 *     dI = sum_k (dT_k alpha_k v_k + T_k dalpha_k v_k + T_k alpha_k dv_k),
 *   with T carried as the running product of the forward.
 * Rays that render nothing contribute nothing.  Returns 0, or -1 on invalid
 * arguments or no memory. */
int oracle_render_pose_gradient(const float *vol, int B, int C, int nz, int ny, int nx,
                                const double *spacing, const double *K, const double *poses,
                                int n_views, int H, int W, int n_samples, int mode, double f,
                                int clip, double margin, const double *tf_xp,
                                const double *tf_yp, int tf_knots, const double *g,
                                double *grad_pose, int n_threads)
{
    if (render_check(B, C, nz, ny, nx, spacing, n_views, H, W, n_samples, mode, f, clip, margin,
                     tf_xp, tf_yp, tf_knots))
        return -1;
    render_params_t P;
    render_init(&P, nz, ny, nx, spacing, n_samples, mode, f, clip, margin);
    long n_vox = (long)nx * ny * nz;
    double *mu = render_mu(vol, (long)B * C, C, n_vox, tf_xp, tf_yp, tf_knots, NULL);
    if (!mu) return -1;
    memset(grad_pose, 0, sizeof(double) * 12 * (size_t)n_views);
    int views_per_vol = n_views / B;
    set_threads(n_threads);
    for (int v = 0; v < n_views; ++v) {
        const double *pose = poses + 12L * v;
        double acc[12] = {0};
#pragma omp parallel
        {
            double mine[12] = {0};
#pragma omp for schedule(dynamic, 16)
            for (long id = 0; id < (long)C * H * W; ++id) {
                int ch = (int)(id / ((long)H * W));
                int r = (int)((id / W) % H);
                int c = (int)(id % W);
                double gp = g[(long)v * C * H * W + id];
                if (gp == 0.0) continue;
                const double *m = mu + ((long)(v / views_per_vol) * C + ch) * n_vox;
                oracle_ray_t ray;
                make_ray(K, pose, P.E, r, c, &ray);
                double t0, t1;
                if (!render_range(&P, &ray, &t0, &t1)) continue;
                /* unnormalised direction w = R^T K^-1 m and its length */
                double mp[3] = { c + 0.5, r + 0.5, 1.0 }, u[3], w[3];
                solve3(K, mp, u);
                for (int a = 0; a < 3; ++a)
                    w[a] = pose[0 * 4 + a] * u[0] + pose[1 * 4 + a] * u[1] + pose[2 * 4 + a] * u[2];
                double len = sqrt(w[0] * w[0] + w[1] * w[1] + w[2] * w[2]);
                /* box clip: the planes that bound the range */
                int a_in = -1, a_out = -1;
                if (clip == ORACLE_CLIP_BOX) {
                    double t_entry = -INFINITY, t_exit = INFINITY;
                    for (int a = 0; a < 3; ++a) {
                        if (ray.d[a] == 0.0) continue;
                        double ta = (-0.5 * P.E[a] - ray.C[a]) / ray.d[a];
                        double tb = (0.5 * P.E[a] - ray.C[a]) / ray.d[a];
                        double tmin = ta < tb ? ta : tb, tmax = ta < tb ? tb : ta;
                        if (tmin > t_entry) { t_entry = tmin; a_in = a; }
                        if (tmax < t_exit) { t_exit = tmax; a_out = a; }
                    }
                    if (!(t_entry > 0.0)) a_in = -1;
                }
                /* near/far: gradients of near and far with respect to C */
                double gnear[3] = {0.0, 0.0, 0.0}, gfar[3] = {0.0, 0.0, 0.0};
                if (clip == ORACLE_CLIP_NEAR_FAR) {
                    double e[3], ne = 0.0, fa2 = 0.0;
                    for (int a = 0; a < 3; ++a) {
                        double h = 0.5 * P.E[a];
                        e[a] = ray.C[a] < -h ? ray.C[a] + h : (ray.C[a] > h ? ray.C[a] - h : 0.0);
                        ne += e[a] * e[a];
                        fa2 += (fabs(ray.C[a]) + h) * (fabs(ray.C[a]) + h);
                    }
                    ne = sqrt(ne);
                    double fa = sqrt(fa2);
                    for (int a = 0; a < 3; ++a) {
                        double h = 0.5 * P.E[a];
                        if (ne - margin > 0.0) gnear[a] = e[a] / ne;
                        double sg = ray.C[a] > 0.0 ? 1.0 : (ray.C[a] < 0.0 ? -1.0 : 0.0);
                        gfar[a] = (fabs(ray.C[a]) + h) * sg / fa;
                    }
                }
                double dz = (t1 - t0) / (double)n_samples;
                double dC[12][3], dd[12][3], dt0[12], ddz[12];
                for (int j = 0; j < 12; ++j) {
                    double dR[9] = {0}, dtv[3] = {0}, dw[3];
                    if (j < 9) dR[j] = 1.0; else dtv[j - 9] = 1.0;
                    for (int a = 0; a < 3; ++a) {
                        dC[j][a] = -(dR[0 * 3 + a] * pose[0 * 4 + 3] + dR[1 * 3 + a] * pose[1 * 4 + 3] +
                                     dR[2 * 3 + a] * pose[2 * 4 + 3])
                                   - (pose[0 * 4 + a] * dtv[0] + pose[1 * 4 + a] * dtv[1] +
                                      pose[2 * 4 + a] * dtv[2]);
                        dw[a] = dR[0 * 3 + a] * u[0] + dR[1 * 3 + a] * u[1] + dR[2 * 3 + a] * u[2];
                    }
                    double ddw = ray.d[0] * dw[0] + ray.d[1] * dw[1] + ray.d[2] * dw[2];
                    for (int a = 0; a < 3; ++a) dd[j][a] = (dw[a] - ray.d[a] * ddw) / len;
                    double dt1;
                    if (clip == ORACLE_CLIP_BOX) {
                        dt0[j] = a_in >= 0 ? -(dC[j][a_in] + t0 * dd[j][a_in]) / ray.d[a_in] : 0.0;
                        dt1 = -(dC[j][a_out] + t1 * dd[j][a_out]) / ray.d[a_out];
                    } else {
                        dt0[j] = gnear[0] * dC[j][0] + gnear[1] * dC[j][1] + gnear[2] * dC[j][2];
                        dt1 = gfar[0] * dC[j][0] + gfar[1] * dC[j][1] + gfar[2] * dC[j][2];
                    }
                    ddz[j] = (dt1 - dt0[j]) / (double)n_samples;
                }
                /* march: value and tangents of each sample, then the output */
                double sum_v = 0.0, sum_dv[12] = {0};
                double T = 1.0, dT[12] = {0}, dI[12] = {0};
                for (int k = 0; k < n_samples; ++k) {
                    double tk = t0 + ((double)k + 0.5) * dz, q[3], gq[3], dv[12];
                    for (int a = 0; a < 3; ++a)
                        q[a] = (ray.C[a] + tk * ray.d[a] + 0.5 * P.E[a]) / P.s[a] - 0.5;
                    double val = render_value_grad(&P, m, q, gq);
                    for (int j = 0; j < 12; ++j) {
                        double dtk = dt0[j] + ((double)k + 0.5) * ddz[j];
                        dv[j] = 0.0;
                        for (int a = 0; a < 3; ++a) {
                            double dp = dC[j][a] + dtk * ray.d[a] + tk * dd[j][a];
                            dv[j] += gq[a] * dp / P.s[a];
                        }
                    }
                    if (mode != ORACLE_ALPHA_COMPOSITE) {
                        sum_v += val;
                        for (int j = 0; j < 12; ++j) sum_dv[j] += dv[j];
                        continue;
                    }
                    double a_k = f * val * dz, keep = exp(-a_k);
                    double alpha = -expm1(-a_k);
                    for (int j = 0; j < 12; ++j) {
                        double da = f * (dv[j] * dz + val * ddz[j]);
                        double dalpha = keep * da;
                        dI[j] += dT[j] * alpha * val + T * dalpha * val + T * alpha * dv[j];
                        dT[j] = dT[j] * keep - T * keep * da;
                    }
                    T *= keep;
                }
                if (mode != ORACLE_ALPHA_COMPOSITE) {
                    double tau = f * dz * sum_v;
                    double dout = mode == ORACLE_BEER_LAMBERT ? exp(-tau) : 1.0;
                    for (int j = 0; j < 12; ++j)
                        dI[j] = dout * f * (ddz[j] * sum_v + dz * sum_dv[j]);
                }
                for (int j = 0; j < 12; ++j) mine[j] += gp * dI[j];
            }
#pragma omp critical
            for (int j = 0; j < 12; ++j) acc[j] += mine[j];
        }
        for (int rr = 0; rr < 3; ++rr) {
            for (int cc = 0; cc < 3; ++cc) grad_pose[12L * v + rr * 4 + cc] = acc[rr * 3 + cc];
            grad_pose[12L * v + rr * 4 + 3] = acc[9 + rr];
        }
    }
    free(mu);
    return 0;
}

/* Near / far range of the near/far mode for one view, for pins: out = (near,
 * far).  extent = (Ex, Ey, Ez). */
void oracle_view_range(const double *extent, const double *pose, double margin, double *out)
{
    double C[3];
    camera_centre(pose, C);
    near_far(C, extent, margin, &out[0], &out[1]);
}

/* ------------------------------------------------- Gaussian-Poisson surrogate */

/* flashdrr.rendering API, VolumeRaycaster.apply_poisson: Gaussian noise of
 * standard deviation sqrt(T / i0) added to a transmission map T, clamped to
 * [0, 1]; a smooth, differentiable surrogate for photon (Poisson) noise.  The
 * standard-normal draws z are an input.  Readings: a transmission below 0 has
 * no noise (its standard deviation is taken as 0); the derivative follows
 * torch.clamp (passed through where min <= value <= max, else 0) and, where
 * T <= 0, omits the noise term, whose derivative z / (2 sqrt(T i0)) has no
 * finite value there. */
void oracle_poisson_surrogate(const double *T, const double *z, long n, double i0, double *out,
                              const double *g, double *grad)
{
    for (long i = 0; i < n; ++i) {
        double t = T[i];
        double sd = t > 0.0 ? sqrt(t / i0) : 0.0;
        double v = t + z[i] * sd;
        double o = v < 0.0 ? 0.0 : (v > 1.0 ? 1.0 : v);
        out[i] = o;
        if (grad) {
            double pass = (v >= 0.0 && v <= 1.0) ? 1.0 : 0.0;
            double dv = 1.0 + (t > 0.0 ? z[i] / (2.0 * sqrt(t * i0)) : 0.0);
            grad[i] = g[i] * pass * dv;
        }
    }
}

/* Build information for the Python loader. */
int oracle_abi_version(void) { return 1; }

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
