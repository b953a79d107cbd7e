// drr_pose.hip -- gradient of the DRR with respect to each view's pose.
//
// flashdrr.rendering API, VolumeRaycaster class text: rendering is
// differentiable with respect to the input volume and the view matrices
// (flashdrr README, Features: gradients flow through both the volume and the
// camera parameters).  For L = sum_p g_p I_p the kernels return dL/dP_v for
// every view's 3x4 world-to-camera [R | t], the twelve entries treated as
// independent (a caller chains them through its own rotation parameters).
//
// Per ray (C = -R^T t, unnormalised direction w = R^T u with u = K^-1 m,
// d = w / |w|, clipped range [t0, t1], dz = (t1 - t0) / N, samples
// p_k = C + (t0 + (k + 1/2) dz) d):
//   ds = ddz S0 + dz sum_k grad mu(p_k) . dp_k,   S0 = sum_k mu(p_k),
// which with G0 = sum_k grad mu_k and G1 = sum_k b_k grad mu_k,
// b_k = (k + 1/2) / N, collapses to
//   ds = A . dC + Bv . dd + beta0 dt0 + beta1 dt1,
//   A = dz G0,  Bv = dz (t0 G0 + (t1 - t0) G1),
//   beta0 = -S0 / N + dz (G0 - G1) . d,  beta1 = S0 / N + dz G1 . d.
// The range ends move with the planes that bound them: t = (plane - C_a) / d_a
// gives dt = -(dC_a + t dd_a) / d_a (and dt0 = 0 when the range starts at the
// source), so ds = Ac . dC + Bd . dd; with dd = (I - d d^T) dw / |w| this is
// ds = Ac . dC + Bw . dw, Bw = (I - d d^T) Bd / |w|.  Finally dC/dR_ij =
// -t_i e_j, dw/dR_ij = u_i e_j, dC/dt_i = -R_i. (row i), so with y = g dI/ds
// summed over a view's rays, P = sum y Ac and Q_ij = sum y u_i Bw_j:
//   dL/dR_ij = -t_i P_j + Q_ij,   dL/dt_i = -sum_a R_ia P_a.
// In general dI = sum_k c_k dv_k + D ddz with c_k = dI/dv_k and D = dI/ddz at
// fixed values, and the same collapse holds with G0 = sum_k c_k grad v_k,
// G1 = sum_k c_k b_k grad v_k and beta0 = (G0 - G1) . d - D / N,
// beta1 = G1 . d + D / N (A = G0, Bv = t0 G0 + (t1 - t0) G1).  Beer-Lambert
// and the line integral have c_k = dz and D = S0 (times f exp(-f s) or f);
// compositing (flashdrr API, VolumeRaycaster.__init__: use_beer_lambert =
// False) has the over operator's per-sample coefficient and
// D = f sum_k T_k v_k ((1 - alpha_k) v_k - alpha_k P_k), P_k = sum_{j<k} v_j.
// In the near/far mode (flashdrr compute_clipping_distances) the range ends
// are the view's near and far, functions of C alone: dt0 = n0 . dC and
// dt1 = n1 . dC with n0, n1 their gradients, so A gains beta0 n0 + beta1 n1
// and no plane terms enter.
// The march steps 32.32 fixed-point positions (re-anchored on fp64 every eight
// samples, every four in the LDS-staged march), interpolates in fp32 and
// accumulates S0, G0 and sum_k k grad mu_k per ray in fp64 (from fp32 sums of
// each group; compositing's sums per sample); the chain rule runs in fp64 and
// the view sums in fp64 atomics.
#include <limits.h>

#include "drr_device.hpp"
#include "drr_internal.hpp"
#include "drr_sample.hpp"
#include "drr_stage.hpp"

namespace drr {

// Ray geometry of the pose gradient: the same slab clip as ray_setup, the axes
// of the planes that bound the range, and the sample positions in fp64.
struct RayFrame {
    double C[3], d[3], u[3];
    double q0[3], dq[3];     // continuous index of sample 0 and the step, fp64, times 2^32
    double len, t0, t1;
    int a_in;      // entry plane axis, -1 when the range starts at the source (or near/far)
    int a_out;     // exit plane axis (-1 in the near/far mode)
    double gn[3], gf[3];     // near/far mode: gradients of t0 and t1 with respect to C, else 0
};

__device__ inline bool ray_frame(const ViewGeom& G, const double Ki[9], const VolumeDesc& V,
                                 int r, int c, int N, RayFrame& F)
{
    const double m0 = (double)c + 0.5, m1 = (double)r + 0.5;
    double w[3];
#pragma unroll
    for (int a = 0; a < 3; ++a) {
        F.u[a] = Ki[a * 3 + 0] * m0 + Ki[a * 3 + 1] * m1 + Ki[a * 3 + 2];
        w[a] = G.M[a * 3 + 0] * m0 + G.M[a * 3 + 1] * m1 + G.M[a * 3 + 2];
        F.C[a] = G.C[a];
    }
    F.len = sqrt(w[0] * w[0] + w[1] * w[1] + w[2] * w[2]);
    const double inv_len = 1.0 / F.len;
    double t_entry = -__builtin_inf(), t_exit = __builtin_inf();
    int a_in = -1, a_out = -1;
    bool inside = true;
#pragma unroll
    for (int a = 0; a < 3; ++a) {
        F.d[a] = w[a] * inv_len;
        const double lo = -V.half_e[a], hi = V.half_e[a];
        if (F.d[a] == 0.0) {
            inside = inside && !(G.C[a] < lo || G.C[a] > hi);
        } else {
            const double ta = (lo - G.C[a]) / F.d[a];
            const double tb = (hi - G.C[a]) / F.d[a];
            const double tmin = fmin(ta, tb), tmax = fmax(ta, tb);
            if (tmin > t_entry) { t_entry = tmin; a_in = a; }
            if (tmax < t_exit) { t_exit = tmax; a_out = a; }
        }
    }
    F.t0 = fmax(t_entry, 0.0);
    F.t1 = t_exit;
    if (!inside || !(F.t1 > F.t0)) return false;
    if (!(t_entry > 0.0)) a_in = -1;
    F.a_in = a_in;
    F.a_out = a_out;
#pragma unroll
    for (int a = 0; a < 3; ++a) F.gn[a] = F.gf[a] = 0.0;
    const double dz = (F.t1 - F.t0) / (double)N;
    const double ts = F.t0 + 0.5 * dz;
#pragma unroll
    for (int a = 0; a < 3; ++a) {
        F.q0[a] = ((G.C[a] + ts * F.d[a]) * V.inv_s[a] + V.q_off[a]) * 4294967296.0;
        F.dq[a] = (dz * F.d[a] * V.inv_s[a]) * 4294967296.0;
    }
    return true;
}

// Near/far mode: the ray of pixel (r, c) over the view's [near, far] (the
// forward's view_near_far), no plane axes, and the gradients of near and far
// with respect to the camera centre C: near = |e| - margin with e the offset
// of C from the box's closest point (gradient e / |e|, 0 while near is held at
// 0), far = |(|C_a| + E_a / 2)_a| + margin (gradient (|C_a| + E_a / 2)
// sign(C_a) / (far - margin)).  Returns false when the range is empty.
__device__ inline bool ray_frame_range(const ViewGeom& G, const double Ki[9], const VolumeDesc& V,
                                       float margin, int r, int c, int N, RayFrame& F)
{
    double t_near, t_far;
    view_near_far(G, V, margin, t_near, t_far);
    if (!(t_far > t_near)) return false;
    const double m0 = (double)c + 0.5, m1 = (double)r + 0.5;
    double w[3];
#pragma unroll
    for (int a = 0; a < 3; ++a) {
        F.u[a] = Ki[a * 3 + 0] * m0 + Ki[a * 3 + 1] * m1 + Ki[a * 3 + 2];
        w[a] = G.M[a * 3 + 0] * m0 + G.M[a * 3 + 1] * m1 + G.M[a * 3 + 2];
        F.C[a] = G.C[a];
    }
    F.len = sqrt(w[0] * w[0] + w[1] * w[1] + w[2] * w[2]);
    const double inv_len = 1.0 / F.len;
    F.t0 = t_near;
    F.t1 = t_far;
    F.a_in = F.a_out = -1;
    double e[3], ne = 0.0, fa = 0.0;
#pragma unroll
    for (int a = 0; a < 3; ++a) {
        F.d[a] = w[a] * inv_len;
        const double h = V.half_e[a], ca = G.C[a];
        e[a] = ca < -h ? ca + h : (ca > h ? ca - h : 0.0);
        ne += e[a] * e[a];
        fa += (fabs(ca) + h) * (fabs(ca) + h);
    }
    ne = sqrt(ne);
    fa = sqrt(fa);
    const bool near_moves = ne - (double)margin > 0.0;
#pragma unroll
    for (int a = 0; a < 3; ++a) {
        const double h = V.half_e[a], ca = G.C[a];
        F.gn[a] = near_moves ? e[a] / ne : 0.0;
        F.gf[a] = (fabs(ca) + h) * (ca > 0.0 ? 1.0 : (ca < 0.0 ? -1.0 : 0.0)) / fa;
    }
    const double dz = (F.t1 - F.t0) / (double)N;
    const double ts = F.t0 + 0.5 * dz;
#pragma unroll
    for (int a = 0; a < 3; ++a) {
        F.q0[a] = ((G.C[a] + ts * F.d[a]) * V.inv_s[a] + V.q_off[a]) * 4294967296.0;
        F.dq[a] = (dz * F.d[a] * V.inv_s[a]) * 4294967296.0;
    }
    return true;
}

// Samples [k_lo, k_hi) of a near/far frame whose continuous index lies in
// [-1, n) on every axis (the zero-padded support, as padded_support for the
// forward's march), widened by one sample each way; the others read only
// padding and add exactly 0.
__device__ inline void frame_support(const RayFrame& F, const VolumeDesc& V, int N, int& k_lo,
                                     int& k_hi)
{
    double lo = 0.0, hi = (double)N;
    bool none = false;
#pragma unroll
    for (int a = 0; a < 3; ++a) {
        const double q0 = F.q0[a] * 2.3283064365386963e-10;
        const double dq = F.dq[a] * 2.3283064365386963e-10;
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

// Sample k's position, evaluated in fp64 and rounded once to 32.32 fixed point
// (to nearest, ties to even, as to_fixed).  The frame holds the position and
// step times 2^32, a power of two that commutes with the rounding of the fma,
// so q 2^32 comes out exactly.  Positions lie inside the box and axes stay
// under 2^19 voxels (the library's 16384 limit), so q 2^32 + 1.5 2^52 lands in
// [2^52, 2^53) and its rounding leaves the rounded integer in the low mantissa
// bits.
__device__ inline int64_t sample_fixed(const RayFrame& F, int a, int k)
{
    constexpr double kMagic = 6755399441055744.0;       // 1.5 * 2^52
    const double q32 = fma((double)k, F.dq[a], F.q0[a]);
    return __double_as_longlong(q32 + kMagic) - __double_as_longlong(kMagic);
}

// Fixed-point step of the frame (to_fixed of the fp64 step).
__device__ inline int64_t step_fixed(const RayFrame& F, int a)
{
    return __double2ll_rn(F.dq[a]);
}

// A group of NG samples' terms summed in fp32: ps = sum v_i, pg = sum g_i and
// ph = sum i g_i, formed from the terms themselves (no additions to zero).
template <int NG>
__device__ inline void group_sums(const float v[NG], const float g[NG][3], float& ps, float pg[3],
                                  float ph[3])
{
    static_assert(NG >= 2, "a group has at least two samples");
    ps = v[0] + v[1];
#pragma unroll
    for (int i = 2; i < NG; ++i) ps += v[i];
#pragma unroll
    for (int a = 0; a < 3; ++a) {
        pg[a] = g[0][a] + g[1][a];
        ph[a] = g[1][a];
#pragma unroll
        for (int i = 2; i < NG; ++i) {
            pg[a] += g[i][a];
            ph[a] = fmaf((float)i, g[i][a], ph[a]);
        }
    }
}

// Workgroup sum of twelve doubles, returned to threads 0..11 (one each).
__device__ inline double block_sum12(const double v_in[12], double* red)
{
    double v[12];
#pragma unroll
    for (int i = 0; i < 12; ++i) {
        v[i] = v_in[i];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) v[i] += __shfl_xor(v[i], off, 64);
    }
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (lane == 0) {
#pragma unroll
        for (int i = 0; i < 12; ++i) red[wave * 12 + i] = v[i];
    }
    __syncthreads();
    double t = 0.0;
    if (threadIdx.x < 12)
        for (int w = 0; w < kBlock / 64; ++w) t += red[w * 12 + threadIdx.x];
    return t;
}

// A ray's contribution to its view's sums P (contrib[0..2]) and Q
// (contrib[3..11]) from y (g times what multiplies the ray's sums), G0 =
// sum_k c_k grad v_k and G1 = sum_k c_k b_k grad v_k (per mm) and Dn = D / N,
// chain rule in fp64.
__device__ inline void pose_contrib(const RayFrame& F, double y, const double G0[3],
                                    const double G1[3], double Dn, double contrib[12])
{
    double G0d = 0.0, G1d = 0.0;
#pragma unroll
    for (int a = 0; a < 3; ++a) {
        G0d += G0[a] * F.d[a];
        G1d += G1[a] * F.d[a];
    }
    const double beta0 = G0d - G1d - Dn;
    const double beta1 = G1d + Dn;
    double Ac[3], Bd[3];
#pragma unroll
    for (int a = 0; a < 3; ++a) {
        // gn, gf: the near/far range ends' gradients (0 with the box clip)
        Ac[a] = G0[a] + beta0 * F.gn[a] + beta1 * F.gf[a];
        Bd[a] = F.t0 * G0[a] + (F.t1 - F.t0) * G1[a];
    }
    // the planes that bound the range (unrolled selects: a run-time index into
    // these small arrays would put them in scratch memory)
#pragma unroll
    for (int a = 0; a < 3; ++a) {
        if (a == F.a_in) {
            Ac[a] -= beta0 / F.d[a];
            Bd[a] -= beta0 * F.t0 / F.d[a];
        }
        if (a == F.a_out) {
            Ac[a] -= beta1 / F.d[a];
            Bd[a] -= beta1 * F.t1 / F.d[a];
        }
    }
    const double dBd = Bd[0] * F.d[0] + Bd[1] * F.d[1] + Bd[2] * F.d[2];
    double Bw[3];
#pragma unroll
    for (int a = 0; a < 3; ++a) Bw[a] = (Bd[a] - F.d[a] * dBd) / F.len;
#pragma unroll
    for (int a = 0; a < 3; ++a) contrib[a] = y * Ac[a];
#pragma unroll
    for (int i = 0; i < 3; ++i)
#pragma unroll
        for (int j = 0; j < 3; ++j) contrib[3 + i * 3 + j] = y * F.u[i] * Bw[j];
}

// Beer-Lambert and line integral: c_k = dz, D = S0, y = g f exp(-f s) or g f,
// from the march sums s0 = sum_k mu_k, g0 = sum_k grad mu_k and
// h1 = sum_k k grad mu_k (per voxel index).
template <int MODE>
__device__ inline void pose_chain_rule(const RayFrame& F, const VolumeDesc& V, int N, float g,
                                       float density, double s0, const double g0[3],
                                       const double h1[3], double contrib[12])
{
    const double Nd = (double)N, dz = (F.t1 - F.t0) / Nd;
    double G0[3], G1[3];
#pragma unroll
    for (int a = 0; a < 3; ++a) {
        G0[a] = dz * g0[a] * V.inv_s[a];                          // per mm
        G1[a] = dz * (h1[a] + 0.5 * g0[a]) / Nd * V.inv_s[a];
    }
    const double s = dz * s0, f = (double)density;
    const double y = (double)g * f * (MODE == kBeerLambert ? exp(-f * s) : 1.0);
    pose_contrib(F, y, G0, G1, s0 / Nd, contrib);
}

// Compositing: running state and sums of one ray, samples added in order.
// With e_k = T_k (alpha_k + f dz (1 - alpha_k) v_k) and the running emission
// R_k = sum_{j<=k} T_j alpha_j v_j, sample k's coefficient is
// c_k = e_k - f dz (I - R_k) = W_k - f dz I with W_k = e_k + f dz R_k, so
// sum_k c_k X_k = sum_k W_k X_k - f dz I sum_k X_k: one pass gives it once
// I = R_{N-1} is known, without the forward's image.  T, R, the prefix
// P_k = sum_{j<k} v_j and every sum are fp64 (the difference above cancels
// where later samples carry little of I).
struct AlphaPoseSums {
    double T, R, P, D;
    double sw[3], swk[3], sx[3], sxk[3];
    float fdz;

    __device__ void init(float f_dz)
    {
        fdz = f_dz;
        T = 1.0;
        R = P = D = 0.0;
#pragma unroll
        for (int a = 0; a < 3; ++a) sw[a] = swk[a] = sx[a] = sxk[a] = 0.0;
    }

    // sample k: value v, gradient x (per voxel index)
    __device__ void add(int k, float v, const float x[3])
    {
        const float alpha = -expm1f(-(fdz * v));
        const float e = (float)T * (alpha + fdz * (1.0f - alpha) * v);
        D = fma(T * (double)v, (double)((1.0f - alpha) * v) - (double)alpha * P, D);
        R = fma(T, (double)(alpha * v), R);
        T = fma(-T, (double)alpha, T);
        P += (double)v;
        const double W = fma((double)fdz, R, (double)e);
        const double Wk = W * (double)k;
#pragma unroll
        for (int a = 0; a < 3; ++a) {
            sw[a] = fma(W, (double)x[a], sw[a]);
            swk[a] = fma(Wk, (double)x[a], swk[a]);
            sx[a] += (double)x[a];
            sxk[a] = fma((double)k, (double)x[a], sxk[a]);
        }
    }
};

// Compositing: y = g, D = f sum_k T_k v_k ((1 - alpha_k) v_k - alpha_k P_k).
__device__ inline void alpha_pose_chain(const RayFrame& F, const VolumeDesc& V, int N, float g,
                                        float density, const AlphaPoseSums& S,
                                        double contrib[12])
{
    const double Nd = (double)N, fdz = (double)S.fdz, I = S.R;
    double G0[3], G1[3];
#pragma unroll
    for (int a = 0; a < 3; ++a) {
        G0[a] = (S.sw[a] - fdz * I * S.sx[a]) * V.inv_s[a];
        G1[a] = ((S.swk[a] + 0.5 * S.sw[a]) - fdz * I * (S.sxk[a] + 0.5 * S.sx[a])) / Nd *
                V.inv_s[a];
    }
    pose_contrib(F, (double)g, G0, G1, (double)density * S.D / Nd, contrib);
}

// One group of samples' value and gradient terms, summed in fp32 (at most four
// terms), added to the ray's fp64 sums; the group starts at sample k.
__device__ inline void pose_add_group(int k, float ps, const float pg[3], const float ph[3],
                                      double& s0, double g0[3], double h1[3])
{
    s0 += (double)ps;
#pragma unroll
    for (int a = 0; a < 3; ++a) {
        g0[a] += (double)pg[a];
        h1[a] = fma((double)k, (double)pg[a], h1[a] + (double)ph[a]);
    }
}

// The tiles of a launch run over (view, channel) pairs (a tile lies in one
// pair); every channel of a view adds to that view's sums, and the density
// factor enters dI/ds (f exp(-f s) or f; the coefficients when compositing).
// `src` holds one channel-volume of `src_bytes` every b.src_stride bytes: the
// read plan's layout L, zero-padded (Cell or ZPair) in the near/far mode
// (CLIP = kClipNearFar), whose rays march only the samples of the padded
// support.
template <typename T, Layout L, int MODE, int CLIP>
__global__ __launch_bounds__(kBlock) void drr_pose_grad_kernel(
    const T* __restrict__ src, uint32_t src_bytes, VolumeDesc V, Intrinsics K,
    const float* __restrict__ poses, int H, int W, int N, int tiles_x, int tiles_per_view,
    Batch b, const float* __restrict__ grad_out, double* __restrict__ acc)
{
    constexpr bool ZP = CLIP == kClipNearFar;
    static_assert(!ZP || L == Layout::Cell || L == Layout::ZPair,
                  "the near/far mode reads zero-padded cells or z-pairs");
    __shared__ double red[(kBlock / 64) * 12];
    const int tile = xcd_contiguous_tile((int)blockIdx.x, (int)gridDim.x);
    const PixelCoord px = tile_pixel(tile, tiles_x, tiles_per_view);
    const int view = px.view / b.C, ch = px.view - view * b.C;
    const int cvol = (view / b.vpv) * b.C + ch;
    double contrib[12];
#pragma unroll
    for (int i = 0; i < 12; ++i) contrib[i] = 0.0;

    const float g = (px.r < H && px.c < W) ? grad_out[((size_t)px.view * H + px.r) * W + px.c]
                                           : 0.0f;
    RayFrame F;
    bool hit = false;
    if (g != 0.0f) {
        ViewGeom G;
        view_setup(poses + 12 * view, K, G);
        double Ki[9];
        intrinsics_inverse(K, Ki);
        hit = ZP ? ray_frame_range(G, Ki, V, b.margin, px.r, px.c, N, F)
                 : ray_frame(G, Ki, V, px.r, px.c, N, F);
    }
    if (hit) {
        const char* base = reinterpret_cast<const char*>(src) + (uint64_t)cvol * b.src_stride;
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, (int)src_bytes, kBufferWord3);
        int k_lo = 0, k_hi = N;
        if constexpr (ZP) frame_support(F, V, N, k_lo, k_hi);
        // fp64 ray sums: sum grad mu . d telescopes to about mu(exit) - mu(entry),
        // a small difference of large edge terms that fp32 sums over a whole ray
        // would round away (a group of eight fp32 terms is summed first)
        double s0 = 0.0, g0[3] = {0.0, 0.0, 0.0}, h1[3] = {0.0, 0.0, 0.0};
        AlphaPoseSums asum;
        if constexpr (MODE == kAlpha) asum.init(b.f * (float)((F.t1 - F.t0) / (double)N));
        // sample positions in 32.32 fixed point.  The gradient of trilinear mu
        // jumps where a sample crosses a cell face, so positions must not
        // drift from their fp64 values: each group of eight starts from its
        // first sample evaluated in fp64 and rounded once, and steps by the
        // rounded increment from there (at most 5.5 2^-32 voxel off).  Eight
        // samples' gathers in flight (against four: 0.596 -> 0.516 ms on 16
        // views of 200^2 from the z-pair copy)
        const int64_t dqx = step_fixed(F, 0), dqy = step_fixed(F, 1), dqz = step_fixed(F, 2);
        constexpr int kGroup = 8;
        int k = k_lo;
        for (; k + kGroup <= k_hi; k += kGroup) {
            SampleAddr A[kGroup];
            CornerVals c[kGroup];
            int64_t qx = sample_fixed(F, 0, k), qy = sample_fixed(F, 1, k), qz = sample_fixed(F, 2, k);
#pragma unroll
            for (int i = 0; i < kGroup; ++i) {
                A[i] = sample_addr<T, L, ZP>(V, qx, qy, qz);
                qx += dqx; qy += dqy; qz += dqz;
                serial_step(qx, qy, qz);
            }
#pragma unroll
            for (int i = 0; i < kGroup; ++i) gather<T, L>(rs, A[i], c[i]);
            __builtin_amdgcn_sched_barrier(0);
            float v[kGroup], gq[kGroup][3];
#pragma unroll
            for (int i = 0; i < kGroup; ++i) {
                v[i] = interpolate_grad(A[i], c[i], gq[i]);
                if constexpr (ZP) v[i] = interpolate_exact(A[i], c[i]);
            }
            if constexpr (MODE == kAlpha) {
#pragma unroll
                for (int i = 0; i < kGroup; ++i) asum.add(k + i, v[i], gq[i]);
            } else {
                // the group's sums in fp32 (four terms), then into the ray's fp64 sums
                float ps, pg[3], ph[3];
                group_sums<kGroup>(v, gq, ps, pg, ph);
                pose_add_group(k, ps, pg, ph, s0, g0, h1);
            }
        }
        for (; k < k_hi; ++k) {
            const SampleAddr A = sample_addr<T, L, ZP>(V, sample_fixed(F, 0, k),
                                                       sample_fixed(F, 1, k),
                                                       sample_fixed(F, 2, k));
            CornerVals c;
            gather<T, L>(rs, A, c);
            float gq[3];
            float v = interpolate_grad(A, c, gq);
            if constexpr (ZP) v = interpolate_exact(A, c);
            if constexpr (MODE == kAlpha) {
                asum.add(k, v, gq);
            } else {
                s0 += (double)v;
#pragma unroll
                for (int a = 0; a < 3; ++a) {
                    g0[a] += (double)gq[a];
                    h1[a] = fma((double)k, (double)gq[a], h1[a]);
                }
            }
        }
        if constexpr (MODE == kAlpha)
            alpha_pose_chain(F, V, N, g, b.f, asum, contrib);
        else
            pose_chain_rule<MODE>(F, V, N, g, b.f, s0, g0, h1, contrib);
    }
    const double t = block_sum12(contrib, red);
    if (threadIdx.x < 12 && t != 0.0) unsafeAtomicAdd(acc + 12 * view + threadIdx.x, t);
}

// LDS-staged pose gradient (box clip), the forward's staging applied to the
// pose march: the workgroup loads the box of voxels a chunk of its tile's
// samples touch (clamped, mapped by the transfer function when TF) and the
// samples read their corners from LDS.  Positions are stepped as in the linear
// kernel but in groups of four (each re-anchored on its fp64 position, then
// stepped by the rounded increment, at most 2.5 fixed-point units from each
// sample's own fp64 position), so the chunk box is widened by 4 units each way.
template <typename T, int MODE, bool TF>
__global__ __launch_bounds__(kBlock) void drr_pose_staged_kernel(
    const T* __restrict__ src, uint32_t src_bytes, VolumeDesc V, Intrinsics K,
    const float* __restrict__ poses, int H, int W, int N, int tiles_x, int tiles_per_view,
    Batch b, TransferFn tf, const float* __restrict__ grad_out, double* __restrict__ acc)
{
    __shared__ float box[kStageCap];
    __shared__ int ired[(kBlock / 64) * 6];
    __shared__ int bb[6];
    __shared__ double red[(kBlock / 64) * 12];
    const int tile = xcd_contiguous_tile((int)blockIdx.x, (int)gridDim.x);
    const PixelCoord px = tile_pixel(tile, tiles_x, tiles_per_view);
    const int view = px.view / b.C, ch = px.view - view * b.C;
    const int cvol = (view / b.vpv) * b.C + ch;
    double contrib[12];
#pragma unroll
    for (int i = 0; i < 12; ++i) contrib[i] = 0.0;

    const float g = (px.r < H && px.c < W) ? grad_out[((size_t)px.view * H + px.r) * W + px.c]
                                           : 0.0f;
    RayFrame F;
    bool hit = false;
    if (g != 0.0f) {
        ViewGeom G;
        view_setup(poses + 12 * view, K, G);
        double Ki[9];
        intrinsics_inverse(K, Ki);
        hit = ray_frame(G, Ki, V, px.r, px.c, N, F);
    }
    const char* base = reinterpret_cast<const char*>(src) + (uint64_t)cvol * b.src_stride;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, (int)src_bytes, kBufferWord3);
    int64_t dq[3] = {0, 0, 0};
    if (hit) {
#pragma unroll
        for (int a = 0; a < 3; ++a) dq[a] = step_fixed(F, a);
    }
    double s0 = 0.0, g0[3] = {0.0, 0.0, 0.0}, h1[3] = {0.0, 0.0, 0.0};
    AlphaPoseSums asum;
    if constexpr (MODE == kAlpha) {
        if (hit) asum.init(b.f * (float)((F.t1 - F.t0) / (double)N));
    }
    constexpr int64_t kSlack = 4;          // fixed-point units, see above
    constexpr int kGroup = 4;

    int S = N;
    int k0 = 0;
    while (k0 < N) {
        S = min(S, N - k0);
        int ext[3] = {1, 1, 1}, lo[3] = {0, 0, 0};
        long long vol_cells = 1;
        bool any;
        for (;;) {
            int lo_f[3] = {INT_MAX, INT_MAX, INT_MAX}, hi_f[3] = {INT_MAX, INT_MAX, INT_MAX};
            if (hit) {
#pragma unroll
                for (int a = 0; a < 3; ++a) {
                    const int64_t qa = sample_fixed(F, a, k0), qb = sample_fixed(F, a, k0 + S - 1);
                    lo_f[a] = fixed_floor(min(qa, qb) - kSlack);
                    hi_f[a] = fixed_floor(max(qa, qb) + kSlack);
                }
            }
            any = chunk_box(lo_f, hi_f, ired, bb, lo, ext, vol_cells);
            if (!any || vol_cells <= kStageCap || S == 1) break;
            S = max(1, S >> 1);
        }
        if (!any) break;                             // no ray of this tile contributes
        if (vol_cells <= kStageCap) {
            stage_fill<T, TF>(box, (int)vol_cells, rs, V, lo, ext, tf, ch);
            __syncthreads();
            if (hit) {
                const uint32_t sy = 4u * (uint32_t)ext[0], sz = 4u * (uint32_t)(ext[0] * ext[1]);
                const char* bx = reinterpret_cast<const char*>(box);
                const int64_t shift[3] = {(int64_t)lo[0] * kFixedOne, (int64_t)lo[1] * kFixedOne,
                                          (int64_t)lo[2] * kFixedOne};
                int k = k0;
                for (; k + kGroup <= k0 + S; k += kGroup) {
                    int64_t qx = sample_fixed(F, 0, k) - shift[0];
                    int64_t qy = sample_fixed(F, 1, k) - shift[1];
                    int64_t qz = sample_fixed(F, 2, k) - shift[2];
                    SampleAddr A[kGroup];
                    CornerVals c[kGroup];
#pragma unroll
                    for (int i = 0; i < kGroup; ++i) {
                        A[i].fx = fixed_frac(qx);
                        A[i].fy = fixed_frac(qy);
                        A[i].fz = fixed_frac(qz);
                        A[i].gxs = A[i].gzs = 1.0f;
                        A[i].o = box_offset(qx, qy, qz, sy, sz);
                        qx += dq[0]; qy += dq[1]; qz += dq[2];
                        serial_step(qx, qy, qz);
                    }
#pragma unroll
                    for (int i = 0; i < kGroup; ++i) box_corners(bx + A[i].o, sy, sz, c[i]);
                    float v[kGroup], gq[kGroup][3];
#pragma unroll
                    for (int i = 0; i < kGroup; ++i) v[i] = interpolate_grad(A[i], c[i], gq[i]);
                    if constexpr (MODE == kAlpha) {
#pragma unroll
                        for (int i = 0; i < kGroup; ++i) asum.add(k + i, v[i], gq[i]);
                    } else {
                        float ps, pg[3], ph[3];
                        group_sums<kGroup>(v, gq, ps, pg, ph);
                        pose_add_group(k, ps, pg, ph, s0, g0, h1);
                    }
                }
                for (; k < k0 + S; ++k) {
                    const int64_t qx = sample_fixed(F, 0, k) - shift[0];
                    const int64_t qy = sample_fixed(F, 1, k) - shift[1];
                    const int64_t qz = sample_fixed(F, 2, k) - shift[2];
                    SampleAddr A;
                    A.fx = fixed_frac(qx);
                    A.fy = fixed_frac(qy);
                    A.fz = fixed_frac(qz);
                    A.gxs = A.gzs = 1.0f;
                    A.o = box_offset(qx, qy, qz, sy, sz);
                    CornerVals c;
                    box_corners(bx + A.o, sy, sz, c);
                    float gq[3];
                    const float v = interpolate_grad(A, c, gq);
                    if constexpr (MODE == kAlpha) {
                        asum.add(k, v, gq);
                    } else {
                        const float zero[3] = {0.0f, 0.0f, 0.0f};
                        pose_add_group(k, v, gq, zero, s0, g0, h1);
                    }
                }
            }
            __syncthreads();
        } else if (hit) {
            // the box does not fit: gather this chunk's corners from global memory
            for (int k = k0; k < k0 + S; ++k) {
                const int64_t qx = sample_fixed(F, 0, k), qy = sample_fixed(F, 1, k);
                const int64_t qz = sample_fixed(F, 2, k);
                const int ix = fixed_floor(qx), iy = fixed_floor(qy), iz = fixed_floor(qz);
                SampleAddr A;
                A.fx = fixed_frac(qx);
                A.fy = fixed_frac(qy);
                A.fz = fixed_frac(qz);
                A.gxs = A.gzs = 1.0f;
                CornerVals c;
#pragma unroll
                for (int n = 0; n < 8; ++n)
                    c.v[n] = staged_value<T, TF>(rs, V, ix + (n & 1), iy + ((n >> 1) & 1),
                                                 iz + (n >> 2), tf, ch);
                float gq[3];
                const float v = interpolate_grad(A, c, gq);
                if constexpr (MODE == kAlpha) {
                    asum.add(k, v, gq);
                } else {
                    const float zero[3] = {0.0f, 0.0f, 0.0f};
                    pose_add_group(k, v, gq, zero, s0, g0, h1);
                }
            }
        }
        k0 += S;
        if (vol_cells * 2 <= kStageCap) S *= 2;
    }
    if (hit) {
        if constexpr (MODE == kAlpha)
            alpha_pose_chain(F, V, N, g, b.f, asum, contrib);
        else
            pose_chain_rule<MODE>(F, V, N, g, b.f, s0, g0, h1, contrib);
    }
    const double t = block_sum12(contrib, red);
    if (threadIdx.x < 12 && t != 0.0) unsafeAtomicAdd(acc + 12 * view + threadIdx.x, t);
}

// dL/dR_ij = -t_i P_j + Q_ij, dL/dt_i = -sum_a R_ia P_a, written as 3x4 rows.
__global__ __launch_bounds__(64) void drr_pose_finalize_kernel(const double* __restrict__ acc,
                                                                const float* __restrict__ poses,
                                                                int n_views,
                                                                float* __restrict__ grad_poses)
{
    const int id = (int)(blockIdx.x * blockDim.x + threadIdx.x);
    if (id >= n_views * 12) return;
    const int v = id / 12, e = id % 12, r = e / 4, c = e % 4;
    const double* P = acc + 12 * v;
    const double* Q = P + 3;
    const float* pose = poses + 12 * v;
    double val;
    if (c < 3) {
        val = -(double)pose[r * 4 + 3] * P[c] + Q[r * 3 + c];
    } else {
        val = -((double)pose[r * 4 + 0] * P[0] + (double)pose[r * 4 + 1] * P[1] +
                (double)pose[r * 4 + 2] * P[2]);
    }
    grad_poses[id] = (float)val;
}

__global__ __launch_bounds__(256) void drr_zero_f64_kernel(double* __restrict__ p, int n)
{
    const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
    if (i < n) p[i] = 0.0;
}

template <typename T, Layout L, int CLIP>
static void launch_pose(const LaunchArgs& a, const T* src, uint32_t src_bytes, const Batch& b,
                        const float* grad_out, double* acc, hipStream_t stream)
{
    const int tiles_x = (a.W + kTile - 1) / kTile, tiles_y = (a.H + kTile - 1) / kTile;
    const int tiles_per_view = tiles_x * tiles_y;
    const dim3 grid(tiles_per_view * a.n_views * a.C), block(kBlock);
    if (a.mode == kBeerLambert)
        hipLaunchKernelGGL((drr_pose_grad_kernel<T, L, kBeerLambert, CLIP>), grid, block, 0,
                           stream, src, src_bytes, a.V, a.K, a.poses, a.H, a.W, a.N, tiles_x,
                           tiles_per_view, b, grad_out, acc);
    else if (a.mode == kLineIntegral)
        hipLaunchKernelGGL((drr_pose_grad_kernel<T, L, kLineIntegral, CLIP>), grid, block, 0,
                           stream, src, src_bytes, a.V, a.K, a.poses, a.H, a.W, a.N, tiles_x,
                           tiles_per_view, b, grad_out, acc);
    else
        hipLaunchKernelGGL((drr_pose_grad_kernel<T, L, kAlpha, CLIP>), grid, block, 0, stream,
                           src, src_bytes, a.V, a.K, a.poses, a.H, a.W, a.N, tiles_x,
                           tiles_per_view, b, grad_out, acc);
}

// The march reads T elements in layout L from `src`: the read plan decides.
template <typename T>
static void pose_typed(const LaunchArgs& a, const RenderPlan& p, const T* src, const Batch& b,
                       const float* grad_out, double* acc, hipStream_t stream)
{
    if (a.clip == kClipNearFar) {
        // zero-padded cells or z-pairs (the near/far plan always makes one)
        if (p.cells)
            launch_pose<T, Layout::Cell, kClipNearFar>(a, src, a.V.cell_total_bytes, b, grad_out,
                                                       acc, stream);
        else
            launch_pose<T, Layout::ZPair, kClipNearFar>(a, src, a.V.total_bytes, b, grad_out,
                                                        acc, stream);
        return;
    }
    if (p.cells) {
        launch_pose<T, Layout::Cell, kClipBox>(a, src, a.V.cell_total_bytes, b, grad_out, acc,
                                               stream);
        return;
    }
    if (p.zpair) {
        launch_pose<T, Layout::ZPair, kClipBox>(a, src, a.V.total_bytes, b, grad_out, acc,
                                                stream);
        return;
    }
    const uint32_t bytes = (uint32_t)((size_t)a.V.n[0] * a.V.n[1] * a.V.n[2] * sizeof(T));
    if (a.V.n[0] >= 2)
        launch_pose<T, Layout::Pair, kClipBox>(a, src, bytes, b, grad_out, acc, stream);
    else
        launch_pose<T, Layout::Single, kClipBox>(a, src, bytes, b, grad_out, acc, stream);
}

template <typename T, int MODE>
static void launch_pose_staged_mode(const LaunchArgs& a, const T* vol, const Batch& b,
                                    const float* grad_out, double* acc, hipStream_t stream)
{
    const int tiles_x = (a.W + kTile - 1) / kTile, tiles_y = (a.H + kTile - 1) / kTile;
    const int tiles_per_view = tiles_x * tiles_y;
    const dim3 grid(tiles_per_view * a.n_views * a.C), block(kBlock);
    const uint32_t bytes = (uint32_t)((size_t)a.V.n[0] * a.V.n[1] * a.V.n[2] * sizeof(T));
    if (a.has_tf)
        hipLaunchKernelGGL((drr_pose_staged_kernel<T, MODE, true>), grid, block, 0, stream, vol,
                           bytes, a.V, a.K, a.poses, a.H, a.W, a.N, tiles_x, tiles_per_view, b,
                           a.tf, grad_out, acc);
    else
        hipLaunchKernelGGL((drr_pose_staged_kernel<T, MODE, false>), grid, block, 0, stream, vol,
                           bytes, a.V, a.K, a.poses, a.H, a.W, a.N, tiles_x, tiles_per_view, b,
                           a.tf, grad_out, acc);
}

template <typename T>
static void launch_pose_staged(const LaunchArgs& a, const T* vol, const Batch& b,
                               const float* grad_out, double* acc, hipStream_t stream)
{
    if (a.mode == kBeerLambert)
        launch_pose_staged_mode<T, kBeerLambert>(a, vol, b, grad_out, acc, stream);
    else if (a.mode == kLineIntegral)
        launch_pose_staged_mode<T, kLineIntegral>(a, vol, b, grad_out, acc, stream);
    else
        launch_pose_staged_mode<T, kAlpha>(a, vol, b, grad_out, acc, stream);
}

hipError_t launch_backward_pose(const LaunchArgs& a, const RenderPlan& plan, const void* vol,
                                int dtype, void* read_buf, double* acc, const float* grad_out,
                                float* grad_poses, hipStream_t stream, bool reuse_copy)
{
    if (a.n_views == 0) return hipSuccess;
    const int n_acc = 12 * a.n_views;
    hipLaunchKernelGGL(drr_zero_f64_kernel, dim3((n_acc + 255) / 256), dim3(256), 0, stream, acc,
                       n_acc);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if ((long long)a.H * a.W > 0) {
        if (plan.staged) {
            // boxes of the caller's volumes, staged in LDS tile by tile
            Batch b;
            b.src_stride = (uint64_t)plan.per_volume_bytes;
            b.grad_stride = 0;
            b.C = a.C;
            b.vpv = a.n_views / a.n_volumes;
            b.f = a.f;
            b.margin = a.margin;
            if (dtype == 0)
                launch_pose_staged<float>(a, static_cast<const float*>(vol), b, grad_out, acc,
                                          stream);
            else
                launch_pose_staged<uint16_t>(a, static_cast<const uint16_t*>(vol), b, grad_out,
                                             acc, stream);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
            hipLaunchKernelGGL(drr_pose_finalize_kernel, dim3((n_acc + 63) / 64), dim3(64), 0,
                               stream, acc, a.poses, a.n_views, grad_poses);
            return hipGetLastError();
        }
        if (!reuse_copy) {
            e = launch_read_copy(a, plan, vol, dtype, read_buf, stream);
            if (e != hipSuccess) return e;
        }
        Batch b;
        b.src_stride = (uint64_t)plan.per_volume_bytes;
        b.grad_stride = 0;
        b.C = a.C;
        b.vpv = a.n_views / a.n_volumes;
        b.f = a.f;
        b.margin = a.margin;
        const void* src = (plan.cells || plan.zpair || plan.mapped) ? read_buf : vol;
        if (plan.mapped || dtype == 0)
            pose_typed<float>(a, plan, static_cast<const float*>(src), b, grad_out, acc, stream);
        else
            pose_typed<uint16_t>(a, plan, static_cast<const uint16_t*>(src), b, grad_out, acc,
                                 stream);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(drr_pose_finalize_kernel, dim3((n_acc + 63) / 64), dim3(64), 0, stream, acc,
                       a.poses, a.n_views, grad_poses);
    return hipGetLastError();
}

}  // namespace drr
