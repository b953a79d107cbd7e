// drr_brick.hip -- the brick-owned volume backward (Beer-Lambert and line
// integral, box clip): a ray-record pass, then one workgroup per brick of the
// gradient that adds every sample touching its voxels in LDS and writes them
// once.  No global atomics, no zero fill, and the sums are exact integers in
// a fixed-point scale chosen per brick, so the result does not depend on the
// order of the adds.  The same for the cell-constant (Siddon) backward, at the
// end of the file.
//
// Method (source pages): flashdrr.rendering VolumeRaycaster class text --
// rendering is differentiable with respect to the volume; diffct 2.1.0
// Quickstart -- backproject() applies the matched adjoint A^T, and for
// 0.5 ||A x - y||^2 the gradient is A^T (A x - y).  Every sample of a ray adds
// y dz w_corner to each of its eight trilinear corners (clamped corners that
// coincide add together), with y = g f exp(-tau) (Beer-Lambert) or g f (line
// integral), f the density factor.
#include <hip/hip_runtime.h>

#include "drr_brick.hpp"
#include "drr_internal.hpp"
#include "drr_siddon.hpp"
#include "drr_window.hpp"

namespace drr {

// ------------------------------------------------------------ ray records

// The record of ray i: the forward's ray setup (same fp64 arithmetic, so the
// fixed-point sample positions are bit-identical) and the ray's coefficient.
// Returns its cell bound (0 for a ray that adds nothing).
template <int MODE>
__device__ inline float ray_record(const VolumeDesc& V, const Intrinsics& K,
                                   const float* __restrict__ poses, int H, int W, int N, int C,
                                   float f, long long i, const float* __restrict__ grad_out,
                                   const float* __restrict__ s_in, RayRecord* __restrict__ rec)
{
    const long long hw = (long long)H * W;
    const int pair = (int)(i / hw);
    const int rem = (int)(i - (long long)pair * hw);
    const int r = rem / W, c = rem - (rem / W) * W;
    const int view = pair / C;
    ViewGeom G;
    view_setup(poses + 12 * view, K, G);
    MarchRay R;
    RayRecord out;
    out.n = 0;
    out.coef = 0.0f;
    out.cell_bound = 0.0f;
    out.pad = 0;
    if (ray_setup(G, V, r, c, N, R)) {
        float y = grad_out[i] * f;
        if (MODE == kBeerLambert) y *= expf(-s_in[i]);
        const float coef = y * R.dz;
#pragma unroll
        for (int a = 0; a < 3; ++a) {
            out.q0[a] = R.q0[a];
            out.dq[a] = R.dq[a];
        }
        if (coef != 0.0f) {          // (NaN too: it must reach the gradient)
            out.n = N;
            out.coef = coef;
            out.cell_bound = fabsf(coef) * (float)samples_per_cell_bound(R.dq, N);
        }
    } else {
#pragma unroll
        for (int a = 0; a < 3; ++a) out.q0[a] = out.dq[a] = 0;
    }
    const int4* src = reinterpret_cast<const int4*>(&out);
    int4* dst = reinterpret_cast<int4*>(rec + i);
#pragma unroll
    for (int k = 0; k < 4; ++k) dst[k] = src[k];
    return out.cell_bound;
}

// One thread per ray of every (view, channel) pair.
//   block_max  one float per 256 consecutive rays: the largest cell bound
//              among them, +inf when one of their coefficients is not finite
template <int MODE>
__global__ __launch_bounds__(256) void drr_ray_record_kernel(
    VolumeDesc V, Intrinsics K, const float* __restrict__ poses, int H, int W, int N, int C,
    float f, long long n_rays, const float* __restrict__ grad_out, const float* __restrict__ s_in,
    RayRecord* __restrict__ rec, float* __restrict__ block_max)
{
    __shared__ float red[4];
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    float cb = 0.0f;
    if (i < n_rays) cb = ray_record<MODE>(V, K, poses, H, W, N, C, f, i, grad_out, s_in, rec);
    cb = isfinite(cb) ? cb : __builtin_inff();
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) cb = fmaxf(cb, __shfl_xor(cb, off, 64));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = cb;
    __syncthreads();
    if (threadIdx.x == 0)
        block_max[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// A view's fp32 projection K [R | t] (from fp64 products).
__device__ inline BrickView brick_view_of(const Intrinsics& K, const float* __restrict__ pose)
{
    BrickView out;
#pragma unroll
    for (int r = 0; r < 3; ++r) {
#pragma unroll
        for (int c = 0; c < 4; ++c)
            out.P[r * 4 + c] = (float)((double)K.k[r * 3 + 0] * (double)pose[0 * 4 + c] +
                                       (double)K.k[r * 3 + 1] * (double)pose[1 * 4 + c] +
                                       (double)K.k[r * 3 + 2] * (double)pose[2 * 4 + c]);
    }
    return out;
}

// One thread per view: its projection.
__global__ __launch_bounds__(64) void drr_brick_views_kernel(Intrinsics K,
                                                              const float* __restrict__ poses,
                                                              int n_views,
                                                              BrickView* __restrict__ views)
{
    const int v = blockIdx.x * blockDim.x + threadIdx.x;
    if (v >= n_views) return;
    views[v] = brick_view_of(K, poses + 12 * v);
}

// ------------------------------------------------------------ brick scatter

constexpr int kBrickThreads = 256;
constexpr int kViewChunk = 64;      // views whose pixel rectangles and rays sit in LDS at once

// Workgroup-wide exclusive prefix sum of one int per thread; returns the total.
__device__ inline int block_exclusive_scan(int v, int* red, int& excl)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int incl = wave_inclusive_scan(v);
    if (lane == 63) red[wave] = incl;
    __syncthreads();
    int base = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kBrickThreads / 64; ++w) {
        const int s = red[w];
        base += w < wave ? s : 0;
        total += s;
    }
    excl = base + incl - v;
    __syncthreads();
    return total;
}

// The same for two ints at once (a and b, exclusive sums in ea and eb);
// returns both totals.  It ends without a barrier: `red` must not be written
// again before the next one (the brick kernel's rounds have two in between).
__device__ inline int2 block_exclusive_scan2(int a, int b, int* red, int& ea, int& eb)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int ia = wave_inclusive_scan(a), ib = wave_inclusive_scan(b);
    if (lane == 63) {
        red[2 * wave] = ia;
        red[2 * wave + 1] = ib;
    }
    __syncthreads();
    int base_a = 0, base_b = 0, tot_a = 0, tot_b = 0;
#pragma unroll
    for (int w = 0; w < kBrickThreads / 64; ++w) {
        const int sa = red[2 * w], sb = red[2 * w + 1];
        base_a += w < wave ? sa : 0;
        base_b += w < wave ? sb : 0;
        tot_a += sa;
        tot_b += sb;
    }
    ea = base_a + ia - a;
    eb = base_b + ib - b;
    return make_int2(tot_a, tot_b);
}

// The candidate rays of a brick, kViewChunk views at a time: for each view of
// its channel-volume the detector rectangle that can reach its cells
// (brick_pixel_rect), walked row by row in batches of kBrickThreads rows, each
// row cut to the span of the region's projection (brick_row_span).  Row p of
// a chunk is row p - start[v] of view slot v's rectangle (start[v] <= p <
// start[v + 1]); candidate j of a batch is column j - rowpre[i] of the
// batch's row i (rowpre[i] <= j < rowpre[i + 1]).
struct BrickCandidates {
    int* start;          // kViewChunk + 1: exclusive prefix sums of the rectangles' heights
    int* rect;           // kViewChunk x 3: r0, c0, width
    int* rowpre;         // kBrickThreads + 1: exclusive prefix sums of the batch's row spans
    int* rowinfo;        // kBrickThreads x 2: view slot << 16 | row, first column

    // view slot of chunk row p (0 <= p < start[n_in_chunk])
    __device__ int view_of_row(int p, int n_in_chunk) const
    {
        int lo = 0, hi = n_in_chunk - 1;               // last v with start[v] <= p
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (start[mid] <= p) lo = mid; else hi = mid - 1;
        }
        return lo;
    }

    // view slot and pixel of candidate j of the current batch
    __device__ void pixel(int j, int& v, int& r, int& c) const
    {
        int lo = 0, hi = kBrickThreads - 1;            // last i with rowpre[i] <= j
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (rowpre[mid] <= j) lo = mid; else hi = mid - 1;
        }
        const int info = rowinfo[2 * lo];
        v = info >> 16;
        r = info & 0xffff;
        c = rowinfo[2 * lo + 1] + (j - rowpre[lo]);
    }
};

// One record, loaded as four 16-byte reads.
__device__ inline RayRecord load_record(const RayRecord* __restrict__ rec, long long i)
{
    RayRecord r;
    const int4* src = reinterpret_cast<const int4*>(rec + i);
    int4* dst = reinterpret_cast<int4*>(&r);
#pragma unroll
    for (int k = 0; k < 4; ++k) dst[k] = src[k];
    return r;
}

// Sets up the candidate rectangles of views [first, first + count) for the
// brick region `g` (count <= kViewChunk) in `cand`; returns their total
// number of rows.
__device__ inline int brick_chunk(const BrickView* __restrict__ views, int H, int W,
                                  const BrickRegion& g, int first, int count,
                                  BrickCandidates& cand, int* red)
{
    int rows = 0;
    const int t = threadIdx.x;
    if (t < count) {
        const PixelRect R = brick_pixel_rect(views[first + t].P, g, H, W);
        const int w = R.c1 - R.c0 + 1, h = R.r1 - R.r0 + 1;
        rows = (w > 0 && h > 0) ? h : 0;
        cand.rect[3 * t] = R.r0;
        cand.rect[3 * t + 1] = R.c0;
        cand.rect[3 * t + 2] = w > 0 ? w : 1;
    }
    int excl;
    const int total = block_exclusive_scan(rows, red, excl);
    if (t < count) cand.start[t] = excl;
    if (t == 0) cand.start[count] = total;
    __syncthreads();
    return total;
}

// Rows [p0, p0 + kBrickThreads) of a chunk's rectangles, one per thread: its
// span (the projection's when `spans`, else the whole rectangle row) into
// `cand`; returns the batch's candidate total.
__device__ inline int brick_row_batch(const BrickView* __restrict__ views, const BrickRegion& g,
                                      int first, int count, int n_rows, int p0, bool spans,
                                      BrickCandidates& cand, int* red)
{
    const int t = threadIdx.x, p = p0 + t;
    int width = 0;
    if (p < n_rows) {
        const int v = cand.view_of_row(p, count);
        const int r = cand.rect[3 * v] + (p - cand.start[v]);
        int c0 = cand.rect[3 * v + 1], c1 = c0 + cand.rect[3 * v + 2] - 1;
        if (spans) brick_row_span(brick_hull(views[first + v].P, g), r, c0, c1, c0, c1);
        width = c1 >= c0 ? c1 - c0 + 1 : 0;
        cand.rowinfo[2 * t] = (v << 16) | r;
        cand.rowinfo[2 * t + 1] = c0;
    }
    int excl;
    const int total = block_exclusive_scan(width, red, excl);
    cand.rowpre[t] = excl;
    if (t == 0) cand.rowpre[kBrickThreads] = total;
    __syncthreads();
    return total;
}

// Fixed-point value of a register sum, rounded to nearest (halves up) in one
// conversion: the sums are at most 2^30 in magnitude.
__device__ inline int to_fixed_rn(float v)
{
    int r;
    asm("v_cvt_rpi_i32_f32 %0, %1" : "=v"(r) : "v"(v));
    return r;
}

// Eight fixed-point adds of a cell's register sums at LDS entry `e0` of the
// brick copy (pitch B + 2): corner n at e0 + brick_corner_offset(B, n).
template <int B>
__device__ inline void brick_add8(unsigned long long* acc, int e0, const float s[8])
{
#pragma unroll
    for (int n = 0; n < 8; ++n) {
        const int e = e0 + brick_corner_offset(B, n);
        const long long v = (long long)to_fixed_rn(s[n]);
        atomicAdd(acc + e, (unsigned long long)v);
    }
}

// Eight trilinear weights of fractions (fx, fy, fz) times c, corner order x
// fastest: w[n] = c w_x(n & 1) w_y((n >> 1) & 1) w_z(n >> 2).
__device__ inline void weights8(float fx, float fy, float fz, float c, float w[8])
{
    const float wz1 = c * fz, wz0 = c - wz1;
    const float w11 = wz1 * fy, w10 = wz1 - w11;
    const float w01 = wz0 * fy, w00 = wz0 - w01;
    w[1] = w00 * fx; w[0] = w00 - w[1];
    w[3] = w01 * fx; w[2] = w01 - w[3];
    w[5] = w10 * fx; w[4] = w10 - w[5];
    w[7] = w11 * fx; w[6] = w11 - w[7];
}

// The work queue of one round: the candidate rays with samples in the brick,
// compacted: the position of each one's first in-brick sample relative to the
// copy's origin (voxel lo - 1 at 0, fixed point), its step, its scaled
// coefficient and the exclusive prefix sum of the sample counts in queue
// order; and for every thread the queue entry that holds the first sample of
// its run.
template <int Q>
struct BrickQueue {
    static_assert(Q <= 256, "queue entries are indexed by bytes");
    int64_t q[3][Q];
    int64_t d[3][Q];
    float c[Q];
    int pre[Q + 1];
    unsigned char first[Q];
};

// The brick kernel.  Grid: (bricks of one channel-volume, channel-volumes).
// With B the brick side, the LDS copy holds (B + 2)^3 int64 entries.
//
// The fixed-point scale comes from the record pass's block maxima over the
// rows of every view's candidate rectangle.  Candidate rays (brick_pixel_rect
// over the views) are then taken kBrickThreads at a time, one per thread: its
// exact range of samples in the brick region (brick_exact_range) goes to the
// LDS queue, compacted to the rays that have some.  The queue's samples,
// counted in queue order, are split into kBrickThreads equal runs, one per
// thread (each queue entry marks the threads whose run starts in it): a
// thread steps through its run by fixed-point adds and moves to the next
// queued ray where one ends, so every lane of a wave has the same number of
// samples whatever the lengths of the rays.
// MERGE (views dense against the voxels, several samples of a ray per
// cell) sums consecutive samples of one cell in registers before adding them
// to the copy.
//
// Four workgroups per CU (the LDS allows four): the register budget is held
// to 128, which spills 14 registers of the cold per-row and per-chunk code to
// scratch (60 bytes per lane; the sample loops stay in registers).  Measured
// on MI355X, 16 views of 200^2 x 256 over 256^3: 1.51 ms at three
// workgroups per CU (151 registers), 1.36 ms at four.
template <int B, int Q, bool MERGE>
__global__ __launch_bounds__(kBrickThreads, 4) void drr_brick_scatter_kernel(
    VolumeDesc V, const BrickView* __restrict__ views, int H, int W, Batch bt,
    const RayRecord* __restrict__ rec, const float* __restrict__ block_max,
    float* __restrict__ grad, int nbx, int nby)
{
    static_assert(Q == kBrickThreads, "one queued ray per thread and round");
    constexpr int P = brick_pitch(B);
    constexpr int NE = P * P * P;
    __shared__ unsigned long long acc[NE];
    __shared__ BrickQueue<Q> qu;
    __shared__ int start[kViewChunk + 1];
    __shared__ int rect[3 * kViewChunk];
    __shared__ int rowpre[kBrickThreads + 1];
    __shared__ int rowinfo[2 * kBrickThreads];
    __shared__ int red[2 * (kBrickThreads / 64)];
    __shared__ float fred[kBrickThreads / 64];

    const int brick = xcd_contiguous_tile((int)blockIdx.x, (int)gridDim.x);
    const int bx = brick % nbx, by = (brick / nbx) % nby, bz = brick / (nbx * nby);
    const BrickBox b = brick_box(V.n, B, bx, by, bz);
    const BrickRegion reg = brick_region(V.n, V.s, V.q_off, b);
    const int cv = (int)blockIdx.y;                     // channel-volume
    const int vol = cv / bt.C, ch = cv - vol * bt.C;
    const int first_view = vol * bt.vpv;
    grad += (size_t)cv * bt.grad_stride;
    BrickCandidates cand{start, rect, rowpre, rowinfo};
    const int t = threadIdx.x;

    for (int i = t; i < NE; i += kBrickThreads) acc[i] = 0ull;

    // pass 1: the fixed-point scale from the largest cell bound among the
    // record blocks that hold the candidates' rows (a cell's register sum never
    // exceeds its ray's |c| m); +inf marks a block with a non-finite
    // coefficient
    float cmax = 0.0f;
    for (int v0 = 0; v0 < bt.vpv; v0 += kViewChunk) {
        const int count = min(kViewChunk, bt.vpv - v0);
        const int n_rows = brick_chunk(views, H, W, reg, first_view + v0, count, cand, red);
        // one rectangle row per thread, over all views of the chunk
        for (int p = t; p < n_rows; p += kBrickThreads) {
            const int v = cand.view_of_row(p, count);
            const int w = rect[3 * v + 2];
            const long long pair = (long long)(first_view + v0 + v) * bt.C + ch;
            const long long lin =
                (pair * H + rect[3 * v] + (p - start[v])) * W + rect[3 * v + 1];
            const long long b0 = lin >> 8, b1 = (lin + w - 1) >> 8;
            for (long long k = b0; k <= b1; ++k) cmax = fmaxf(cmax, block_max[k]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) cmax = fmaxf(cmax, __shfl_xor(cmax, off, 64));
    if ((t & 63) == 0) fred[t >> 6] = cmax;
    __syncthreads();
    cmax = fred[0];
#pragma unroll
    for (int w = 1; w < kBrickThreads / 64; ++w) cmax = fmaxf(cmax, fred[w]);
    // a non-finite coefficient among the candidates: their rays go through
    // float atomics after the brick is written, the others through the copy
    // with the largest finite cell bound as the scale
    const bool any_poison = !isfinite(cmax);
    if (any_poison) {
        cmax = 0.0f;
        for (int v0 = 0; v0 < bt.vpv; v0 += kViewChunk) {
            const int count = min(kViewChunk, bt.vpv - v0);
            const int n_rows = brick_chunk(views, H, W, reg, first_view + v0, count, cand, red);
            for (int p0 = 0; p0 < n_rows; p0 += kBrickThreads) {
                const int total = brick_row_batch(views, reg, first_view + v0, count, n_rows, p0,
                                                  true, cand, red);
                for (int j = t; j < total; j += kBrickThreads) {
                    int v, r, c;
                    cand.pixel(j, v, r, c);
                    const long long pair = (long long)(first_view + v0 + v) * bt.C + ch;
                    const long long ri = (pair * H + r) * W + c;
                    const float cb = rec[ri].cell_bound;
                    if (rec[ri].n != 0 && isfinite(cb)) cmax = fmaxf(cmax, cb);
                }
                __syncthreads();
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) cmax = fmaxf(cmax, __shfl_xor(cmax, off, 64));
        if ((t & 63) == 0) fred[t >> 6] = cmax;
        __syncthreads();
        cmax = fred[0];
#pragma unroll
        for (int w = 1; w < kBrickThreads / 64; ++w) cmax = fmaxf(cmax, fred[w]);
    }

    float scale = 0.0f, inv_scale = 0.0f;
    if (cmax > 0.0f) {
        // |sum| <= cmax 2^e <= 2^30 for every cell's register sum
        const int e = clampi((int)floorf(log2f(1073741824.0f / cmax)), -126, 126);
        scale = ldexpf(1.0f, e);
        inv_scale = ldexpf(1.0f, -e);
    }

    // pass 2: every finite ray's samples in the brick's cells into the copy
    if (cmax > 0.0f) {
        for (int v0 = 0; v0 < bt.vpv; v0 += kViewChunk) {
          const int count = min(kViewChunk, bt.vpv - v0);
          const int n_rows = brick_chunk(views, H, W, reg, first_view + v0, count, cand, red);
          for (int p0 = 0; p0 < n_rows; p0 += kBrickThreads) {
            const int total = brick_row_batch(views, reg, first_view + v0, count, n_rows, p0,
                                              true, cand, red);
            // this thread's candidate of a round: its record, loaded one round
            // ahead so the load's latency hides behind the previous round's
            // samples
            auto fetch = [&](int j, RayRecord& r) {
                r.n = 0;
                if (j >= total) return;
                int v, cr, cc;
                cand.pixel(j, v, cr, cc);
                const long long pair = (long long)(first_view + v0 + v) * bt.C + ch;
                r = load_record(rec, (pair * H + cr) * W + cc);
            };
            RayRecord next;
            fetch(t, next);
            for (int jb = 0; jb < total; jb += kBrickThreads) {
                // fill: this thread's candidate and its samples in the brick
                const RayRecord r = next;
                fetch(jb + kBrickThreads + t, next);
                int cnt = 0;
                int64_t q[3], dq[3];
                float cs = 0.0f;
                if (r.n != 0 && isfinite(r.cell_bound)) {
                    int k_lo, k_hi;
                    brick_exact_range(r, b, k_lo, k_hi, q);
                    cnt = k_hi - k_lo;
#pragma unroll
                    for (int a = 0; a < 3; ++a) dq[a] = r.dq[a];
                    cs = r.coef * scale;
                }
                int pos, first_sample;
                const int2 tot =
                    block_exclusive_scan2(cnt > 0 ? 1 : 0, cnt, red, pos, first_sample);
                const int m = tot.x, n_samples = tot.y;
                if (cnt > 0) {
#pragma unroll
                    for (int a = 0; a < 3; ++a) {
                        qu.q[a][pos] = q[a];
                        qu.d[a][pos] = dq[a];
                    }
                    qu.c[pos] = cs;
                    qu.pre[pos] = first_sample;
                    // the threads whose run [n u / Q, n (u + 1) / Q) starts in
                    // this entry: n u / Q in [first, first + cnt)
                    const uint64_t nn = (uint64_t)n_samples;
                    const int u0 = (int)(((uint64_t)first_sample * Q + nn - 1) / nn);
                    const int u1 = (int)(((uint64_t)(first_sample + cnt) * Q + nn - 1) / nn);
                    for (int u = u0; u < u1; ++u) qu.first[u] = (unsigned char)pos;
                }
                if (t == 0) qu.pre[m] = n_samples;
                __syncthreads();
                // this thread's run [s0, s1) of the queue's samples
                const uint32_t s0 = (uint32_t)(((uint64_t)n_samples * t) / kBrickThreads);
                const uint32_t s1 = (uint32_t)(((uint64_t)n_samples * (t + 1)) / kBrickThreads);
                if (s1 > s0) {
                    int e = qu.first[t];
                    const int64_t off = (int64_t)(s0 - (uint32_t)qu.pre[e]);
                    int64_t qx = qu.q[0][e] + off * qu.d[0][e];
                    int64_t qy = qu.q[1][e] + off * qu.d[1][e];
                    int64_t qz = qu.q[2][e] + off * qu.d[2][e];
                    int64_t dx = qu.d[0][e], dy = qu.d[1][e], dz = qu.d[2][e];
                    float c = qu.c[e];
                    uint32_t left = (uint32_t)qu.pre[e + 1] - s0;   // samples left in entry e
                    float sum[8];
#pragma unroll
                    for (int n = 0; n < 8; ++n) sum[n] = 0.0f;
                    int pcell = -1;
                    for (uint32_t s = s0; s < s1; ++s) {
                        const int cell = brick_cell_entry(B, fixed_floor(qx), fixed_floor(qy),
                                                          fixed_floor(qz));
                        const float fx = fixed_frac(qx), fy = fixed_frac(qy);
                        const float fz = fixed_frac(qz);
                        // the last sample of entry e: read the next entry now,
                        // ahead of this sample's adds, so that taking it over
                        // below waits for these reads only (LDS operations
                        // complete in order) and the adds stay in flight.  The
                        // reads are clamped in range; unused when the run ends.
                        const bool last = left == 1;
                        int64_t nq[3], nd[3];
                        float nc;
                        int np0, np1;          // (nothing computed from the reads here)
                        if (last) {
                            const int k = min(e + 1, Q - 1);
#pragma unroll
                            for (int a = 0; a < 3; ++a) {
                                nq[a] = qu.q[a][k];
                                nd[a] = qu.d[a][k];
                            }
                            nc = qu.c[k];
                            np0 = qu.pre[min(e + 1, Q)];
                            np1 = qu.pre[min(e + 2, Q)];
                        }
                        __builtin_amdgcn_sched_barrier(0);
                        if constexpr (MERGE) {
                            if (cell != pcell) {
                                if (pcell >= 0) brick_add8<B>(acc, pcell, sum);
#pragma unroll
                                for (int n = 0; n < 8; ++n) sum[n] = 0.0f;
                                pcell = cell;
                            }
                            add_weights8(fx, fy, fz, c, sum);
                        } else {
                            float w[8];
                            weights8(fx, fy, fz, c, w);
                            brick_add8<B>(acc, cell, w);
                        }
                        __builtin_amdgcn_sched_barrier(0);
                        qx += dx;
                        qy += dy;
                        qz += dz;
                        --left;
                        if (last) {
                            // entry e ends: continue with the next one
                            ++e;
                            qx = nq[0]; qy = nq[1]; qz = nq[2];
                            dx = nd[0]; dy = nd[1]; dz = nd[2];
                            c = nc;
                            left = (uint32_t)(np1 - np0);
                        }
                    }
                    if (MERGE && pcell >= 0) brick_add8<B>(acc, pcell, sum);
                }
                __syncthreads();
            }
          }
        }
    }
    __syncthreads();

    // clamp to edge: apron entries at voxel -1 or n fold into the edge voxel,
    // one axis after the other (entries at -1 / n of several axes fold through
    // each in turn)
    const int e3[3] = {b.e[0], b.e[1], b.e[2]};
#pragma unroll
    for (int a = 0; a < 3; ++a) {
        const bool low = b.lo[a] == 0, high = b.lo[a] + b.e[a] == V.n[a];
        if (low || high) {
            // the other two axes span their full copy (P entries)
            for (int i = threadIdx.x; i < P * P; i += kBrickThreads) {
                int step;
                const int base = brick_line_base(B, a, i, step);
                if (low) acc[base + step] += acc[base];
                if (high) acc[base + e3[a] * step] += acc[base + (e3[a] + 1) * step];
            }
        }
        __syncthreads();
    }

    // the brick's voxels, written once
    const uint32_t sy = (uint32_t)V.n[0], sz = (uint32_t)V.n[0] * (uint32_t)V.n[1];
    const double inv = (double)inv_scale;
    for (int i = threadIdx.x; i < B * B * B; i += kBrickThreads) {
        const int x = i % B, y = (i / B) % B, z = i / (B * B);
        if (x >= b.e[0] || y >= b.e[1] || z >= b.e[2]) continue;
        const long long v = (long long)acc[brick_entry(B, x + 1, y + 1, z + 1)];
        grad[(uint32_t)(b.lo[2] + z) * sz + (uint32_t)(b.lo[1] + y) * sy +
             (uint32_t)(b.lo[0] + x)] = (float)((double)v * inv);
    }
    if (!any_poison) return;

    // rays whose coefficient is not finite: float atomics straight to the
    // brick's own voxels (NaN and Inf propagate as in a float sum; a zero
    // weight times Inf is NaN), after the stores above are visible
    __threadfence();
    __syncthreads();
    for (int v0 = 0; v0 < bt.vpv; v0 += kViewChunk) {
      const int count = min(kViewChunk, bt.vpv - v0);
      const int n_rows = brick_chunk(views, H, W, reg, first_view + v0, count, cand, red);
      for (int p0 = 0; p0 < n_rows; p0 += kBrickThreads) {
        const int total = brick_row_batch(views, reg, first_view + v0, count, n_rows, p0, true,
                                          cand, red);
        for (int j = threadIdx.x; j < total; j += kBrickThreads) {
            int cv_slot, cr, cc;
            cand.pixel(j, cv_slot, cr, cc);
            const long long pair = (long long)(first_view + v0 + cv_slot) * bt.C + ch;
            const RayRecord r = load_record(rec, (pair * H + cr) * W + cc);
            if (r.n == 0 || isfinite(r.cell_bound)) continue;
            int k_lo, k_hi;
            brick_sample_range(r, b, k_lo, k_hi);
            for (int k = k_lo; k < k_hi; ++k) {
                const int64_t q[3] = {r.q0[0] + (int64_t)k * r.dq[0],
                                      r.q0[1] + (int64_t)k * r.dq[1],
                                      r.q0[2] + (int64_t)k * r.dq[2]};
                int cl[3];
                bool inside = true;
#pragma unroll
                for (int a = 0; a < 3; ++a) {
                    cl[a] = fixed_floor(q[a]);
                    inside = inside && cl[a] >= b.lo[a] - 1 && cl[a] <= b.lo[a] + b.e[a] - 1;
                }
                if (!inside) continue;
                // products of the per-axis weights (as the definition reads),
                // so an infinite coefficient gives infinities, and NaN only
                // where a weight is 0
                const float fx = fixed_frac(q[0]), fy = fixed_frac(q[1]), fz = fixed_frac(q[2]);
                const float wz[2] = {r.coef * (1.0f - fz), r.coef * fz};
                const float wy[2] = {1.0f - fy, fy}, wx[2] = {1.0f - fx, fx};
                float w[8];
#pragma unroll
                for (int n = 0; n < 8; ++n) w[n] = wz[n >> 2] * wy[(n >> 1) & 1] * wx[n & 1];
#pragma unroll
                for (int n = 0; n < 8; ++n) {
                    const int g[3] = {clampi(cl[0] + (n & 1), 0, V.n[0] - 1),
                                      clampi(cl[1] + ((n >> 1) & 1), 0, V.n[1] - 1),
                                      clampi(cl[2] + (n >> 2), 0, V.n[2] - 1)};
                    bool own = true;
#pragma unroll
                    for (int a = 0; a < 3; ++a)
                        own = own && g[a] >= b.lo[a] && g[a] < b.lo[a] + b.e[a];
                    if (own)
                        unsafeAtomicAdd(grad + (uint32_t)g[2] * sz + (uint32_t)g[1] * sy +
                                            (uint32_t)g[0],
                                        w[n]);
                }
            }
        }
        __syncthreads();
      }
    }
}

// ------------------------------------------------------------ launcher

hipError_t launch_brick_backward(const LaunchArgs& a, const float* grad_out, const float* s_in,
                                 float* grad, void* workspace, hipStream_t stream)
{
    const long long n_rays = (long long)a.n_views * a.C * a.H * a.W;
    RayRecord* rec = static_cast<RayRecord*>(workspace);
    float* block_max = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                                ray_record_bytes(a.n_views, a.C, a.H, a.W));
    BrickView* views = reinterpret_cast<BrickView*>(
        reinterpret_cast<char*>(block_max) + ray_block_max_bytes(a.n_views, a.C, a.H, a.W));
    if (a.n_views > 0) {
        hipLaunchKernelGGL(drr_brick_views_kernel, dim3((a.n_views + 63) / 64), dim3(64), 0,
                           stream, a.K, a.poses, a.n_views, views);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int rb = (int)((n_rays + 255) / 256);
    if (n_rays > 0) {
        if (a.mode == kBeerLambert)
            hipLaunchKernelGGL((drr_ray_record_kernel<kBeerLambert>), dim3(rb), dim3(256), 0,
                               stream, a.V, a.K, a.poses, a.H, a.W, a.N, a.C, a.f, n_rays,
                               grad_out, s_in, rec, block_max);
        else
            hipLaunchKernelGGL((drr_ray_record_kernel<kLineIntegral>), dim3(rb), dim3(256), 0,
                               stream, a.V, a.K, a.poses, a.H, a.W, a.N, a.C, a.f, n_rays,
                               grad_out, s_in, rec, block_max);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    constexpr int B = kBrickSide;
    const int nbx = (a.V.n[0] + B - 1) / B, nby = (a.V.n[1] + B - 1) / B;
    const int nbz = (a.V.n[2] + B - 1) / B;
    // samples one view puts per cell: from about two, a ray's consecutive
    // samples often share a cell and are worth summing in registers first
    const double cells = (double)(a.V.n[0] + 1) * (a.V.n[1] + 1) * (a.V.n[2] + 1);
    const bool merge = (double)a.H * a.W * a.N / cells >= kBrickMergeMinViewReuse;
    Batch bt;
    bt.src_stride = 0;
    bt.grad_stride = (uint32_t)((size_t)a.V.n[0] * a.V.n[1] * a.V.n[2]);
    bt.C = a.C;
    bt.vpv = a.n_views / a.n_volumes;
    bt.f = a.f;
    bt.margin = a.margin;
    const dim3 grid((unsigned)(nbx * nby * nbz), (unsigned)(a.n_volumes * a.C));
    if (merge)
        hipLaunchKernelGGL((drr_brick_scatter_kernel<B, kBrickThreads, true>), grid,
                           dim3(kBrickThreads), 0, stream, a.V, views, a.H, a.W, bt, rec,
                           block_max, grad, nbx, nby);
    else
        hipLaunchKernelGGL((drr_brick_scatter_kernel<B, kBrickThreads, false>), grid,
                           dim3(kBrickThreads), 0, stream, a.V, views, a.H, a.W, bt, rec,
                           block_max, grad, nbx, nby);
    return hipGetLastError();
}

// ------------------------------------------------------- Siddon bricks
//
// Method (source pages): diffct 2.1.0, "Why diffct" feature list -- project()
// and backproject() are an exact adjoint pair for the cell-constant Siddon
// model, so every voxel receives sum over rays of y l_v, l_v the length of the
// ray inside it, y = g exp(-s) (Beer-Lambert) or g (line integral).
//
// The brick-owned backward of the cell-constant (Siddon) pair, for views sparse
// against the voxels: one workgroup per brick of B^3 voxels finds the rays that
// cross it (the candidate search of the trilinear bricks, over the brick's own
// voxel box), walks each one's pieces inside the brick and adds y l_v to an LDS
// copy of the brick in 64-bit fixed point, then writes every voxel once.  A
// piece lies in one voxel, so the copy needs no apron, and nothing is read
// from a workspace: the views' projections and cameras are made per chunk of
// views in LDS, and each candidate's ray is set up again from its pixel (the
// forward's fp64 arithmetic).  The walk inside a brick: drr_siddon.hpp.

// Brick side and views per chunk of the Siddon bricks: 16^3 int64 sums (32 KB)
// and 16 views' projections and cameras keep a workgroup's LDS under 40 KB, so
// four fit on a CU.  Measured on MI355X (16 views of 200^2 over 256^3): 12^3
// bricks with 64-view chunks 1.12 ms, 16^3 with 64-view chunks (three per CU)
// 0.99 ms, 16^3 with 16-view chunks 0.92 ms; the tile windows 2.69 ms.
constexpr int kSiddonBrickSide = 16;
constexpr int kSiddonViewChunk = 16;

// Views [v0, v0 + count) into LDS, one thread per view: the fp32 projection
// for the candidate search and the fp64 camera for the rays.
__device__ inline void siddon_view_chunk(const Intrinsics& K, const float* __restrict__ poses,
                                         int v0, int count, BrickView* pv, ViewGeom* geo)
{
    const int t = threadIdx.x;
    if (t < count) {
        const float* pose = poses + 12 * (v0 + t);
        pv[t] = brick_view_of(K, pose);
        ViewGeom G;
        view_setup(pose, K, G);
        geo[t] = G;
    }
    __syncthreads();
}

// y of ray i: g exp(-s) (Beer-Lambert) or g (line integral).
template <int MODE>
__device__ inline float siddon_coef(const float* __restrict__ grad_out,
                                    const float* __restrict__ s_in, long long i)
{
    float y = grad_out[i];
    if (MODE == kBeerLambert) y *= expf(-s_in[i]);
    return y;
}

// Grid: the bricks of the volume.  The fixed-point scale: a piece is at most
// the voxel diagonal D long, so with ymax the largest finite |y| among the rays
// that cross the brick a scale 2^e with 2^e ymax D <= 2^30 keeps every piece's
// value in int32, and the 64-bit sums cannot overflow.  In Beer-Lambert mode
// the candidate pixels (a superset of the brick's rays) whose ray misses the
// volume have y = g (s = 0), and would set the unit far above the pieces of a
// brick deep in an attenuating volume (seen at optical depths of 17 and more,
// where such a brick's gradient lost several percent): a candidate with s = 0
// counts only if its ray crosses the brick, tested when its |y| is above the
// thread's running maximum.  Every other candidate counts as it is (a ray with
// s != 0 met the volume; in line-integral mode y = g whatever the ray).
// Measured on 16 views of 200^2 over 256^3: 0.918 ms with the bound over all
// candidates, 0.949 ms with this one, 1.000 ms testing every candidate that
// way.  Rays whose y is not finite add by float atomics after the brick is
// written (their voxels' gradient is not finite anyway).
// Four workgroups per CU hold the register budget to 128, which spills some
// registers of the per-candidate setup to scratch; the walk loop stays in
// registers (measured 0.92 ms against 0.99 ms at three workgroups per CU
// without spills).
template <int MODE>
__global__ __launch_bounds__(kBrickThreads, 4) void drr_siddon_brick_kernel(
    VolumeDesc V, Intrinsics K, const float* __restrict__ poses, int n_views, int H, int W,
    const float* __restrict__ grad_out, const float* __restrict__ s_in,
    float* __restrict__ grad, int nbx, int nby)
{
    constexpr int B = kSiddonBrickSide;
    __shared__ unsigned long long acc[B * B * B];
    __shared__ BrickView pv[kSiddonViewChunk];
    __shared__ ViewGeom geo[kSiddonViewChunk];
    __shared__ int start[kSiddonViewChunk + 1];
    __shared__ int rect[3 * kSiddonViewChunk];
    __shared__ int rowpre[kBrickThreads + 1];
    __shared__ int rowinfo[2 * kBrickThreads];
    __shared__ int red[2 * (kBrickThreads / 64)];
    __shared__ float fred[kBrickThreads / 64];
    __shared__ int late;

    const int brick = xcd_contiguous_tile((int)blockIdx.x, (int)gridDim.x);
    const int bx = brick % nbx, by = (brick / nbx) % nby, bz = brick / (nbx * nby);
    const BrickBox b = brick_box(V.n, B, bx, by, bz);
    const BrickRegion reg = siddon_brick_region(V, b);
    BrickCandidates cand{start, rect, rowpre, rowinfo};
    const int t = threadIdx.x;
    for (int i = t; i < B * B * B; i += kBrickThreads) acc[i] = 0ull;
    if (t == 0) late = 0;

    // the candidates of every chunk of views, kBrickThreads at a time: `each`
    // gets (view, row, column, ray index) of one candidate per thread
    auto for_candidates = [&](auto each) {
        for (int v0 = 0; v0 < n_views; v0 += kSiddonViewChunk) {
            const int count = min(kSiddonViewChunk, n_views - v0);
            siddon_view_chunk(K, poses, v0, count, pv, geo);
            const int n_rows = brick_chunk(pv, H, W, reg, 0, count, cand, red);
            for (int p0 = 0; p0 < n_rows; p0 += kBrickThreads) {
                const int total = brick_row_batch(pv, reg, 0, count, n_rows, p0, true, cand, red);
                for (int j = t; j < total; j += kBrickThreads) {
                    int v, r, c;
                    cand.pixel(j, v, r, c);
                    each(v, r, c, ((long long)(v0 + v) * H + r) * W + c);
                }
                __syncthreads();
            }
        }
    };

    // pass 1: the largest finite |y| among the rays that cross the brick
    float ymax = 0.0f;
    int poison = 0, any = 0;
    for_candidates([&](int v, int r, int c, long long i) {
        const float ay = fabsf(siddon_coef<MODE>(grad_out, s_in, i));
        if (!isfinite(ay)) {
            poison = 1;
            return;
        }
        any |= ay > 0.0f;
        if (!(ay > ymax)) return;
        // a ray with s != 0 met the volume (a miss integrates to exactly 0):
        // taken as it is; a Beer-Lambert ray with s = 0, most often a miss
        // with y = g, only if it crosses the brick
        if (MODE != kBeerLambert || s_in[i] != 0.0f) {
            ymax = ay;
            return;
        }
        SiddonRay S;
        double t_in, t_out;
        if (siddon_clip(geo[v], V, r, c, S) && siddon_brick_range(S, V, b, t_in, t_out))
            ymax = ay;
    });
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ymax = fmaxf(ymax, __shfl_xor(ymax, off, 64));
    if ((t & 63) == 0) fred[t >> 6] = ymax;
    poison = __builtin_amdgcn_readfirstlane(__syncthreads_or(poison));
    any = __builtin_amdgcn_readfirstlane(__syncthreads_or(any));
    ymax = fred[0];
#pragma unroll
    for (int w = 1; w < kBrickThreads / 64; ++w) ymax = fmaxf(ymax, fred[w]);
    // the same in every lane: held in a scalar register through pass 2
    ymax = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(ymax)));

    float scale = 0.0f, inv_scale = 0.0f;
    if (ymax > 0.0f) {
        const double diag = sqrt(V.s[0] * V.s[0] + V.s[1] * V.s[1] + V.s[2] * V.s[2]);
        const int e =
            clampi((int)floor(log2(1073741824.0 / ((double)ymax * diag))), -126, 126);
        scale = ldexpf(1.0f, e);
        inv_scale = ldexpf(1.0f, -e);
    }

    // pass 2: every finite ray's pieces in the brick into the copy; a ray the
    // brick test takes here but did not take in pass 1 (the two inlined copies
    // could round a tie apart) goes with the non-finite ones below, so no piece
    // exceeds the int32 range
    if (any) {
        for_candidates([&](int v, int r, int c, long long i) {
            const float y = siddon_coef<MODE>(grad_out, s_in, i);
            if (y == 0.0f || !isfinite(y)) return;
            SiddonRay S;
            double t_in, t_out;
            if (!siddon_clip(geo[v], V, r, c, S) || !siddon_brick_range(S, V, b, t_in, t_out))
                return;
            if (fabsf(y) > ymax) {
                late = 1;                            // (rare: one LDS store)
                return;
            }
            siddon_brick_start(S, V, b, t_in);
            const float ys = y * scale;
            siddon_brick_walk<B>(S, b, t_in, t_out, [&](int e, double len) {
                const long long val = (long long)__float2int_rn((float)len * ys);
                atomicAdd(&acc[e], (unsigned long long)val);
            });
        });
    }
    __syncthreads();
    poison |= late;

    // the brick's voxels, written once
    const uint32_t sy = (uint32_t)V.n[0], sz = (uint32_t)V.n[0] * (uint32_t)V.n[1];
    const double inv = (double)inv_scale;
    for (int i = t; i < B * B * B; i += kBrickThreads) {
        const int x = i % B, y = (i / B) % B, z = i / (B * B);
        if (x >= b.e[0] || y >= b.e[1] || z >= b.e[2]) continue;
        grad[(uint32_t)(b.lo[2] + z) * sz + (uint32_t)(b.lo[1] + y) * sy +
             (uint32_t)(b.lo[0] + x)] = (float)((double)(long long)acc[i] * inv);
    }
    if (!poison) return;

    // rays whose y is not finite or above ymax: float atomics to the brick's
    // own voxels, after the stores above are visible
    __threadfence();
    __syncthreads();
    for_candidates([&](int v, int r, int c, long long i) {
        const float y = siddon_coef<MODE>(grad_out, s_in, i);
        if (isfinite(y) && fabsf(y) <= ymax) return;
        SiddonRay S;
        double t_in, t_out;
        if (!siddon_clip(geo[v], V, r, c, S) || !siddon_brick_range(S, V, b, t_in, t_out))
            return;
        siddon_brick_start(S, V, b, t_in);
        siddon_brick_walk<B>(S, b, t_in, t_out, [&](int e, double len) {
            if (!(len > 0.0)) return;               // (infinity times 0 would be NaN)
            const int x = e % B, yy = (e / B) % B, z = e / (B * B);
            unsafeAtomicAdd(grad + (uint32_t)(b.lo[2] + z) * sz + (uint32_t)(b.lo[1] + yy) * sy +
                                (uint32_t)(b.lo[0] + x),
                            y * (float)len);
        });
    });
}

hipError_t launch_siddon_brick_backward(const LaunchArgs& a, const float* grad_out,
                                        const float* s_in, float* grad, hipStream_t stream)
{
    constexpr int B = kSiddonBrickSide;
    const int nbx = (a.V.n[0] + B - 1) / B, nby = (a.V.n[1] + B - 1) / B;
    const int nbz = (a.V.n[2] + B - 1) / B;
    const dim3 grid((unsigned)(nbx * nby * nbz)), block(kBrickThreads);
    if (a.mode == kBeerLambert)
        hipLaunchKernelGGL((drr_siddon_brick_kernel<kBeerLambert>), grid, block, 0, stream, a.V,
                           a.K, a.poses, a.n_views, a.H, a.W, grad_out, s_in, grad, nbx, nby);
    else
        hipLaunchKernelGGL((drr_siddon_brick_kernel<kLineIntegral>), grid, block, 0, stream, a.V,
                           a.K, a.poses, a.n_views, a.H, a.W, grad_out, s_in, grad, nbx, nby);
    return hipGetLastError();
}

}  // namespace drr
