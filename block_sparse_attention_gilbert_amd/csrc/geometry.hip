// Geometric overlap and coverage of query blocks against historical frustum
// slabs: camera-facing oriented boxes, a separating-axis test, a grid
// intersection-over-union, and the share of a query block's tokens that fall
// inside a historical slab.
//
// [Velox: Spatial Memory Makes World Models Efficient -- Methodology, Step 1:
//  a historical block is kept as frustum slabs (a token rectangle in its
//  source camera plus a depth interval); Step 3: query and historical slabs
//  are approximated by camera-facing oriented boxes, the score is the IoU of
//  the query box with the best-matching historical box, computed on a
//  deterministic grid after a separating-axis test, and a coverage score
//  counts the query tokens that fall inside a valid historical slab both
//  spatially and in depth]
//
// Camera record (16 float64): fx, fy, cx, cy (token units), R row-major
// (world-from-camera; its columns are the camera's right, down and forward
// axes), C (centre).  A camera point (x, y, z), z > 0, sits at token
// coordinates u = fx x / z + cx, v = fy y / z + cy.  Slab record (6 float64):
// u0, v0, u1, v1 (the rectangle [u0, u1) x [v0, v1)), z_lo, z_hi.
//
// The box of a slab has the camera's axes, its centre on the ray through
// the rectangle's centre at the middle depth z_m, and half extents equal to
// the rectangle's half width and height at z_m and half the depth interval.
// Arithmetic is float64.
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace bsa {
namespace {

constexpr double kAxisEps2 = 1e-12;

struct Box {
    double c[3];
    double a[3][3];  // a[k] = unit axis k in world space
    double e[3];
};

__device__ __forceinline__ double dot3(const double* x, const double* y) {
    return x[0] * y[0] + x[1] * y[1] + x[2] * y[2];
}

__device__ __forceinline__ void slab_box(const double* __restrict__ cam, const double* __restrict__ g, Box& b) {
    const double fx = cam[0], fy = cam[1], cx = cam[2], cy = cam[3];
    const double* R = cam + 4;
    const double* C = cam + 13;
    const double zm = (g[4] + g[5]) / 2.0;
    const double uc = (g[0] + g[2]) / 2.0, vc = (g[1] + g[3]) / 2.0;
    const double pc[3] = {(uc - cx) * zm / fx, (vc - cy) * zm / fy, zm};
#pragma unroll
    for (int r = 0; r < 3; ++r) b.c[r] = dot3(R + 3 * r, pc) + C[r];
#pragma unroll
    for (int k = 0; k < 3; ++k)
#pragma unroll
        for (int r = 0; r < 3; ++r) b.a[k][r] = R[3 * r + k];
    b.e[0] = (g[2] - g[0]) * zm / (2.0 * fx);
    b.e[1] = (g[3] - g[1]) * zm / (2.0 * fy);
    b.e[2] = (g[5] - g[4]) / 2.0;
}

// Whether axis L separates the boxes.
__device__ __forceinline__ bool separates(const double* L, const Box& A, const Box& B, const double* d) {
    double ra = 0.0, rb = 0.0;
#pragma unroll
    for (int k = 0; k < 3; ++k) ra += A.e[k] * fabs(dot3(L, A.a[k]));
#pragma unroll
    for (int k = 0; k < 3; ++k) rb += B.e[k] * fabs(dot3(L, B.a[k]));
    return fabs(dot3(L, d)) > ra + rb;
}

// Separating-axis test over the 15 axes (face normals of both boxes and the
// cross products of their edges; near-parallel edge pairs are skipped).
__device__ bool separated(const Box& A, const Box& B) {
    const double d[3] = {B.c[0] - A.c[0], B.c[1] - A.c[1], B.c[2] - A.c[2]};
    for (int k = 0; k < 3; ++k)
        if (separates(A.a[k], A, B, d)) return true;
    for (int k = 0; k < 3; ++k)
        if (separates(B.a[k], A, B, d)) return true;
    for (int i = 0; i < 3; ++i) {
        for (int j = 0; j < 3; ++j) {
            const double* x = A.a[i];
            const double* y = B.a[j];
            const double L[3] = {x[1] * y[2] - x[2] * y[1], x[2] * y[0] - x[0] * y[2], x[0] * y[1] - x[1] * y[0]};
            if (dot3(L, L) >= kAxisEps2 && separates(L, A, B, d)) return true;
        }
    }
    return false;
}

// IoU of query box A and historical box B on the n^3 cell centres of A.
__device__ double grid_iou(const Box& A, const Box& B, int n) {
    if (separated(A, B)) return 0.0;
    int cnt = 0;
    for (int i = 0; i < n; ++i) {
        const double si = (2.0 * i + 1.0) / n - 1.0;
        double pi[3];
#pragma unroll
        for (int r = 0; r < 3; ++r) pi[r] = (si * A.e[0]) * A.a[0][r];
        for (int j = 0; j < n; ++j) {
            const double sj = (2.0 * j + 1.0) / n - 1.0;
            double pj[3];
#pragma unroll
            for (int r = 0; r < 3; ++r) pj[r] = pi[r] + (sj * A.e[1]) * A.a[1][r];
            for (int l = 0; l < n; ++l) {
                const double sl = (2.0 * l + 1.0) / n - 1.0;
                double q[3];
#pragma unroll
                for (int r = 0; r < 3; ++r) q[r] = A.c[r] + (pj[r] + (sl * A.e[2]) * A.a[2][r]) - B.c[r];
                bool in = true;
#pragma unroll
                for (int m = 0; m < 3; ++m) in = in && fabs(dot3(q, B.a[m])) <= B.e[m];
                cnt += in ? 1 : 0;
            }
        }
    }
    const double va = 8.0 * A.e[0] * A.e[1] * A.e[2];
    const double vb = 8.0 * B.e[0] * B.e[1] * B.e[2];
    const double inter = va * cnt / (double)(n * n * n);
    const double uni = va + vb - inter;
    return uni > 0.0 ? inter / uni : 0.0;
}

__device__ __forceinline__ int clamp_range(int x, int n) { return x < 0 ? 0 : (x > n ? n : x); }

// One thread per (query block i, historical block j): the largest IoU over
// the pairs of their slabs.  grid = (ceil(nkb / 256), nqb).
__global__ void __launch_bounds__(256)
slab_overlap_kernel(const double* __restrict__ cams, int n_cams, const int32_t* __restrict__ q_ptr,
                    const int32_t* __restrict__ q_cam, const double* __restrict__ q_geom, int n_q,
                    const int32_t* __restrict__ h_ptr, const int32_t* __restrict__ h_cam,
                    const double* __restrict__ h_geom, int n_h, int nkb, int n, float* __restrict__ overlap,
                    int64_t stride) {
    const int i = blockIdx.y;
    const int j = blockIdx.x * 256 + threadIdx.x;
    if (j >= nkb) return;
    const int qa = clamp_range(q_ptr[i], n_q), qb = clamp_range(q_ptr[i + 1], n_q);
    const int ha = clamp_range(h_ptr[j], n_h), hb = clamp_range(h_ptr[j + 1], n_h);
    double best = 0.0;
    for (int a = qa; a < qb; ++a) {
        const int ca = q_cam[a];
        if (ca < 0 || ca >= n_cams) continue;
        Box A;
        slab_box(cams + 16 * ca, q_geom + 6 * a, A);
        for (int b = ha; b < hb; ++b) {
            const int cb = h_cam[b];
            if (cb < 0 || cb >= n_cams) continue;
            Box B;
            slab_box(cams + 16 * cb, h_geom + 6 * b, B);
            best = fmax(best, grid_iou(A, B, n));
        }
    }
    overlap[(int64_t)i * stride + j] = (float)best;
}

// One workgroup of 16 waves per query block.  The block's tokens are split
// in groups of 64 (one per lane); the historical slabs are split among the
// waves of a token group (wave-uniform slab index, so slab and camera loads
// are scalar).  A token is covered when its point lies inside any slab.
__global__ void __launch_bounds__(1024)
slab_coverage_kernel(const double* __restrict__ cams, int n_cams, const int32_t* __restrict__ perm, int L, int H,
                     int W, int block, const int32_t* __restrict__ frame_cam, const float* __restrict__ depth,
                     const int32_t* __restrict__ h_cam, const double* __restrict__ h_geom, int n_h,
                     float* __restrict__ coverage) {
    __shared__ int flag[256];
    const int i = blockIdx.x, t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int groups = (block + 63) / 64, per = 16 / groups;
    const int g = w / per, s = w % per;
    const int g0 = i * block, g1 = min(L, g0 + block), ntok = g1 - g0;
    if (t < 256) flag[t] = 0;
    __syncthreads();
    const int tok = g * 64 + lane;
    const bool mine = g < groups && tok < ntok;
    double X[3] = {0.0, 0.0, 0.0};
    bool has_point = false;
    if (mine) {
        const int cell = perm[g0 + tok];
        const bool in_grid = cell >= 0 && cell < L;
        const int c = in_grid ? cell : 0;
        const int tt = c / (H * W), rem = c % (H * W), hh = rem / W, ww = rem % W;
        const int cf = frame_cam[tt];
        const double z = (double)depth[c];
        if (in_grid && cf >= 0 && cf < n_cams && z > 0.0) {
            const double* cam = cams + 16 * cf;
            const double pc[3] = {((ww + 0.5) - cam[2]) * z / cam[0], ((hh + 0.5) - cam[3]) * z / cam[1], z};
#pragma unroll
            for (int r = 0; r < 3; ++r) X[r] = dot3(cam + 4 + 3 * r, pc) + cam[13 + r];
            has_point = true;
        }
    }
    bool covered = false;
    if (g < groups) {
        for (int k = s; k < n_h; k += per) {
            if (__all(!has_point || covered)) break;
            const int cs = h_cam[k];
            if (cs < 0 || cs >= n_cams) continue;
            const double* cam = cams + 16 * cs;
            const double* geo = h_geom + 6 * k;
            const double d[3] = {X[0] - cam[13], X[1] - cam[14], X[2] - cam[15]};
            // camera coordinates: R^T d (R's columns are the camera axes)
            const double x = cam[4] * d[0] + cam[7] * d[1] + cam[10] * d[2];
            const double y = cam[5] * d[0] + cam[8] * d[1] + cam[11] * d[2];
            const double z = cam[6] * d[0] + cam[9] * d[1] + cam[12] * d[2];
            if (has_point && !covered && z > 0.0) {
                const double u = cam[0] * x / z + cam[2], v = cam[1] * y / z + cam[3];
                covered = geo[0] <= u && u < geo[2] && geo[1] <= v && v < geo[3] && geo[4] <= z && z <= geo[5];
            }
        }
    }
    if (mine && covered) atomicOr(&flag[tok], 1);
    __syncthreads();
    if (w == 0) {
        int cnt = 0;
        for (int x = lane; x < ntok; x += 64) cnt += flag[x];
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o);
        if (lane == 0) coverage[i] = ntok > 0 ? (float)((double)cnt / (double)ntok) : 0.0f;
    }
}

}  // namespace

hipError_t launch_slab_overlap(const double* cams, int n_cams, const int32_t* q_ptr, const int32_t* q_cam,
                               const double* q_geom, int nqb, int n_q, const int32_t* h_ptr, const int32_t* h_cam,
                               const double* h_geom, int nkb, int n_h, int grid_n, float* overlap, int64_t stride,
                               hipStream_t stream) {
    const dim3 grid((nkb + 255) / 256, nqb);
    hipLaunchKernelGGL(slab_overlap_kernel, grid, dim3(256), 0, stream, cams, n_cams, q_ptr, q_cam, q_geom, n_q, h_ptr,
                       h_cam, h_geom, n_h, nkb, grid_n, overlap, stride);
    return hipGetLastError();
}

hipError_t launch_slab_coverage(const double* cams, int n_cams, const int32_t* perm, int T, int H, int W, int block,
                                const int32_t* frame_cam, const float* depth, const int32_t* h_cam,
                                const double* h_geom, int n_h, float* coverage, hipStream_t stream) {
    const int L = T * H * W;
    const int nqb = (L + block - 1) / block;
    hipLaunchKernelGGL(slab_coverage_kernel, dim3(nqb), dim3(1024), 0, stream, cams, n_cams, perm, L, H, W, block,
                       frame_cam, depth, h_cam, h_geom, n_h, coverage);
    return hipGetLastError();
}

}  // namespace bsa
