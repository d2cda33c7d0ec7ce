// Geometric overlap and coverage of query blocks against historical frustum
// slabs: camera-facing oriented boxes, a separating-axis test, a grid
// intersection-over-union, and the share of a query block's tokens that fall
// inside a historical slab.
//
// [Velox: Spatial Memory Makes World Models Efficient -- Methodology, Step 1:
//  the geometry of a historical block is a set of frustum slabs, each a
//  rectangle of tokens in the camera that saw it and a range of depths;
//  Step 3: every slab becomes an oriented box facing its camera; the score
//  of a query block is the largest IoU of its box with a historical box,
//  measured on a fixed grid once a separating-axis test has not ruled the
//  pair out; coverage is the share of its tokens that lie in some valid
//  historical slab, inside the rectangle and the depth range]
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

__device__ __forceinline__ int clamp_range(int x, int n) { return x < 0 ? 0 : (x > n ? n : x); }

constexpr int kMaxGrid = 64;

// One lane per (query block i, historical block j), 64 consecutive j per
// wave; grid = (ceil(nkb / 256), nqb).  For each query slab (the same for
// the whole workgroup) and each position b in the historical block's slab
// list, every lane builds its historical box and runs the separating-axis
// test; the pairs that pass are then counted one at a time by the whole
// wave, each lane taking every 64th point of the query box's grid.  A
// lane's largest IoU is its result.
__global__ void __launch_bounds__(256)
slab_overlap_kernel(const double* __restrict__ cams, int n_cams, const int32_t* __restrict__ q_ptr,
                    const int32_t* __restrict__ q_cam, const double* __restrict__ q_geom, int n_q,
                    const int32_t* __restrict__ h_ptr, const int32_t* __restrict__ h_cam,
                    const double* __restrict__ h_geom, int n_h, int nkb, int n, float* __restrict__ overlap,
                    int64_t stride) {
    __shared__ double sgrid[kMaxGrid];
    __shared__ Box hb_all[4][64];
    const int i = blockIdx.y, t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int j = blockIdx.x * 256 + t;
    if (t < n) sgrid[t] = (2.0 * t + 1.0) / n - 1.0;
    __syncthreads();
    const bool live = j < nkb;
    const int qa = clamp_range(q_ptr[i], n_q), qb = clamp_range(q_ptr[i + 1], n_q);
    int ha = 0, hn = 0;
    if (live) {
        ha = clamp_range(h_ptr[j], n_h);
        hn = clamp_range(h_ptr[j + 1], n_h) - ha;
        hn = hn < 0 ? 0 : hn;
    }
    int hmax = hn;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) hmax = max(hmax, __shfl_xor(hmax, o));
    Box* hb = hb_all[w];
    const int n3 = n * n * n, nn = n * n;
    double best = 0.0;
    for (int a = qa; a < qb; ++a) {
        const int ca = q_cam[a];
        if (ca < 0 || ca >= n_cams) continue;
        Box A;
        slab_box(cams + 16 * ca, q_geom + 6 * a, A);
        const double va = 8.0 * A.e[0] * A.e[1] * A.e[2];
        for (int b = 0; b < hmax; ++b) {
            bool need = false;
            if (b < hn) {
                const int cb = h_cam[ha + b];
                if (cb >= 0 && cb < n_cams) {
                    Box B;
                    slab_box(cams + 16 * cb, h_geom + 6 * (ha + b), B);
                    need = !separated(A, B);
                    hb[lane] = B;
                }
            }
            __builtin_amdgcn_wave_barrier();
            __asm__ volatile("" ::: "memory");
            unsigned long long pend = __ballot(need);
            while (pend) {
                const int owner = __ffsll((long long)pend) - 1;
                pend &= pend - 1;
                const Box& B = hb[owner];
                int cnt = 0;
                for (int idx = lane; idx < n3; idx += 64) {
                    const double si = sgrid[idx / nn], sj = sgrid[(idx / n) % n], sl = sgrid[idx % n];
                    double q[3];
#pragma unroll
                    for (int r = 0; r < 3; ++r)
                        q[r] = A.c[r] + (((si * A.e[0]) * A.a[0][r] + (sj * A.e[1]) * A.a[1][r]) +
                                         (sl * A.e[2]) * A.a[2][r]) - B.c[r];
                    bool in = true;
#pragma unroll
                    for (int m = 0; m < 3; ++m) in = in && fabs(dot3(q, B.a[m])) <= B.e[m];
                    cnt += in ? 1 : 0;
                }
#pragma unroll
                for (int o = 32; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o);
                if (lane == owner) {
                    const double vb = 8.0 * B.e[0] * B.e[1] * B.e[2];
                    const double inter = va * cnt / (double)n3;
                    const double uni = va + vb - inter;
                    best = fmax(best, uni > 0.0 ? inter / uni : 0.0);
                }
            }
            __builtin_amdgcn_wave_barrier();
            __asm__ volatile("" ::: "memory");
        }
    }
    if (live) overlap[(int64_t)i * stride + j] = (float)best;
}

// Coverage, first pass: one thread per token (curve position), a chunk of
// kCovChunk historical slabs per workgroup row (grid = (ceil(L / 256),
// ceil(n_h / kCovChunk))).  The chunk's slabs and their cameras are staged
// in LDS and read as broadcasts; a covered token sets its bit in `flags`
// (integer OR, so the order of the chunks does not matter).
constexpr int kCovChunk = 128;

struct SlabCam {
    double geo[6];
    double cam[16];
};

__global__ void __launch_bounds__(256)
slab_cover_flags_kernel(const double* __restrict__ cams, int n_cams, const int32_t* __restrict__ perm, int L, int H,
                        int W, const int32_t* __restrict__ frame_cam, const float* __restrict__ depth,
                        const int32_t* __restrict__ h_cam, const double* __restrict__ h_geom, int n_h,
                        uint32_t* __restrict__ flags) {
    __shared__ SlabCam sc[kCovChunk];
    __shared__ int ok[kCovChunk];
    const int t = threadIdx.x;
    const int k0 = blockIdx.y * kCovChunk, nk = min(kCovChunk, n_h - k0);
    for (int x = t; x < nk * 22; x += 256) {
        const int k = x / 22, f = x % 22;
        const int cs = h_cam[k0 + k];
        const bool good = cs >= 0 && cs < n_cams;
        double v = 0.0;
        if (f < 6)
            v = h_geom[6 * (k0 + k) + f];
        else if (good)
            v = cams[16 * cs + (f - 6)];
        if (f < 6)
            sc[k].geo[f] = v;
        else
            sc[k].cam[f - 6] = v;
        if (f == 0) ok[k] = good ? 1 : 0;
    }
    __syncthreads();
    const int gp = blockIdx.x * 256 + t;
    if (gp >= L) return;
    const int cell = perm[gp];
    if (cell < 0 || cell >= L) return;
    const int tt = cell / (H * W), rem = cell % (H * W), hh = rem / W, ww = rem % W;
    const int cf = frame_cam[tt];
    const double z0 = (double)depth[cell];
    if (cf < 0 || cf >= n_cams || !(z0 > 0.0)) return;
    const double* cam = cams + 16 * cf;
    const double pc[3] = {((ww + 0.5) - cam[2]) * z0 / cam[0], ((hh + 0.5) - cam[3]) * z0 / cam[1], z0};
    double X[3];
#pragma unroll
    for (int r = 0; r < 3; ++r) X[r] = dot3(cam + 4 + 3 * r, pc) + cam[13 + r];
    for (int k = 0; k < nk; ++k) {
        if (!ok[k]) continue;
        const double* c = sc[k].cam;
        const double* geo = sc[k].geo;
        const double d[3] = {X[0] - c[13], X[1] - c[14], X[2] - c[15]};
        // camera coordinates: R^T d (R's columns are the camera axes)
        const double x = c[4] * d[0] + c[7] * d[1] + c[10] * d[2];
        const double y = c[5] * d[0] + c[8] * d[1] + c[11] * d[2];
        const double z = c[6] * d[0] + c[9] * d[1] + c[12] * d[2];
        if (!(z > 0.0) || z < geo[4] || z > geo[5]) continue;
        const double u = c[0] * x / z + c[2], v = c[1] * y / z + c[3];
        if (geo[0] <= u && u < geo[2] && geo[1] <= v && v < geo[3]) {
            atomicOr(&flags[gp >> 5], 1u << (gp & 31));
            break;
        }
    }
}

__global__ void __launch_bounds__(256) fill_u32_kernel(uint32_t* __restrict__ p, int n) {
    const int x = blockIdx.x * 256 + threadIdx.x;
    if (x < n) p[x] = 0u;
}

// Coverage, second pass: one wave per query block counts the set bits of
// its curve positions.
__global__ void __launch_bounds__(256)
slab_cover_count_kernel(const uint32_t* __restrict__ flags, int L, int block, int nqb, float* __restrict__ coverage) {
    const int lane = threadIdx.x & 63;
    const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (i >= nqb) return;
    const int g0 = i * block, g1 = min(L, g0 + block);
    int cnt = 0;
    for (int gp = g0 + lane; gp < g1; gp += 64) cnt += (flags[gp >> 5] >> (gp & 31)) & 1u;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o);
    if (lane == 0) coverage[i] = g1 > g0 ? (float)((double)cnt / (double)(g1 - g0)) : 0.0f;
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
                                const double* h_geom, int n_h, float* coverage, void* ws, hipStream_t stream) {
    const int L = T * H * W;
    const int nqb = (L + block - 1) / block;
    const int words = (L + 31) / 32;
    uint32_t* flags = static_cast<uint32_t*>(ws);
    hipLaunchKernelGGL(fill_u32_kernel, dim3((words + 255) / 256), dim3(256), 0, stream, flags, words);
    if (n_h > 0) {
        const dim3 grid((L + 255) / 256, (n_h + kCovChunk - 1) / kCovChunk);
        hipLaunchKernelGGL(slab_cover_flags_kernel, grid, dim3(256), 0, stream, cams, n_cams, perm, L, H, W, frame_cam,
                           depth, h_cam, h_geom, n_h, flags);
    }
    hipLaunchKernelGGL(slab_cover_count_kernel, dim3((nqb + 3) / 4), dim3(256), 0, stream, flags, L, block, nqb,
                       coverage);
    return hipGetLastError();
}

}  // namespace bsa
