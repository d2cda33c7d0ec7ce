// Kernel launchers of the bsa library (internal; the C ABI is in bsa.h).
// Each launcher enqueues on `stream` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>

#include "common.h"

namespace bsa {

hipError_t launch_gilbert_index(int T, int H, int W, int32_t* perm, int32_t* inv, hipStream_t stream);

hipError_t launch_gilbert_perm(const void* src, void* dst, const int32_t* perm, int L, int heads, int d,
                               int block, int64_t raster_token_stride, int64_t gilbert_head_stride,
                               int inverse, int dtype, hipStream_t stream);

hipError_t launch_gilbert_perm_pool(const void* src, void* dst, const int32_t* perm, int L, int heads, int d,
                                    int block, int64_t raster_token_stride, int64_t gilbert_head_stride, int dtype,
                                    double* pool, int64_t pool_head_stride, hipStream_t stream);

hipError_t launch_gilbert_perm_pool_batch(const bsa_perm_job* jobs, int n_jobs, const int32_t* perm, int L,
                                          int heads, int d, int block, int dtype, hipStream_t stream);

hipError_t launch_route(const bsa_route_args* a, const RouteLayout& lay, void* ws, hipStream_t stream);

// Device address of the router's fixed scratch (BSA_ROUTE_STATIC_SCRATCH_BYTES)
// on the current device, looked up once per device.
hipError_t static_route_scratch(void** ptr);

hipError_t launch_block_window(const int32_t* perm, const int32_t* inv, int T, int H, int W, int block, int q_chunk,
                               int32_t* window, int32_t* window_len, int stride, hipStream_t stream);

hipError_t launch_tile_block_window(const int32_t* row_cell, const int32_t* cell_row, int n_rows, int T, int H, int W,
                                    int block, int q_chunk, int32_t* window, int32_t* window_len, int stride,
                                    hipStream_t stream);

hipError_t launch_tile_index(int T, int H, int W, int tt, int th, int tw, int32_t* row_cell, int32_t* block_len,
                             int32_t* cell_row, hipStream_t stream);

hipError_t launch_tile_perm(const void* src, void* dst, const int32_t* row_cell, int n_rows, int L, int heads, int d,
                            int64_t raster_token_stride, int64_t tiled_head_stride, int inverse, int dtype,
                            hipStream_t stream);

hipError_t launch_materialize(const bsa_route_args* a, const bsa_materialize_args* m, const RouteLayout& lay,
                              void* ws, hipStream_t stream);

hipError_t launch_slab_overlap(const double* cams, int n_cams, const int32_t* q_ptr, const int32_t* q_cam,
                               const double* q_geom, int nqb, int n_q, const int32_t* h_ptr, const int32_t* h_cam,
                               const double* h_geom, int nkb, int n_h, int grid_n, float* overlap, int64_t stride,
                               hipStream_t stream);

hipError_t launch_slab_coverage(const double* cams, int n_cams, const int32_t* perm, int T, int H, int W, int block,
                                const int32_t* frame_cam, const float* depth, const int32_t* h_cam,
                                const double* h_geom, int n_h, float* coverage, void* ws, hipStream_t stream);

hipError_t launch_mfma_probe(int workgroups, int iters, float* sink, hipStream_t stream);

hipError_t launch_attn(const AttnProblem& p, bool dense, hipStream_t stream);

}  // namespace bsa
