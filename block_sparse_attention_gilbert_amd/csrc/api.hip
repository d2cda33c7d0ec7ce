// C ABI entry points: validate on the host, then enqueue on the caller's
// stream.  See include/bsa.h for the contract of each function.
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace {

int hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return BSA_OK;
    return bsa::fail(BSA_EHIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

extern "C" {

int bsa_gilbert_index(int T, int H, int W, int32_t* perm, int32_t* inv, hipStream_t stream) {
    bsa::clear_error();
    const int st = bsa::validate_gilbert_index(T, H, W, perm);
    if (st != BSA_OK) return st;
    return hip_status(bsa::launch_gilbert_index(T, H, W, perm, inv, stream), "gilbert_index launch");
}

int bsa_gilbert_perm(const void* src, void* dst, const int32_t* perm, int L, int heads, int d, int block,
                     int64_t raster_token_stride, int64_t gilbert_head_stride, int inverse, int dtype,
                     hipStream_t stream) {
    bsa::clear_error();
    const int st = bsa::validate_gilbert_perm(src, dst, perm, L, heads, d, block, raster_token_stride,
                                              gilbert_head_stride, inverse, dtype);
    if (st != BSA_OK) return st;
    return hip_status(bsa::launch_gilbert_perm(src, dst, perm, L, heads, d, block, raster_token_stride,
                                               gilbert_head_stride, inverse, dtype, stream),
                      "gilbert_perm launch");
}

int bsa_gilbert_perm_pool(const void* src, void* dst, const int32_t* perm, int L, int heads, int d, int block,
                          int64_t raster_token_stride, int64_t gilbert_head_stride, int dtype, double* pool,
                          int64_t pool_head_stride, hipStream_t stream) {
    bsa::clear_error();
    const int st = bsa::validate_gilbert_perm_pool(src, dst, perm, L, heads, d, block, raster_token_stride,
                                                   gilbert_head_stride, dtype, pool, pool_head_stride);
    if (st != BSA_OK) return st;
    return hip_status(bsa::launch_gilbert_perm_pool(src, dst, perm, L, heads, d, block, raster_token_stride,
                                                    gilbert_head_stride, dtype, pool, pool_head_stride, stream),
                      "gilbert_perm_pool launch");
}

int bsa_gilbert_perm_pool_batch(const bsa_perm_job* jobs, int n_jobs, const int32_t* perm, int L, int heads, int d,
                                int block, int dtype, hipStream_t stream) {
    bsa::clear_error();
    const int st = bsa::validate_gilbert_perm_pool_batch(jobs, n_jobs, perm, L, heads, d, block, dtype);
    if (st != BSA_OK) return st;
    return hip_status(bsa::launch_gilbert_perm_pool_batch(jobs, n_jobs, perm, L, heads, d, block, dtype, stream),
                      "gilbert_perm_pool_batch launch");
}

int bsa_route_topk(const bsa_route_args* args, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    bsa::clear_error();
    bsa::RouteLayout lay;
    const int st = bsa::validate_route(args, &lay);
    if (st != BSA_OK) return st;
    if (!workspace) return bsa::fail(BSA_EWORKSPACE, "workspace is NULL (%zu bytes needed)", lay.total);
    if (workspace_bytes < lay.total)
        return bsa::fail(BSA_EWORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, lay.total);
    if (reinterpret_cast<uintptr_t>(workspace) & 255u)
        return bsa::fail(BSA_EWORKSPACE, "workspace must be 256-byte aligned");
    return hip_status(bsa::launch_route(args, lay, workspace, stream), "route launch");
}

int bsa_route_topk_static(const bsa_route_args* args, hipStream_t stream) {
    bsa::clear_error();
    bsa::RouteLayout lay;
    const int st = bsa::validate_route(args, &lay);
    if (st != BSA_OK) return st;
    if (lay.total > (size_t)BSA_ROUTE_STATIC_SCRATCH_BYTES)
        return bsa::fail(BSA_EWORKSPACE,
                         "these arguments need %zu bytes of scratch; the static scratch holds %zu (pass kpool and "
                         "sel_keys to shrink the need, or call bsa_route_topk with a workspace)",
                         lay.total, (size_t)BSA_ROUTE_STATIC_SCRATCH_BYTES);
    void* ws = nullptr;
    const int rs = hip_status(bsa::static_route_scratch(&ws), "static scratch lookup");
    if (rs != BSA_OK) return rs;
    return hip_status(bsa::launch_route(args, lay, ws, stream), "route launch");
}

int bsa_gilbert_block_window(const int32_t* perm, const int32_t* inv, int T, int H, int W, int block, int q_chunk,
                             int32_t* window, int32_t* window_len, int window_stride, hipStream_t stream) {
    bsa::clear_error();
    const int st = bsa::validate_block_window(perm, inv, T, H, W, block, q_chunk, window, window_len, window_stride);
    if (st != BSA_OK) return st;
    return hip_status(bsa::launch_block_window(perm, inv, T, H, W, block, q_chunk, window, window_len, window_stride,
                                               stream),
                      "gilbert_block_window launch");
}

int bsa_gilbert_tile_index(int T, int H, int W, int tile_t, int tile_h, int tile_w, int32_t* row_cell,
                           int32_t* block_len, int32_t* cell_row, hipStream_t stream) {
    bsa::clear_error();
    const int st = bsa::validate_tile_index(T, H, W, tile_t, tile_h, tile_w, row_cell, block_len);
    if (st != BSA_OK) return st;
    return hip_status(bsa::launch_tile_index(T, H, W, tile_t, tile_h, tile_w, row_cell, block_len, cell_row, stream),
                      "gilbert_tile_index launch");
}

int bsa_tile_perm(const void* src, void* dst, const int32_t* row_cell, int n_rows, int L, int heads, int d,
                  int64_t raster_token_stride, int64_t tiled_head_stride, int inverse, int dtype, hipStream_t stream) {
    bsa::clear_error();
    const int st = bsa::validate_tile_perm(src, dst, row_cell, n_rows, L, heads, d, raster_token_stride,
                                           tiled_head_stride, inverse, dtype);
    if (st != BSA_OK) return st;
    return hip_status(bsa::launch_tile_perm(src, dst, row_cell, n_rows, L, heads, d, raster_token_stride,
                                            tiled_head_stride, inverse, dtype, stream),
                      "tile_perm launch");
}

int bsa_tile_block_window(const int32_t* row_cell, const int32_t* cell_row, int n_rows, int T, int H, int W, int block,
                          int q_chunk, int32_t* window, int32_t* window_len, int window_stride, hipStream_t stream) {
    bsa::clear_error();
    const int st = bsa::validate_tile_block_window(row_cell, cell_row, n_rows, T, H, W, block, q_chunk, window,
                                                   window_len, window_stride);
    if (st != BSA_OK) return st;
    return hip_status(bsa::launch_tile_block_window(row_cell, cell_row, n_rows, T, H, W, block, q_chunk, window,
                                                    window_len, window_stride, stream),
                      "tile_block_window launch");
}

int bsa_route_materialize(const bsa_route_args* args, const bsa_materialize_args* margs, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
    bsa::clear_error();
    bsa::RouteLayout lay;
    const int st = bsa::validate_materialize(args, margs, &lay);
    if (st != BSA_OK) return st;
    if (!workspace) return bsa::fail(BSA_EWORKSPACE, "workspace is NULL (%zu bytes needed)", lay.total);
    if (workspace_bytes < lay.total)
        return bsa::fail(BSA_EWORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, lay.total);
    if (reinterpret_cast<uintptr_t>(workspace) & 255u)
        return bsa::fail(BSA_EWORKSPACE, "workspace must be 256-byte aligned");
    return hip_status(bsa::launch_materialize(args, margs, lay, workspace, stream), "route_materialize launch");
}

int bsa_slab_overlap(const double* cams, int n_cams, const int32_t* q_slab_ptr, const int32_t* q_slab_cam,
                     const double* q_slab_geom, int nqb, int n_q_slabs, const int32_t* h_slab_ptr,
                     const int32_t* h_slab_cam, const double* h_slab_geom, int nkb, int n_h_slabs, int grid_n,
                     float* overlap, int64_t overlap_row_stride, hipStream_t stream) {
    bsa::clear_error();
    const int st = bsa::validate_slab_overlap(cams, n_cams, q_slab_ptr, q_slab_cam, q_slab_geom, nqb, n_q_slabs,
                                              h_slab_ptr, h_slab_cam, h_slab_geom, nkb, n_h_slabs, grid_n, overlap,
                                              overlap_row_stride);
    if (st != BSA_OK) return st;
    return hip_status(bsa::launch_slab_overlap(cams, n_cams, q_slab_ptr, q_slab_cam, q_slab_geom, nqb, n_q_slabs,
                                               h_slab_ptr, h_slab_cam, h_slab_geom, nkb, n_h_slabs, grid_n, overlap,
                                               overlap_row_stride, stream),
                      "slab_overlap launch");
}

int bsa_slab_coverage(const double* cams, int n_cams, const int32_t* perm, int T, int H, int W, int block,
                      const int32_t* frame_cam, const float* depth, const int32_t* h_slab_cam,
                      const double* h_slab_geom, int n_h_slabs, float* coverage, void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
    bsa::clear_error();
    const int st = bsa::validate_slab_coverage(cams, n_cams, perm, T, H, W, block, frame_cam, depth, h_slab_cam,
                                               h_slab_geom, n_h_slabs, coverage);
    if (st != BSA_OK) return st;
    const size_t need = bsa_slab_coverage_workspace_size(T, H, W);
    if (!workspace) return bsa::fail(BSA_EWORKSPACE, "workspace is NULL (%zu bytes needed)", need);
    if (workspace_bytes < need)
        return bsa::fail(BSA_EWORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
    if (reinterpret_cast<uintptr_t>(workspace) & 3u) return bsa::fail(BSA_EWORKSPACE, "workspace must be 4-byte aligned");
    return hip_status(bsa::launch_slab_coverage(cams, n_cams, perm, T, H, W, block, frame_cam, depth, h_slab_cam,
                                                h_slab_geom, n_h_slabs, coverage, workspace, stream),
                      "slab_coverage launch");
}

int bsa_block_sparse_attn(const void* q, const void* k, const void* v, void* o, float* lse, int dtype, int heads,
                          int d, int block, int nqb, int nkb, int64_t q_head_stride, int64_t k_head_stride,
                          int64_t v_head_stride, int64_t o_head_stride, const int32_t* q_block_len,
                          const int32_t* kv_block_len, const int32_t* row_ptr, const int32_t* col_idx,
                          int64_t col_len, float scale, hipStream_t stream) {
    bsa::clear_error();
    bsa::AttnProblem p{q,      k,     v,    o,       lse,          dtype,        heads,   d,       block,
                       nqb,    nkb,   q_head_stride, k_head_stride, v_head_stride, o_head_stride,
                       q_block_len, kv_block_len, row_ptr, col_idx, col_len, scale};
    const int st = bsa::validate_attn(p, false);
    if (st != BSA_OK) return st;
    return hip_status(bsa::launch_attn(p, false, stream), "block_sparse_attn launch");
}

int bsa_block_sparse_attn_raster(const void* q, const void* k, const void* v, void* o, float* lse, int dtype,
                                 int heads, int d, int block, int nqb, int nkb, int q_raster, int64_t q_stride,
                                 int64_t k_head_stride, int64_t v_head_stride, const int32_t* row_map, int rows,
                                 int64_t o_token_stride, const int32_t* q_block_len, const int32_t* kv_block_len,
                                 const int32_t* row_ptr, const int32_t* col_idx, int64_t col_len, float scale,
                                 hipStream_t stream) {
    bsa::clear_error();
    // the blocked strides of raster operands are not used; the raster
    // layouts are checked below
    const int64_t blocked = (int64_t)nqb * block * d;
    const bool qr = q_raster == 1;
    bsa::AttnProblem p{q,      k,     v,    o,       lse,          dtype,        heads,   d,       block,
                       nqb,    nkb,   qr ? blocked : q_stride, k_head_stride, v_head_stride, blocked,
                       q_block_len, kv_block_len, row_ptr, col_idx, col_len, scale, row_map, rows,
                       o_token_stride, qr ? row_map : nullptr, qr ? rows : 0, qr ? q_stride : 0};
    if (q_raster != 0 && q_raster != 1) return bsa::fail(BSA_EINVAL, "q_raster = %d (0 or 1)", q_raster);
    int st = bsa::validate_attn(p, false);
    if (st == BSA_OK) st = bsa::validate_raster_out(p);
    if (st != BSA_OK) return st;
    return hip_status(bsa::launch_attn(p, false, stream), "block_sparse_attn_raster launch");
}

int bsa_dense_attn(const void* q, const void* k, const void* v, void* o, float* lse, int dtype, int heads, int d,
                   int block, int nqb, int nkb, int64_t q_head_stride, int64_t k_head_stride,
                   int64_t v_head_stride, int64_t o_head_stride, const int32_t* q_block_len,
                   const int32_t* kv_block_len, float scale, hipStream_t stream) {
    bsa::clear_error();
    bsa::AttnProblem p{q,      k,     v,    o,       lse,          dtype,        heads,   d,       block,
                       nqb,    nkb,   q_head_stride, k_head_stride, v_head_stride, o_head_stride,
                       q_block_len, kv_block_len, nullptr, nullptr, 0, scale};
    const int st = bsa::validate_attn(p, true);
    if (st != BSA_OK) return st;
    return hip_status(bsa::launch_attn(p, true, stream), "dense_attn launch");
}

int bsa_diag_mfma_bf16(int workgroups, int iters, float* sink, hipStream_t stream) {
    bsa::clear_error();
    if (workgroups < 1 || workgroups > 1 << 20 || iters < 1 || !sink)
        return bsa::fail(BSA_EINVAL, "workgroups %d, iters %d must be >= 1 (workgroups <= 2^20), sink non-NULL",
                         workgroups, iters);
    return hip_status(bsa::launch_mfma_probe(workgroups, iters, sink, stream), "mfma probe launch");
}

}  // extern "C"
