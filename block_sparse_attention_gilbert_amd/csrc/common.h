// Shared host-side helpers of the bsa library: status reporting and the
// argument records that the validation layer fills and the launchers read.
#pragma once

#include <cstddef>
#include <cstdint>

#include "bsa.h"

namespace bsa {

// Record a formatted detail for the calling thread and return `code`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();
const char* last_detail();

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline int dtype_bytes(int dtype) { return dtype == BSA_BF16 ? 2 : 4; }

// Validated attention problem (shared by the sparse and dense entry points).
struct AttnProblem {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int dtype;
    int heads, d, block, nqb, nkb;
    int64_t q_hs, k_hs, v_hs, o_hs;
    const int32_t* q_len;
    const int32_t* kv_len;
    const int32_t* row_ptr;  // NULL for dense
    const int32_t* col_idx;  // NULL for dense
    int64_t col_len;
    float scale;
    const int32_t* o_map;  // raster output: row map (NULL: blocked output)
    int o_map_len;
    int64_t o_ts;          // raster token stride of o, elements
    const int32_t* q_map;  // raster queries: row map (NULL: blocked queries)
    int q_map_len;
    int64_t q_ts;          // raster token stride of q, elements
};

// Workspace layout of the router (byte offsets, 256-byte aligned).  Rows
// with more than kSegCandidates candidates are selected in two levels: the
// top-K of each segment of kSegCandidates candidates (n_seg segments, at
// most seg_cap pairs each: order keys at seg_key, candidate indices at
// seg_idx, counts at seg_cnt), then the top-K over those pairs.
struct RouteLayout {
    size_t qbar, kbar, keys, keff, flags, bitmap, counts, seg_key, seg_idx, seg_cnt, total;
    int n_cand, n_seg, seg_cap;
    bool kbar_in_ws, keys_in_ws;
};

int validate_gilbert_index(int T, int H, int W, const int32_t* perm);
int validate_gilbert_perm(const void* src, const void* dst, const int32_t* perm, int L, int heads,
                          int d, int block, int64_t raster_token_stride,
                          int64_t gilbert_head_stride, int inverse, int dtype);
int validate_gilbert_perm_pool(const void* src, const void* dst, const int32_t* perm, int L, int heads, int d,
                               int block, int64_t raster_token_stride, int64_t gilbert_head_stride, int dtype,
                               const double* pool, int64_t pool_head_stride);
int validate_gilbert_perm_pool_batch(const bsa_perm_job* jobs, int n_jobs, const int32_t* perm, int L, int heads,
                                     int d, int block, int dtype);
int validate_attn(const AttnProblem& p, bool dense);
int validate_raster_out(const AttnProblem& p);
int validate_route(const bsa_route_args* a, RouteLayout* lay);
int validate_materialize(const bsa_route_args* a, const bsa_materialize_args* m, RouteLayout* lay);
int validate_block_window(const int32_t* perm, const int32_t* inv, int T, int H, int W, int block, int q_chunk,
                          const int32_t* window, const int32_t* window_len, int window_stride);
size_t route_layout(const bsa_route_args* a, RouteLayout* lay);

// Candidates one wave selects over (64 lanes x 64 keys in registers).
constexpr int kSegCandidates = 4096;
// Largest candidate count of the router (16 segments; the second level
// needs segments x min(K cap, kSegCandidates) <= kSegCandidates).
constexpr int kMaxCandidates = 16 * kSegCandidates;
// Largest KV block count of the route materialisation (one LDS bitmap bit
// per block and row).
constexpr int kMaxMaterializeBlocks = 4096;
int validate_tile_index(int T, int H, int W, int tt, int th, int tw, const int32_t* row_cell, const int32_t* block_len);
int validate_tile_perm(const void* src, const void* dst, const int32_t* row_cell, int n_rows, int L, int heads, int d,
                       int64_t raster_token_stride, int64_t tiled_head_stride, int inverse, int dtype);
int validate_tile_block_window(const int32_t* row_cell, const int32_t* cell_row, int n_rows, int T, int H, int W,
                               int block, int q_chunk, const int32_t* window, const int32_t* window_len,
                               int window_stride);
int validate_slab_overlap(const double* cams, int n_cams, const int32_t* q_ptr, const int32_t* q_cam,
                          const double* q_geom, int nqb, int n_q, const int32_t* h_ptr, const int32_t* h_cam,
                          const double* h_geom, int nkb, int n_h, int grid_n, const float* overlap, int64_t stride);
int validate_slab_coverage(const double* cams, int n_cams, const int32_t* perm, int T, int H, int W, int block,
                           const int32_t* frame_cam, const float* depth, const int32_t* h_cam, const double* h_geom,
                           int n_h, const float* coverage);

// Largest K_unc of the route materialisation.
constexpr int kMaxUncovered = 256;
// Largest number of blocks per chunk of the local-window builder.
constexpr int kMaxWindowChunkBlocks = 1024;

}  // namespace bsa
