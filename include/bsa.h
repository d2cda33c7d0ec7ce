/*
 * bsa.h -- C ABI of the routed, indexed block-sparse attention library for
 * AMD Instinct MI355X (gfx950).
 *
 * The library implements one hot path of chunked video world models whose
 * new chunk attends to a growing KV history:
 *
 *   1. a generalized-Hilbert ("Gilbert") token order of a latent chunk, so a
 *      run of consecutive tokens (a KV block) is a compact 3-D tile, and the
 *      permutation of raster tensors into that order
 *      [Velox: Spatial Memory Makes World Models Efficient -- Key
 *      Contributions 3; Methodology, Step 6] [Light Interaction -- abstract];
 *   2. a router: mean-pooled Q and K per block, a score for every
 *      (query block, KV block) pair, an optional soft geometric bias with
 *      unbiased fallback, and a top-K list per (head, query block)
 *      [Velox -- Key Contributions 1-2; Methodology, Steps 4-5];
 *   3. attention that visits only the listed KV blocks with an online
 *      softmax, and the dense case through the same kernel
 *      [Velox -- Methodology, Step 6; Main Findings].
 *
 * Conventions for every entry point
 * ---------------------------------
 * - Every function returns an int status (BSA_OK on success).  Arguments are
 *   validated on the host, synchronously, before anything is enqueued; on
 *   error nothing is enqueued and bsa_last_error_detail() describes the
 *   problem.  Kernel launch failures return BSA_EHIP.  Execution is
 *   asynchronous on the caller's stream; no entry point synchronises the
 *   host.
 * - Every data pointer is caller-owned DEVICE memory unless stated
 *   otherwise.  The library never allocates or frees; scratch memory is a
 *   caller buffer sized by the matching *_workspace_size function.  The
 *   library holds no mutable global state and is safe to call from several
 *   threads on different streams; the one exception is the fixed scratch
 *   of bsa_route_topk_static, which its own comment describes.
 * - Tensor pointers must be 16-byte aligned and head strides must keep every
 *   row 16-byte aligned.
 * - Results are deterministic: identical inputs give bitwise identical
 *   outputs (no atomics).
 * - dtype is BSA_BF16 (bfloat16 storage, fp32 accumulation) or BSA_F32.
 * - d (head dim) and block (tokens per block) are 64 or 128.
 */
#ifndef BSA_H
#define BSA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define BSA_OK 0
#define BSA_EINVAL 1        /* null, negative or inconsistent arguments */
#define BSA_EUNSUPPORTED 2  /* d, block or dtype outside what the kernels build for */
#define BSA_EWORKSPACE 3    /* workspace missing or too small */
#define BSA_EHIP 4          /* a HIP launch or runtime call failed */

/* dtypes */
#define BSA_BF16 0
#define BSA_F32 1

/* Library version, major * 10000 + minor * 100 + patch. */
int bsa_version(void);

/* Static description of a status code (never NULL). */
const char* bsa_strerror(int status);

/* Detail of the last error reported on the calling thread (never NULL;
 * empty after a successful call). */
const char* bsa_last_error_detail(void);

/*
 * bsa_gilbert_index -- generalized-Hilbert order of a T x H x W grid.
 * [Velox -- Key Contributions 3 ("global-aligned Gilbert KV storage");
 *  Methodology, Step 6 (neighbouring regions contiguous in memory)]
 *
 * perm[i] (int32, T*H*W entries) receives the raster index t*H*W + h*W + w of
 * the i-th cell on the curve; inv (nullable, T*H*W entries) receives the
 * inverse, inv[perm[i]] = i.  The curve starts at (0,0,0) and travels along
 * the longest axis (ties: w, then h); it takes unit steps whenever the
 * grid's parity allows a corner-to-corner path.  One thread per index
 * descends the curve's recursive subdivision.
 * Errors: BSA_EINVAL if a dimension is < 1, T*H*W exceeds 2^31-1, or perm is
 * NULL.
 */
int bsa_gilbert_index(int T, int H, int W, int32_t* perm, int32_t* inv, hipStream_t stream);

/*
 * bsa_gilbert_perm -- permute one chunk between raster token-major layout
 * and Gilbert-ordered, head-major, block-padded layout.
 * [Velox -- Key Contributions 3; Methodology, Step 6]
 *
 * Raster layout: element (token t, head h, channel c) at
 *   raster[t * raster_token_stride + h * d + c],   t < L.
 * Gilbert layout: element (head h, row i, channel c) at
 *   gil[h * gilbert_head_stride + i * d + c],      i < n_blocks * block,
 * with n_blocks = ceil(L / block).
 * inverse = 0: src is raster, dst is Gilbert; gil row i < L takes raster
 *   token perm[i]; rows L .. n_blocks*block-1 are written as zeros.
 * inverse = 1: src is Gilbert, dst is raster; raster token perm[i] takes
 *   gil row i (padded rows are not read).
 * The copy is bitwise.  dst may be a slice of a larger KV store (set
 * gilbert_head_stride to the store's head stride).  src and dst must not
 * overlap.  perm is device int32[L] (a permutation of 0..L-1).
 * Errors: BSA_EINVAL (null pointers, L < 1, heads < 1, strides too small,
 * misalignment), BSA_EUNSUPPORTED (d, block or dtype).
 */
int bsa_gilbert_perm(const void* src, void* dst, const int32_t* perm, int L, int heads, int d,
                     int block, int64_t raster_token_stride, int64_t gilbert_head_stride,
                     int inverse, int dtype, hipStream_t stream);

/*
 * bsa_gilbert_perm_pool -- the forward permutation of bsa_gilbert_perm
 * (inverse = 0) and, in the same pass, the mean of every block's valid
 * rows, for the router's pooled queries or pooled-key cache.
 * [Velox -- Methodology, Step 4 (per-block averages of queries and keys);
 *  Key Contributions 3; Methodology, Step 6]
 *
 * src, dst, perm, L, heads, d, block, raster_token_stride,
 * gilbert_head_stride, dtype   as bsa_gilbert_perm with inverse = 0;
 *                dst may be NULL: then only the block means are written
 *                (gilbert_head_stride is ignored).
 * pool           device float64: block b of head h (b < n_blocks =
 *                ceil(L / block)) receives, at pool[h * pool_head_stride +
 *                b * d + c], the mean over the block's valid rows (rows
 *                i < L) of channel c, summed in float64 (the same value as
 *                the router pools from dst).  pool may be a slice of a
 *                larger cache (pool_head_stride >= n_blocks * d, in
 *                elements); it must not overlap src or dst.
 * Errors: those of bsa_gilbert_perm (its src-side checks without dst);
 * BSA_EINVAL (pool NULL or not 8-byte aligned, pool_head_stride too small,
 * heads > 65535, pool overlapping src or dst).
 */
int bsa_gilbert_perm_pool(const void* src, void* dst, const int32_t* perm, int L, int heads, int d, int block,
                          int64_t raster_token_stride, int64_t gilbert_head_stride, int dtype, double* pool,
                          int64_t pool_head_stride, hipStream_t stream);

/*
 * bsa_gilbert_perm_pool_batch -- bsa_gilbert_perm_pool over several tensors
 * of one chunk that share its curve (say Q, K and V) in a single launch.
 * [Velox -- Methodology, Step 4 (per-block averages of queries and keys);
 *  Key Contributions 3; Methodology, Step 6]
 *
 * jobs           host array of n_jobs descriptions (1 <= n_jobs <=
 *                BSA_MAX_PERM_JOBS), read during the call only.  Job z
 *                moves jobs[z].src (raster, jobs[z].raster_token_stride) as
 *                bsa_gilbert_perm_pool does with its own dst (Gilbert
 *                slot, jobs[z].gilbert_head_stride; NULL = block means
 *                only) and pool (jobs[z].pool_head_stride; NULL = the
 *                permutation only, as bsa_gilbert_perm with inverse = 0).
 *                A job needs a dst or a pool.
 * perm, L, heads, d, block, dtype   shared by every job, as in
 *                bsa_gilbert_perm_pool.
 * The results are bitwise those of the single-tensor calls.  No job's dst or
 * pool may overlap any job's src, dst or pool.
 * Errors: those of bsa_gilbert_perm_pool for each job; BSA_EINVAL (jobs
 * NULL, n_jobs out of range, a job with neither dst nor pool, overlap
 * between jobs).
 */
#define BSA_MAX_PERM_JOBS 4

typedef struct bsa_perm_job {
    const void* src;
    void* dst;
    int64_t raster_token_stride;
    int64_t gilbert_head_stride;
    double* pool;
    int64_t pool_head_stride;
} bsa_perm_job;

int bsa_gilbert_perm_pool_batch(const bsa_perm_job* jobs, int n_jobs, const int32_t* perm, int L, int heads, int d,
                                int block, int dtype, hipStream_t stream);

/*
 * Router arguments.  Set struct_size = sizeof(bsa_route_args).
 * [Velox -- Methodology, Step 4 (block scores from the per-block averages
 *  of queries and keys; overlaps above tau, rescaled, scale them by
 *  (1 + lambda * g_hat) before normalising again, a boost of at most
 *  1 + lambda); Key Contributions 2 (without geometric cover the model's own
 *  scores decide); Methodology, Step 5 (the highest-scoring blocks, up to a
 *  budget)]
 *
 * Inputs (device unless noted):
 *  q, k           [heads][rows][d] in dtype, rows contiguous; q rows =
 *                 nqb*block, k rows = nkb*block; head strides in elements.
 *  q_block_len    int32[nqb] valid tokens per query block (NULL: all full).
 *  kv_block_len   int32[nkb] valid tokens per KV block (NULL: all full).
 *                 Rows past a block's valid length are never read; they
 *                 may hold anything.
 *  scale          score scale (normally 1/sqrt(d)).
 *  overlap        float32[nqb][overlap_row_stride] (NULL: no bias); entry
 *                 (i, j) is the geometric overlap of query block i with
 *                 candidate KV block j, shared by all heads.
 *  lambda, g_ref, tau   fusion constants (g_ref > 0).
 *  k_fixed        budget of every row, used when k_per_row is NULL.
 *  k_per_row      int32[heads*nqb] per-row budgets (NULL: k_fixed); values
 *                 are clamped to [0, k_max].
 *  k_max          upper bound of the per-row budgets (sizes col_idx).
 *  n_dense_tail_blocks  the last n_dense_tail_blocks KV blocks are not
 *                 candidates; every non-empty list ends with those of them
 *                 that hold a valid token (the current chunk, attended
 *                 densely).  Candidates are blocks 0 .. nkb-n_dense_tail-1.
 *  kpool          float64[heads][kpool_head_blocks][d] pooled-key cache
 *                 (NULL: pool every candidate into the workspace).  Blocks
 *                 < kpool_valid_blocks are taken from the cache as they
 *                 are; blocks >= kpool_valid_blocks are pooled and written
 *                 into it.  A KV history only grows by appending, so a
 *                 caller keeps the cache across calls and pools only the
 *                 blocks appended (or rewritten) since the last call.
 *  kpool_head_blocks  blocks per head of the cache (its head stride is
 *                 kpool_head_blocks*d); 0 means n_candidates.  Must be 0 or
 *                 >= n_candidates, so one cache can serve a growing history.
 *  qpool          float64 pooled queries (NULL: pool q): entry (h, i, c) at
 *                 qpool[h * qpool_head_stride + i * d + c] is the mean of
 *                 query block i's valid rows, as bsa_gilbert_perm_pool
 *                 writes it.  When given, q is not read and may be NULL.
 *  qpool_head_stride  elements between heads of qpool (>= nqb*d).
 * Outputs (device):
 *  row_ptr        int32[heads*nqb + 1]; row r = h*nqb + i.
 *  col_idx        int32[col_capacity]; row r's list is col_idx[row_ptr[r] ..
 *                 row_ptr[r+1]-1], ascending block indices.
 *  fallback_counts int32[2] (nullable): [0] query blocks whose overlap row is
 *                 all zero (unbiased fallback), [1] query blocks with no
 *                 overlap above tau (includes [0]).  Both 0 without overlap.
 *  sel_keys       float64[heads][nqb][n_candidates] (nullable): the
 *                 selection keys kappa = s + log1p(lambda * g_hat).
 *
 * Semantics: qbar, kbar = means over valid rows in float64 (exact sums);
 * s_ij = (qbar_i . kbar_j) * scale in float64; g_hat = 0 if g <= tau else
 * min(1, g / g_ref); the fused importance softmax(s)_j * (1 + lambda g_hat_j)
 * renormalised has the same order within a row as kappa_ij = s_ij +
 * log1p(lambda g_hat_ij), which is what is ranked.  A row keeps
 * K_eff = min(K_r, candidates with a valid token) blocks: the largest kappa,
 * ties to the lower block index; a query block with no valid token gets an
 * empty list.
 */
typedef struct bsa_route_args {
    size_t struct_size;
    const void* q;
    const void* k;
    int dtype;
    int heads;
    int d;
    int block;
    int nqb;
    int nkb;
    int64_t q_head_stride;
    int64_t k_head_stride;
    const int32_t* q_block_len;
    const int32_t* kv_block_len;
    double scale;
    const float* overlap;
    int64_t overlap_row_stride;
    double lambda;
    double g_ref;
    double tau;
    int k_fixed;
    const int32_t* k_per_row;
    int k_max;
    int n_dense_tail_blocks;
    double* kpool;
    int kpool_valid_blocks;
    int kpool_head_blocks;
    int32_t* row_ptr;
    int32_t* col_idx;
    int64_t col_capacity;
    int32_t* fallback_counts;
    double* sel_keys;
    const double* qpool;
    int64_t qpool_head_stride;
} bsa_route_args;

/* Bytes of workspace bsa_route_topk needs for these arguments (0 if the
 * arguments are invalid). */
size_t bsa_route_workspace_size(const bsa_route_args* args);

/*
 * bsa_route_topk -- pool, score, fuse and select; see bsa_route_args.
 * workspace: device memory of at least bsa_route_workspace_size(args) bytes,
 * 256-byte aligned, owned by the caller, not read before it is written.
 * Rows of up to 4096 candidates are selected by one wave each; longer
 * rows in segments of 4096 candidates, whose top-K are merged into the
 * row's top-K (the same lists, bit for bit).
 * Errors: BSA_EINVAL (arguments; col_capacity below
 * heads*nqb*(min(k cap, candidates) + n_dense_tail_blocks)),
 * BSA_EUNSUPPORTED (more than 65536 candidates, or more than 4096
 * candidates with ceil(candidates / 4096) * min(k cap, candidates) above
 * 4096; d, block or dtype), BSA_EWORKSPACE.
 */
int bsa_route_topk(const bsa_route_args* args, void* workspace, size_t workspace_bytes,
                   hipStream_t stream);

/*
 * bsa_route_topk_static -- bsa_route_topk with no workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  The scratch is a
 * fixed array of BSA_ROUTE_STATIC_SCRATCH_BYTES inside the library, one
 * copy per GPU, held from the library's load to the end of the process; its
 * device address is looked up on the first call on each device (the
 * caller's current device, which must be the one stream belongs to).  The
 * call itself allocates nothing.
 * Results are bitwise those of bsa_route_topk with the same arguments.
 * Calls that overlap in time on one GPU (different streams, or different
 * host threads) share that scratch and race: serialise them.  Nothing in
 * the scratch has to start at zero; each call writes what it reads.
 * Errors: those of bsa_route_topk; BSA_EWORKSPACE when
 * bsa_route_workspace_size(args) exceeds BSA_ROUTE_STATIC_SCRATCH_BYTES
 * (passing kpool and sel_keys leaves only the pooled queries, list lengths
 * and row flags in the scratch); BSA_EHIP if the address lookup fails.
 */
#define BSA_ROUTE_STATIC_SCRATCH_BYTES (32u << 20)

int bsa_route_topk_static(const bsa_route_args* args, hipStream_t stream);

/*
 * bsa_gilbert_block_window -- the local window of every query block of one
 * chunk, in block indices of the Gilbert-ordered history.
 * [Velox -- Methodology, Step 5 (every route also takes the block's 26
 *  neighbours in the Gilbert block order); Key Contributions 3 (KV storage
 *  in one Gilbert order aligned across chunks)]
 *
 * perm, inv      device int32[T*H*W]: a chunk grid's curve and its inverse
 *                (bsa_gilbert_index).  Chunk c of the history occupies
 *                blocks c*n_blocks .. (c+1)*n_blocks - 1, n_blocks =
 *                ceil(T*H*W / block), its tokens in curve order.
 * window         device int32[n_blocks][window_stride]: row b receives,
 *                ascending, the absolute indices of the KV blocks holding
 *                any cell of the 3 x 3 x 3 neighbourhood (the cell itself
 *                included, cut at the spatial border) of any token of
 *                query block b of chunk q_chunk.  A step back in time from
 *                a chunk's first frame lands in the last frame of chunk
 *                q_chunk - 1 (none for q_chunk = 0); a step forward from its
 *                last frame would land in chunk q_chunk + 1, which is not
 *                history and is left out.  Entries past window_len[b] are
 *                not written.
 * window_len     device int32[n_blocks]: entries of each row (<= 2*n_blocks).
 * Errors: BSA_EINVAL (null pointers, a dimension < 1, block < 1,
 * q_chunk < 0, window_stride < 2*n_blocks, block indices past 2^31-1),
 * BSA_EUNSUPPORTED (n_blocks > 1024).
 */
int bsa_gilbert_block_window(const int32_t* perm, const int32_t* inv, int T, int H, int W, int block,
                             int q_chunk, int32_t* window, int32_t* window_len, int window_stride,
                             hipStream_t stream);

/*
 * Fixed 3-D tile blocks.
 * [Light Interaction -- abstract (3-D block-sparse attention); Velox -- Key
 *  Contributions 3 (global-aligned Gilbert KV storage); Methodology,
 *  Step 5 (26-neighbour window in the Gilbert block ordering)]
 *
 * A block is a tile_t x tile_h x tile_w tile of the T x H x W chunk grid, on
 * the tile grid ceil(T/tile_t) x ceil(H/tile_h) x ceil(W/tile_w) aligned to
 * the chunk's origin (tiles at the far edges are clipped).  Block b is the
 * tile at position b of the Gilbert curve over the tile grid (the curve of
 * bsa_gilbert_index).  A block has V = tile_t*tile_h*tile_w rows: its
 * tile's cells in raster order, then padding, so every block carries a
 * valid length and every kernel that takes per-block lengths works on it
 * unchanged (attention and routing need V = 64 or 128).
 */

/*
 * bsa_gilbert_tile_index -- the tile layout of a chunk.
 * row_cell   int32[n_tiles*V]: raster cell of each row, -1 for padding.
 * block_len  int32[n_tiles]: valid rows of each block.
 * cell_row   int32[T*H*W] (nullable): the row of each cell.
 * Errors: BSA_EINVAL (dimensions < 1, rows or cells past 2^31-1, NULL
 * outputs).
 */
int bsa_gilbert_tile_index(int T, int H, int W, int tile_t, int tile_h, int tile_w, int32_t* row_cell,
                           int32_t* block_len, int32_t* cell_row, hipStream_t stream);

/*
 * bsa_tile_perm -- permute a chunk between raster token-major layout
 * (element (token t, head h, channel c) at raster[t * raster_token_stride +
 * h * d + c], t < L) and the tiled head-major layout (element (head h, row
 * i, channel c) at tiled[h * tiled_head_stride + i * d + c], i < n_rows)
 * through row_cell (bsa_gilbert_tile_index; entries outside [0, L) are
 * padding).  inverse = 0: raster -> tiled, padding rows written as zeros;
 * inverse = 1: tiled -> raster, padding rows not read.  Bitwise copy; src
 * and dst must not overlap.
 * Errors: BSA_EINVAL (null pointers, sizes, strides, alignment, overlap),
 * BSA_EUNSUPPORTED (d, dtype).
 */
int bsa_tile_perm(const void* src, void* dst, const int32_t* row_cell, int n_rows, int L, int heads,
                  int d, int64_t raster_token_stride, int64_t tiled_head_stride, int inverse,
                  int dtype, hipStream_t stream);

/*
 * bsa_tile_block_window -- bsa_gilbert_block_window for the tile layout:
 * the blocks holding any cell of the 3 x 3 x 3 neighbourhood of any cell of
 * query block b, which for tiles is exactly the 3 x 3 x 3 neighbourhood of
 * b's tile (time stepping back from the first tile layer into chunk
 * q_chunk - 1's last one, never forward into chunk q_chunk + 1).  block =
 * V; n_rows = n_tiles*V; window rows as for bsa_gilbert_block_window.
 * Errors: BSA_EINVAL (null pointers, n_rows not a multiple of block,
 * q_chunk < 0, window_stride < 2*n_tiles), BSA_EUNSUPPORTED (more than
 * 1024 tiles per chunk).
 */
int bsa_tile_block_window(const int32_t* row_cell, const int32_t* cell_row, int n_rows, int T, int H,
                          int W, int block, int q_chunk, int32_t* window, int32_t* window_len,
                          int window_stride, hipStream_t stream);

/*
 * Route materialisation arguments.  Set struct_size =
 * sizeof(bsa_materialize_args).
 * [Velox -- Methodology, Step 3 (a coverage score per query block: the
 *  share of its tokens inside a valid historical slab); Step 4 (the fusion
 *  applies to well-covered blocks); Step 5 (reservation, top-scoring fill
 *  up to K_cov, cumulative-mass prefix capped at K_unc, local window and
 *  reference blocks outside the budget); the calibrated eta_cov = 0.9,
 *  K_cov = 80, K_unc = 150 close the Methodology section]
 *
 *  coverage       device float32[nqb] (NULL: every query block is well
 *                 covered); shared by all heads.  Query block i is well
 *                 covered when coverage[i] >= eta_cov, compared in
 *                 float32 (eta_cov rounded to float32): for a coverage
 *                 that is a ratio of token counts this is the exact
 *                 decision (72 of 80 tokens is covered at eta_cov = 0.9).
 *  k_cov          budget of a well-covered row (reserved blocks count
 *                 towards it).
 *  k_unc          cap of a poorly covered row's prefix, 0 .. 256.
 *  mass           cumulative-mass threshold of a poorly covered row.
 *  prev_begin, prev_end  block range [begin, end) reserved by every
 *                 well-covered row (the previous chunk); clipped to nkb.
 *  window, window_len, window_stride  per-query-block window rows as
 *                 written by bsa_gilbert_block_window (NULL: none); row i
 *                 holds window_len[i] (clamped to [0, window_stride])
 *                 absolute block indices; indices outside [0, nkb) are
 *                 ignored.
 *  ref_begin, ref_end    reference-frame block range [begin, end); clipped
 *                 to nkb.
 */
typedef struct bsa_materialize_args {
    size_t struct_size;
    const float* coverage;
    double eta_cov;
    int k_cov;
    int k_unc;
    double mass;
    int prev_begin;
    int prev_end;
    const int32_t* window;
    const int32_t* window_len;
    int window_stride;
    int ref_begin;
    int ref_end;
} bsa_materialize_args;

/* Bytes of workspace bsa_route_materialize needs (0 if the arguments are
 * invalid). */
size_t bsa_route_materialize_workspace_size(const bsa_route_args* args,
                                            const bsa_materialize_args* margs);

/*
 * bsa_route_materialize -- the routed lists of every (head, query block)
 * row: pool and score as bsa_route_topk (the overlap bias only on
 * well-covered rows; every KV block is a candidate), then per row:
 *  - well covered: the visible blocks of [prev_begin, prev_end), all of
 *    them, plus the max(0, k_cov - reserved) others with the largest
 *    kappa (ties to the lower index);
 *  - poorly covered: with p = softmax(s) over the visible blocks and the
 *    visible blocks ordered by (s descending, index ascending), the
 *    shortest prefix whose running sum of p reaches mass, at most k_unc
 *    blocks (all k_unc, or all visible blocks, if none reaches it);
 *  - either: every visible block of its window row and of
 *    [ref_begin, ref_end).
 * Only blocks with a valid token enter a list; a query block with no valid
 * token gets an empty list.  Lists are ascending and duplicate-free and are
 * written packed: row r's list is col_idx[row_ptr[r] .. row_ptr[r+1]-1].
 * Of bsa_route_args, k_fixed and k_max are ignored; k_per_row and
 * fallback_counts must be NULL and n_dense_tail_blocks 0; kpool and
 * sel_keys work as for bsa_route_topk (sel_keys then hold s on poorly
 * covered rows).  The running sum is taken in float64 in list order, so a
 * sum that reaches mass within rounding can end the prefix one block apart
 * from another summation order.
 * workspace: as for bsa_route_topk, bsa_route_materialize_workspace_size
 * bytes.
 * Errors: BSA_EINVAL (arguments; col_capacity below heads*nqb*min(nkb,
 * max(prev range, k_cov, k_unc) + window_stride + ref range)),
 * BSA_EUNSUPPORTED (k_unc > 256, more than 4096 KV blocks, d or block),
 * BSA_EWORKSPACE.
 */
int bsa_route_materialize(const bsa_route_args* args, const bsa_materialize_args* margs,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Frustum-slab geometry.
 * [Velox -- Methodology, Step 1 (a historical block is kept as frustum
 *  slabs: a token rectangle in its source camera plus a depth interval);
 *  Step 3 (each slab as an oriented box facing its camera; the score is
 *  the largest IoU of the query's box with a historical box, measured on a
 *  fixed grid once a separating-axis test has not ruled the pair out;
 *  coverage = the share of a query block's tokens that lie in some valid
 *  historical slab, inside its rectangle and its depth range)]
 *
 * cams       device float64[n_cams][16]: fx, fy, cx, cy (token units), R
 *            row-major (world-from-camera; columns = the camera's right,
 *            down and forward axes in world space), C (camera centre).  A
 *            camera point (x, y, z), z > 0, sits at token coordinates
 *            u = fx x / z + cx (column), v = fy y / z + cy (row); token
 *            (h, w) covers [w, w+1) x [h, h+1).
 * slabs      grouped by block: block b's slabs are entries ptr[b] ..
 *            ptr[b+1]-1 (clamped to [0, n_slabs)) of cam (int32, index
 *            into cams; entries outside [0, n_cams) are skipped) and geom
 *            (float64[6]: u0, v0, u1, v1, z_lo, z_hi: the rectangle
 *            [u0, u1) x [v0, v1) and the camera-z interval [z_lo, z_hi]).
 *            Only valid slabs are passed.
 * The box of a slab: the camera's axes; centre on the ray through the
 * rectangle's centre at z_m = (z_lo + z_hi)/2; half extents (u1-u0) z_m /
 * (2 fx), (v1-v0) z_m / (2 fy), (z_hi-z_lo)/2.  All arithmetic is float64.
 */

/*
 * bsa_slab_overlap -- overlap[i * overlap_row_stride + j] (float32) = the
 * largest IoU over the pairs (query slab of block i, historical slab of
 * block j); 0 if either block has no slab.  A pair's IoU is 0 when a
 * separating axis exists (15 axes: the 6 face normals and the 9 edge cross
 * products, those of squared length < 1e-12 skipped; touching boxes are not
 * separated); otherwise, with cnt = the cell centres of the query box's
 * grid_n^3 grid that lie inside the historical box (closed), inter =
 * vol_q cnt / grid_n^3 and IoU = inter / (vol_q + vol_h - inter) (0 if the
 * union has no volume).  The result feeds bsa_route_topk /
 * bsa_route_materialize as their overlap input.
 * Errors: BSA_EINVAL (null pointers, counts, grid_n outside [1, 64],
 * overlap_row_stride < nkb), BSA_EUNSUPPORTED (nqb > 65535).
 */
int bsa_slab_overlap(const double* cams, int n_cams, const int32_t* q_slab_ptr,
                     const int32_t* q_slab_cam, const double* q_slab_geom, int nqb, int n_q_slabs,
                     const int32_t* h_slab_ptr, const int32_t* h_slab_cam,
                     const double* h_slab_geom, int nkb, int n_h_slabs, int grid_n, float* overlap,
                     int64_t overlap_row_stride, hipStream_t stream);

/*
 * bsa_slab_coverage -- coverage[i] (float32) of each of the ceil(T*H*W /
 * block) query blocks of a chunk: the share of its tokens whose point lies
 * inside some historical slab.  The tokens of block i are curve positions
 * i*block .. (i+1)*block-1 of perm (bsa_gilbert_index; entries outside
 * [0, T*H*W) are never covered); a token at raster cell (t, h, w) has its
 * point at token coordinates (w + 1/2, h + 1/2) and depth depth[cell]
 * (float32 raster [T][H][W]; NaN or <= 0: no depth, never covered) in
 * camera frame_cam[t] (int32[T]).  The point is inside a slab when, in the
 * slab's camera, z > 0, (u, v) lies in the rectangle and z in [z_lo, z_hi].
 * coverage = covered tokens / tokens of the block, the quotient taken in
 * float64 and rounded to float32.
 * workspace: device memory of bsa_slab_coverage_workspace_size(T, H, W)
 * bytes (one bit per token), 4-byte aligned, owned by the caller, cleared
 * by the call itself.
 * Errors: BSA_EINVAL (null pointers, dimensions, block < 1),
 * BSA_EUNSUPPORTED (more than 65535*128 slabs), BSA_EWORKSPACE.
 */
int bsa_slab_coverage(const double* cams, int n_cams, const int32_t* perm, int T, int H, int W,
                      int block, const int32_t* frame_cam, const float* depth,
                      const int32_t* h_slab_cam, const double* h_slab_geom, int n_h_slabs,
                      float* coverage, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace bsa_slab_coverage needs for a T x H x W chunk (0 if
 * the dimensions are invalid). */
size_t bsa_slab_coverage_workspace_size(int T, int H, int W);

/*
 * bsa_block_sparse_attn -- attention of every query block over its listed
 * KV blocks.
 * [Velox -- Methodology, Step 6: an indexed block-sparse kernel, not a dense
 *  call with a mask; a skipped block costs neither its QK^T tile nor its KV
 *  load; the block size is the attention tile] [Light Interaction --
 *  abstract: 3-D block-sparse attention]
 *
 *  q              [heads][nqb*block][d], head stride q_head_stride.
 *  k, v           [heads][nkb*block][d], head strides k/v_head_stride.
 *  o              [heads][nqb*block][d] output in dtype, head stride
 *                 o_head_stride.
 *  lse            float32[heads][nqb*block] (nullable): natural-log
 *                 log-sum-exp of the scaled scores per query row.
 *  q_block_len, kv_block_len  as for the router (NULL: all full).  K and
 *                 V rows past a block's valid length are never fetched
 *                 (bf16) or never weighted (fp32), and padded query rows
 *                 never reach another row's result, so padding may hold
 *                 anything, NaN included.
 *  row_ptr        int32[heads*nqb + 1], col_idx int32[col_len]: the lists
 *                 (row r = h*nqb + i).  Entries outside [0, nkb) and ranges
 *                 outside [0, col_len) are ignored.
 *  scale          score scale (normally 1/sqrt(d)).
 * For each head h and valid query row t of block i:
 *   O = sum_u softmax_u(scale * q_t . k_u) v_u over the valid keys u of the
 *   listed blocks (no causal mask).  Padded query rows are written as 0 (LSE
 *   -inf); an empty list gives O = 0, LSE = -inf.  bf16: QK^T and PV are bf16
 *   MFMA products with fp32 accumulation and an fp32 online softmax; P is
 *   rounded to bf16 before the PV product; O is rounded to bf16 once.
 * Errors: BSA_EINVAL, BSA_EUNSUPPORTED.
 */
int bsa_block_sparse_attn(const void* q, const void* k, const void* v, void* o, float* lse,
                          int dtype, int heads, int d, int block, int nqb, int nkb,
                          int64_t q_head_stride, int64_t k_head_stride, int64_t v_head_stride,
                          int64_t o_head_stride, const int32_t* q_block_len,
                          const int32_t* kv_block_len, const int32_t* row_ptr,
                          const int32_t* col_idx, int64_t col_len, float scale,
                          hipStream_t stream);

/*
 * bsa_block_sparse_attn_raster -- bsa_block_sparse_attn with the output
 * written straight into raster token order (the inverse permutation fused
 * into the kernel's epilogue) and, optionally, the queries read from raster
 * order too (the forward permutation of Q fused into its loads).
 * [Velox -- Methodology, Step 6; Key Contributions 3 (Gilbert KV storage,
 *  outputs returned in the caller's order)]
 *
 *  row_map        device int32[rows], rows <= nqb*block: query row g (of
 *                 every head) is raster token row_map[g]; a negative entry
 *                 marks a padding row, which is not written (and, for
 *                 raster queries, reads as zeros).  For blocks that are
 *                 runs of the curve this is the curve itself (perm of
 *                 bsa_gilbert_index, rows = T*H*W); for fixed tiles it is
 *                 the row map of bsa_gilbert_tile_index.  Entries must be
 *                 distinct and index tokens of o (and of q).  Rows >= rows
 *                 are padding.
 *  q_raster       0: q is blocked [heads][nqb*block][d] with head stride
 *                 q_stride (as bsa_block_sparse_attn); 1: q is raster,
 *                 element (token t, head h, channel c) at
 *                 q[t * q_stride + h * d + c], query row g reading token
 *                 row_map[g].
 *  o              raster output in dtype: element (token t, head h, channel
 *                 c) at o[t * o_token_stride + h * d + c]; tokens that no
 *                 row maps to are left untouched.
 * Every other argument, the lse layout (blocked, [heads][nqb*block]) and the
 * values written are those of bsa_block_sparse_attn (padding query rows
 * must also be padding in q_block_len).
 * Errors: those of bsa_block_sparse_attn; BSA_EINVAL (row_map NULL, rows
 * outside [1, nqb*block], q_raster not 0 or 1, o_token_stride or a raster
 * q_stride below heads*d or not a multiple of 16 bytes).
 */
int bsa_block_sparse_attn_raster(const void* q, const void* k, const void* v, void* o, float* lse,
                                 int dtype, int heads, int d, int block, int nqb, int nkb,
                                 int q_raster, int64_t q_stride, int64_t k_head_stride,
                                 int64_t v_head_stride, const int32_t* row_map, int rows,
                                 int64_t o_token_stride, const int32_t* q_block_len,
                                 const int32_t* kv_block_len, const int32_t* row_ptr,
                                 const int32_t* col_idx, int64_t col_len, float scale,
                                 hipStream_t stream);

/*
 * bsa_dense_attn -- the dense baseline: bsa_block_sparse_attn with every KV
 * block listed in ascending order, through the same kernel.
 * [Velox -- Main Findings: dense attention over all retained context]
 */
int bsa_dense_attn(const void* q, const void* k, const void* v, void* o, float* lse, int dtype,
                   int heads, int d, int block, int nqb, int nkb, int64_t q_head_stride,
                   int64_t k_head_stride, int64_t v_head_stride, int64_t o_head_stride,
                   const int32_t* q_block_len, const int32_t* kv_block_len, float scale,
                   hipStream_t stream);

/*
 * bsa_diag_mfma_bf16 -- diagnostic, not part of the method: `workgroups`
 * workgroups of 4 waves each issue 4 * iters v_mfma_f32_32x32x16_bf16
 * (32768 FLOP each) from registers, with no memory traffic, and write one
 * float per thread to sink (device float32[workgroups * 256]).  Timing it
 * gives the bf16 matrix rate the GPU delivers at its current clock, beside
 * which the attention kernel's rate is read.
 * Errors: BSA_EINVAL (workgroups outside [1, 2^20], iters < 1, NULL sink).
 */
int bsa_diag_mfma_bf16(int workgroups, int iters, float* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* BSA_H */
