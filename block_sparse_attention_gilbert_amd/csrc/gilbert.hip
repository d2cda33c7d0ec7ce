// Generalized-Hilbert ("Gilbert") order of a latent chunk and the
// raster <-> Gilbert permutation of token tensors.
//
// [Velox: Spatial Memory Makes World Models Efficient -- Key Contributions 3
//  (KV storage in a Gilbert order aligned across chunks); Methodology, Step 6
//  (nearby image regions stay adjacent along the order, so a block of
//  consecutive KV rows is also a spatial neighbourhood)]
// [Light Interaction -- abstract ("3D block sparse attention")]
//
// The pages name the curve but do not define it.  The definition used here:
// a cuboid is filled from corner p along a travel axis a (ending one cell
// short of p + a when parity allows), with two further axes b and c.
// Halving an axis rounds its half up to even when the half is odd and the
// axis is longer than 2.  Rules, in order:
//   |b| = |c| = 1          straight run along a
//   |c| = 1 (or |b| = 1)   the 2-D rule in the plane (a, b) (or (a, c))
//   |a| = 1                the 2-D rule on the (b, c) face along the longer
//   |b| = |c| = 2          |a| = 2: face a=0 by the 2-D rule along b, then
//                          face a=1 from its b-far corner along -b;
//                          otherwise split a at its even half
//   2|a| > 3 max(|b|,|c|)  split a at its even half, both parts along a
//   otherwise              U-turn in the plane of a and the longer L of b, c
//                          (b on ties), the remaining axis O carried whole:
//                          (p, L/2, a/2, O), (p + L/2, a, L - L/2, O),
//                          (p + a - unit(a) + L/2 - unit(L), -L/2, -(a - a/2), O)
// 2-D rule on (a, b): |b| = 1 run along a; |a| = 1 run along b; 2|a| > 3|b|
// split a; otherwise (p, b/2, a/2), (p + b/2, a, b - b/2),
// (p + a - unit(a) + b/2 - unit(b), -b/2, -(a - a/2)).
// Top level: travel axis = longest of (w, h, t), ties in that order, the
// next longest second, start (0, 0, 0).
//
// Each GPU thread finds the cell at one curve position by descending this
// subdivision: at every level it computes the children's cell counts and
// steps into the child that holds its position.
#include <hip/hip_runtime.h>

#include "exact_sum.h"
#include "gilbert_curve.h"
#include "kernels.h"

namespace bsa {
namespace {

using curve::V3;
using curve::gilbert_cell;

__global__ void gilbert_index_kernel(int T, int H, int W, int32_t* __restrict__ perm,
                                     int32_t* __restrict__ inv) {
    const int64_t n = (int64_t)T * H * W;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const V3 cell = gilbert_cell(T, H, W, i);
    const int32_t r = (int32_t)(((int64_t)cell.t * H + cell.h) * W + cell.w);
    perm[i] = r;
    if (inv) inv[r] = (int32_t)i;
}

// One thread moves one 16-byte chunk of one (row, head).  grid.y walks the
// rows (looping when there are more than the grid holds), grid.x the
// (head, chunk) pairs of a row, chunks fastest: raster reads cover a
// token's heads contiguously and Gilbert writes cover whole rows.  The
// chunk count per row is a power of two, so no division is needed.
template <bool INVERSE>
__global__ void __launch_bounds__(256)
gilbert_perm_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst, const int32_t* __restrict__ perm, int L,
                    int heads, int log2_chunks, int64_t rows_total, int64_t raster_token_stride_c,
                    int64_t gilbert_head_stride_c) {
    const int hc = blockIdx.x * 256 + threadIdx.x;
    const int chunks = 1 << log2_chunks;
    if (hc >= heads * chunks) return;
    const int ch = hc & (chunks - 1), h = hc >> log2_chunks;
    for (int64_t i = blockIdx.y; i < rows_total; i += gridDim.y) {
        const int64_t g = h * gilbert_head_stride_c + i * chunks + ch;
        if (!INVERSE) {
            if (i < L) {
                const int64_t r = (int64_t)perm[i] * raster_token_stride_c + (int64_t)h * chunks + ch;
                dst[g] = src[r];
            } else {
                dst[g] = make_uint4(0u, 0u, 0u, 0u);
            }
        } else if (i < L) {
            const int64_t r = (int64_t)perm[i] * raster_token_stride_c + (int64_t)h * chunks + ch;
            dst[r] = src[g];
        }
    }
}

// Forward permutation fused with the block means of the permuted rows (dst
// NULL: the block means only).
// One workgroup per (block, head): thread t copies 16-byte chunk t % chunks
// of the block's rows t / chunks, + groups, ... (raster token perm[i] to
// Gilbert row i; padding rows written as zeros) and sums what it copied,
// exactly (exact_sum.h).  The row groups of a wave are combined with
// shuffles, the four waves through LDS, and the mean over the block's valid
// rows (the exact sum rounded once, divided once) goes to pool: the same
// value whatever the summation order, for a column whose nonzero
// magnitudes span less than 2^39 (bf16) or 2^74 (float32).
// [Velox -- Methodology, Step 4: the router works on per-block averages of
//  the queries and keys; Step 6: nearby regions adjacent in the padded block
//  layout]
template <bool BF16, bool POOL>
__device__ __forceinline__ void perm_pool_block(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                const int32_t* __restrict__ perm, int L, int d, int block, int b,
                                                int h, int64_t raster_token_stride_c, int64_t gilbert_head_stride_c,
                                                double* __restrict__ pool, int64_t pool_head_stride) {
    constexpr int CE = BF16 ? 8 : 4;  // elements per 16-byte chunk
    __shared__ double part_hi[4][128], part_lo[4][128];
    const int t = threadIdx.x, w = t >> 6;
    const int chunks = d / CE, groups = 256 / chunks;
    const int ch = t % chunks, g = t / chunks;
    const int64_t i0 = (int64_t)b * block;
    const int valid = (int)(L - i0 < block ? L - i0 : block);
    const int64_t hc = (int64_t)h * chunks + ch;
    uint4* out = dst ? dst + h * gilbert_head_stride_c + i0 * chunks + ch : nullptr;
    Acc<BF16> acc[CE];
#pragma unroll 4
    for (int k = g; k < block; k += groups) {
        uint4 u = make_uint4(0u, 0u, 0u, 0u);
        if (k < valid) u = src[(int64_t)perm[i0 + k] * raster_token_stride_c + hc];
        if (out) out[(int64_t)k * chunks] = u;
        if (!POOL) continue;
        const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
        if (BF16) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[2 * e].add((double)__uint_as_float(wd[e] << 16));
                acc[2 * e + 1].add((double)__uint_as_float(wd[e] & 0xFFFF0000u));
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e].add((double)__uint_as_float(wd[e]));
        }
    }
    if (!POOL) return;
    for (int off = chunks; off < 64; off <<= 1)
#pragma unroll
        for (int e = 0; e < CE; ++e) acc[e].add(acc[e].shfl_xor(off));
    if ((t & 63) < chunks)
#pragma unroll
        for (int e = 0; e < CE; ++e) {
            part_hi[w][ch * CE + e] = acc[e].hi();
            part_lo[w][ch * CE + e] = acc[e].lo();
        }
    __syncthreads();
    if (t < d) {
        Acc<BF16> sum = Acc<BF16>::make(part_hi[0][t], part_lo[0][t]);
#pragma unroll
        for (int u = 1; u < 4; ++u) sum.add(Acc<BF16>::make(part_hi[u][t], part_lo[u][t]));
        pool[h * pool_head_stride + (int64_t)b * d + t] = sum.hi() / (double)valid;
    }
}

template <bool BF16>
__global__ void __launch_bounds__(256)
gilbert_perm_pool_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst, const int32_t* __restrict__ perm,
                         int L, int d, int block, int64_t raster_token_stride_c, int64_t gilbert_head_stride_c,
                         double* __restrict__ pool, int64_t pool_head_stride) {
    perm_pool_block<BF16, true>(src, dst, perm, L, d, block, blockIdx.x, blockIdx.y, raster_token_stride_c,
                                gilbert_head_stride_c, pool, pool_head_stride);
}

// Several tensors of one chunk (Q, K, V) permuted and/or pooled by one
// launch: grid.z picks the tensor, and each (block, head, tensor) workgroup
// does what the single-tensor kernel above does, the block means skipped
// where the tensor has no pool.  One launch instead of three keeps the copy
// engines busy across the tensors' tails.
constexpr int kMaxPermJobs = BSA_MAX_PERM_JOBS;

struct PermJobs {
    const uint4* src[kMaxPermJobs];
    uint4* dst[kMaxPermJobs];
    double* pool[kMaxPermJobs];
    int64_t rts_c[kMaxPermJobs], ghs_c[kMaxPermJobs], phs[kMaxPermJobs];
};

// job z of the kernel argument (a select chain: indexing a by-value array
// with a runtime index would copy it to scratch memory)
template <class T>
__device__ __forceinline__ T pick(const T (&v)[kMaxPermJobs], int z) {
    static_assert(kMaxPermJobs == 4, "select chain covers four jobs");
    return z == 0 ? v[0] : z == 1 ? v[1] : z == 2 ? v[2] : v[3];
}

template <bool BF16>
__global__ void __launch_bounds__(256)
gilbert_perm_pool_batch_kernel(PermJobs j, const int32_t* __restrict__ perm, int L, int d, int block) {
    const int z = blockIdx.z;
    double* const pool = pick(j.pool, z);
    if (pool)
        perm_pool_block<BF16, true>(pick(j.src, z), pick(j.dst, z), perm, L, d, block, blockIdx.x, blockIdx.y,
                                    pick(j.rts_c, z), pick(j.ghs_c, z), pool, pick(j.phs, z));
    else
        perm_pool_block<BF16, false>(pick(j.src, z), pick(j.dst, z), perm, L, d, block, blockIdx.x, blockIdx.y,
                                     pick(j.rts_c, z), pick(j.ghs_c, z), nullptr, 0);
}

}  // namespace

// Fixed 3-D tile layout: one thread per row of the tiled chunk.  Block b
// is the tile at position b of the Gilbert curve over the tile grid; its
// cells, in raster order inside the (clipped) tile, fill its first rows and
// the rest are padding (-1).
// [Light Interaction -- abstract: 3-D block-sparse attention; Velox -- Key
//  Contributions 3: global-aligned Gilbert KV storage]
__global__ void tile_index_kernel(int T, int H, int W, int tt, int th, int tw, int nT, int nH, int nW,
                                  int32_t* __restrict__ row_cell, int32_t* __restrict__ block_len,
                                  int32_t* __restrict__ cell_row) {
    const int V = tt * th * tw;
    const int64_t rows = (int64_t)nT * nH * nW * V;
    const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= rows) return;
    const int b = (int)(r / V), k = (int)(r % V);
    const V3 tile = gilbert_cell(nT, nH, nW, b);
    const int t0 = tile.t * tt, h0 = tile.h * th, w0 = tile.w * tw;
    const int vt = min(T, t0 + tt) - t0, vh = min(H, h0 + th) - h0, vw = min(W, w0 + tw) - w0;
    const int n = vt * vh * vw;
    if (k == 0) block_len[b] = n;
    if (k < n) {
        const int kt = k / (vh * vw), kh = (k / vw) % vh, kw = k % vw;
        const int cell = ((t0 + kt) * H + (h0 + kh)) * W + (w0 + kw);
        row_cell[r] = cell;
        if (cell_row) cell_row[cell] = (int32_t)r;
    } else {
        row_cell[r] = -1;
    }
}

// Permutation through a row map: row i of the tiled layout holds raster
// token row_cell[i]; rows with a negative entry are padding (written as
// zeros forward, skipped inverse).  Same thread walk as gilbert_perm_kernel.
template <bool INVERSE>
__global__ void __launch_bounds__(256)
tile_perm_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst, const int32_t* __restrict__ row_cell, int L,
                 int heads, int log2_chunks, int64_t rows_total, int64_t raster_token_stride_c,
                 int64_t tiled_head_stride_c) {
    const int hc = blockIdx.x * 256 + threadIdx.x;
    const int chunks = 1 << log2_chunks;
    if (hc >= heads * chunks) return;
    const int ch = hc & (chunks - 1), h = hc >> log2_chunks;
    for (int64_t i = blockIdx.y; i < rows_total; i += gridDim.y) {
        const int64_t g = h * tiled_head_stride_c + i * chunks + ch;
        const int cell = row_cell[i];
        const bool valid = cell >= 0 && cell < L;
        const int64_t r = (int64_t)(valid ? cell : 0) * raster_token_stride_c + (int64_t)h * chunks + ch;
        if (!INVERSE) {
            dst[g] = valid ? src[r] : make_uint4(0u, 0u, 0u, 0u);
        } else if (valid) {
            dst[r] = src[g];
        }
    }
}

// Local window of each query block: one workgroup per block b of the chunk;
// each thread takes tokens of b, walks the 27 cells of their 3 x 3 x 3
// neighbourhood (the cell itself included; time crosses into the previous
// chunk, never into the next) and sets the bit of the block holding each
// cell in an LDS bitmap over the previous and the current chunk's blocks.
// The bitmap is then written out in ascending block order.
// [Velox: Spatial Memory Makes World Models Efficient -- Methodology,
//  Step 5: every route also takes the block's 26 neighbours in the Gilbert
//  block order shared by all chunks]
constexpr int kWindowWords = 2 * kMaxWindowChunkBlocks / 32;  // bitmap words: 2 chunks

static_assert(kWindowWords == 64, "one wave compacts the window bitmap");

// Rows of block b are b*block .. (b+1)*block-1, bounded by row_end; the
// cell of row r is row_cell[r] (negative: a padding row) and the row of a
// cell is cell_row[cell].  For blocks that are runs of the curve, row_cell
// is the curve itself and row_end = T*H*W; for fixed tiles both come from
// the tile layout.
__global__ void __launch_bounds__(256)
block_window_kernel(const int32_t* __restrict__ row_cell, const int32_t* __restrict__ cell_row, int row_end, int T,
                    int H, int W, int block, int nbc, int q_chunk, int32_t* __restrict__ window,
                    int32_t* __restrict__ window_len, int stride) {
    __shared__ unsigned bits[kWindowWords];
    __shared__ int wsum[4];
    const int b = blockIdx.x, t = threadIdx.x;
    const int L = T * H * W;
    if (t < kWindowWords) bits[t] = 0u;
    __syncthreads();
    const int g1 = min(row_end, (b + 1) * block);
    for (int gp = b * block + t; gp < g1; gp += blockDim.x) {
        const int cell = row_cell[gp];
        if (cell < 0 || cell >= L) continue;
        const int tt0 = cell / (H * W), rem = cell % (H * W), h0 = rem / W, w0 = rem % W;
        for (int dt = -1; dt <= 1; ++dt) {
            int tt = tt0 + dt, slot = 1;  // slot 1: the query chunk, 0: the previous one
            if (tt < 0) {
                tt += T;
                slot = 0;
            } else if (tt >= T) {
                continue;
            }
            if (slot == 0 && q_chunk == 0) continue;
            for (int dh = -1; dh <= 1; ++dh) {
                const int hh = h0 + dh;
                if (hh < 0 || hh >= H) continue;
                for (int dw = -1; dw <= 1; ++dw) {
                    const int ww = w0 + dw;
                    if (ww < 0 || ww >= W) continue;
                    const int nb = cell_row[(tt * H + hh) * W + ww] / block;
                    const int bit = slot * nbc + nb;
                    atomicOr(&bits[bit >> 5], 1u << (bit & 31));
                }
            }
        }
    }
    __syncthreads();
    // ascending order: word w holds bits 32w .. 32w+31; threads 0..63 own a
    // word each, an exclusive scan of their counts gives the write offsets
    const int lane = t & 63, wv = t >> 6;
    const unsigned word = t < kWindowWords ? bits[t] : 0u;
    const int cnt = __popc(word);
    int incl = cnt;
    for (int off = 1; off < 64; off <<= 1) {
        const int up = __shfl_up(incl, off);
        if (lane >= off) incl += up;
    }
    if (wv == 0) {
        int pos = incl - cnt;
        unsigned x = word;
        int32_t* row = window + (int64_t)b * stride;
        while (x) {
            const int k = __ffs(x) - 1;
            x &= x - 1;
            const int bit = 32 * t + k;
            const int slot = bit >= nbc ? 1 : 0;
            row[pos++] = (q_chunk - 1 + slot) * nbc + (bit - slot * nbc);
        }
        if (lane == 63) wsum[0] = incl;
    }
    __syncthreads();
    if (t == 0) window_len[b] = wsum[0];
}

hipError_t launch_gilbert_index(int T, int H, int W, int32_t* perm, int32_t* inv, hipStream_t stream) {
    const int64_t n = (int64_t)T * H * W;
    const int threads = 256;
    const unsigned blocks = (unsigned)((n + threads - 1) / threads);
    hipLaunchKernelGGL(gilbert_index_kernel, dim3(blocks), dim3(threads), 0, stream, T, H, W, perm, inv);
    return hipGetLastError();
}

hipError_t launch_gilbert_perm(const void* src, void* dst, const int32_t* perm, int L, int heads, int d,
                               int block, int64_t raster_token_stride, int64_t gilbert_head_stride,
                               int inverse, int dtype, hipStream_t stream) {
    const int eb = dtype == BSA_BF16 ? 2 : 4;
    const int chunk_elems = 16 / eb;
    const int chunks_per_row = d / chunk_elems;
    const int log2c = __builtin_ctz((unsigned)chunks_per_row);
    const int64_t rows_total = inverse ? (int64_t)L : ((int64_t)L + block - 1) / block * block;
    const dim3 grid((unsigned)((heads * chunks_per_row + 255) / 256), (unsigned)(rows_total < 65535 ? rows_total : 65535));
    const int64_t rts_c = raster_token_stride / chunk_elems;
    const int64_t ghs_c = gilbert_head_stride / chunk_elems;
    if (inverse)
        hipLaunchKernelGGL(gilbert_perm_kernel<true>, grid, dim3(256), 0, stream, static_cast<const uint4*>(src),
                           static_cast<uint4*>(dst), perm, L, heads, log2c, rows_total, rts_c, ghs_c);
    else
        hipLaunchKernelGGL(gilbert_perm_kernel<false>, grid, dim3(256), 0, stream, static_cast<const uint4*>(src),
                           static_cast<uint4*>(dst), perm, L, heads, log2c, rows_total, rts_c, ghs_c);
    return hipGetLastError();
}

hipError_t launch_gilbert_perm_pool(const void* src, void* dst, const int32_t* perm, int L, int heads, int d,
                                    int block, int64_t raster_token_stride, int64_t gilbert_head_stride, int dtype,
                                    double* pool, int64_t pool_head_stride, hipStream_t stream) {
    const int chunk_elems = dtype == BSA_BF16 ? 8 : 4;
    const dim3 grid((unsigned)((L + block - 1) / block), (unsigned)heads);
    const int64_t rts_c = raster_token_stride / chunk_elems;
    const int64_t ghs_c = gilbert_head_stride / chunk_elems;
    if (dtype == BSA_BF16)
        hipLaunchKernelGGL(gilbert_perm_pool_kernel<true>, grid, dim3(256), 0, stream, static_cast<const uint4*>(src),
                           static_cast<uint4*>(dst), perm, L, d, block, rts_c, ghs_c, pool, pool_head_stride);
    else
        hipLaunchKernelGGL(gilbert_perm_pool_kernel<false>, grid, dim3(256), 0, stream, static_cast<const uint4*>(src),
                           static_cast<uint4*>(dst), perm, L, d, block, rts_c, ghs_c, pool, pool_head_stride);
    return hipGetLastError();
}

hipError_t launch_gilbert_perm_pool_batch(const bsa_perm_job* jobs, int n_jobs, const int32_t* perm, int L,
                                          int heads, int d, int block, int dtype, hipStream_t stream) {
    const int chunk_elems = dtype == BSA_BF16 ? 8 : 4;
    PermJobs j{};
    for (int z = 0; z < n_jobs; ++z) {
        j.src[z] = static_cast<const uint4*>(jobs[z].src);
        j.dst[z] = static_cast<uint4*>(jobs[z].dst);
        j.pool[z] = jobs[z].pool;
        j.rts_c[z] = jobs[z].raster_token_stride / chunk_elems;
        j.ghs_c[z] = jobs[z].gilbert_head_stride / chunk_elems;
        j.phs[z] = jobs[z].pool_head_stride;
    }
    const dim3 grid((unsigned)((L + block - 1) / block), (unsigned)heads, (unsigned)n_jobs);
    if (dtype == BSA_BF16)
        hipLaunchKernelGGL(gilbert_perm_pool_batch_kernel<true>, grid, dim3(256), 0, stream, j, perm, L, d, block);
    else
        hipLaunchKernelGGL(gilbert_perm_pool_batch_kernel<false>, grid, dim3(256), 0, stream, j, perm, L, d, block);
    return hipGetLastError();
}

hipError_t launch_block_window(const int32_t* perm, const int32_t* inv, int T, int H, int W, int block, int q_chunk,
                               int32_t* window, int32_t* window_len, int stride, hipStream_t stream) {
    const int L = T * H * W;
    const int nbc = (L + block - 1) / block;
    hipLaunchKernelGGL(block_window_kernel, dim3(nbc), dim3(256), 0, stream, perm, inv, L, T, H, W, block, nbc,
                       q_chunk, window, window_len, stride);
    return hipGetLastError();
}

hipError_t launch_tile_block_window(const int32_t* row_cell, const int32_t* cell_row, int n_rows, int T, int H, int W,
                                    int block, int q_chunk, int32_t* window, int32_t* window_len, int stride,
                                    hipStream_t stream) {
    const int nbc = n_rows / block;
    hipLaunchKernelGGL(block_window_kernel, dim3(nbc), dim3(256), 0, stream, row_cell, cell_row, n_rows, T, H, W, block,
                       nbc, q_chunk, window, window_len, stride);
    return hipGetLastError();
}

hipError_t launch_tile_index(int T, int H, int W, int tt, int th, int tw, int32_t* row_cell, int32_t* block_len,
                             int32_t* cell_row, hipStream_t stream) {
    const int nT = (T + tt - 1) / tt, nH = (H + th - 1) / th, nW = (W + tw - 1) / tw;
    const int64_t rows = (int64_t)nT * nH * nW * tt * th * tw;
    hipLaunchKernelGGL(tile_index_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, stream, T, H, W, tt, th,
                       tw, nT, nH, nW, row_cell, block_len, cell_row);
    return hipGetLastError();
}

hipError_t launch_tile_perm(const void* src, void* dst, const int32_t* row_cell, int n_rows, int L, int heads, int d,
                            int64_t raster_token_stride, int64_t tiled_head_stride, int inverse, int dtype,
                            hipStream_t stream) {
    const int eb = dtype == BSA_BF16 ? 2 : 4;
    const int chunk_elems = 16 / eb;
    const int chunks_per_row = d / chunk_elems;
    const int log2c = __builtin_ctz((unsigned)chunks_per_row);
    const dim3 grid((unsigned)((heads * chunks_per_row + 255) / 256), (unsigned)(n_rows < 65535 ? n_rows : 65535));
    const int64_t rts_c = raster_token_stride / chunk_elems;
    const int64_t ths_c = tiled_head_stride / chunk_elems;
    if (inverse)
        hipLaunchKernelGGL(tile_perm_kernel<true>, grid, dim3(256), 0, stream, static_cast<const uint4*>(src),
                           static_cast<uint4*>(dst), row_cell, L, heads, log2c, (int64_t)n_rows, rts_c, ths_c);
    else
        hipLaunchKernelGGL(tile_perm_kernel<false>, grid, dim3(256), 0, stream, static_cast<const uint4*>(src),
                           static_cast<uint4*>(dst), row_cell, L, heads, log2c, (int64_t)n_rows, rts_c, ths_c);
    return hipGetLastError();
}

}  // namespace bsa
