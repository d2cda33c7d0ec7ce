// Host-side argument validation and error reporting of the bsa C ABI.
//
// This file makes no HIP runtime call, so it builds with a plain host
// compiler and every error path can be exercised without a GPU.
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "common.h"

namespace bsa {

namespace {
thread_local char g_detail[512] = {0};

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool supported_dim(int x) { return x == 64 || x == 128; }

// No device buffer reaches 2^48 bytes (256 TiB); extents above it are
// rejected, which also keeps every kernel's int64 element offset in range.
constexpr int64_t kMaxBytes = int64_t(1) << 48;

// (n * stride + tail) elements of eb bytes, in bytes: false when an operand
// is negative or the result overflows or exceeds kMaxBytes.
bool extent(int64_t n, int64_t stride, int64_t tail, int eb, int64_t& bytes) {
    int64_t x;
    if (n < 0 || stride < 0 || tail < 0) return false;
    if (__builtin_mul_overflow(n, stride, &x) || __builtin_add_overflow(x, tail, &x) ||
        __builtin_mul_overflow(x, (int64_t)eb, &x) || x > kMaxBytes)
        return false;
    bytes = x;
    return true;
}

// T x H x W grid cells fit in 2^31-1 (overflow-checked product)
bool cells_fit(int T, int H, int W) {
    int64_t x;
    return !__builtin_mul_overflow((int64_t)T, (int64_t)H, &x) && !__builtin_mul_overflow(x, (int64_t)W, &x) &&
           x <= INT32_MAX;
}

// a stride of eb-byte elements keeps 16-byte alignment (eb is 2, 4 or 8)
bool stride16(int64_t stride, int eb) { return stride % (16 / eb) == 0; }

// [a, a + na) and [b, b + nb) share a byte (address arithmetic unsigned)
bool overlap(const void* a, int64_t na, const void* b, int64_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return na > 0 && nb > 0 && x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
}
}  // namespace

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_detail, sizeof(g_detail), fmt, ap);
    va_end(ap);
    return code;
}

void clear_error() { g_detail[0] = 0; }

const char* last_detail() { return g_detail; }

int validate_gilbert_index(int T, int H, int W, const int32_t* perm) {
    if (T < 1 || H < 1 || W < 1) return fail(BSA_EINVAL, "grid %d x %d x %d: dimensions must be >= 1", T, H, W);
    if (!cells_fit(T, H, W)) return fail(BSA_EINVAL, "grid %d x %d x %d exceeds 2^31-1 cells", T, H, W);
    if (!perm) return fail(BSA_EINVAL, "perm is NULL");
    return BSA_OK;
}

int validate_gilbert_perm(const void* src, const void* dst, const int32_t* perm, int L, int heads,
                          int d, int block, int64_t raster_token_stride,
                          int64_t gilbert_head_stride, int inverse, int dtype) {
    if (!src || !dst || !perm) return fail(BSA_EINVAL, "src, dst and perm must be non-NULL");
    if (dtype != BSA_BF16 && dtype != BSA_F32) return fail(BSA_EUNSUPPORTED, "dtype %d", dtype);
    if (!supported_dim(d)) return fail(BSA_EUNSUPPORTED, "d = %d (64 or 128)", d);
    if (!supported_dim(block)) return fail(BSA_EUNSUPPORTED, "block = %d (64 or 128)", block);
    if (L < 1 || heads < 1) return fail(BSA_EINVAL, "L = %d, heads = %d must be >= 1", L, heads);
    if (inverse != 0 && inverse != 1) return fail(BSA_EINVAL, "inverse = %d (0 or 1)", inverse);
    if (raster_token_stride < (int64_t)heads * d)
        return fail(BSA_EINVAL, "raster_token_stride %lld < heads*d = %lld", (long long)raster_token_stride,
                    (long long)heads * d);
    const int64_t rows = ceil_div(L, block) * block;
    if (gilbert_head_stride < rows * d)
        return fail(BSA_EINVAL, "gilbert_head_stride %lld < n_blocks*block*d = %lld",
                    (long long)gilbert_head_stride, (long long)(rows * d));
    const int eb = dtype_bytes(dtype);
    if (!aligned16(src) || !aligned16(dst) || !stride16(raster_token_stride, eb) || !stride16(gilbert_head_stride, eb))
        return fail(BSA_EINVAL, "pointers and strides must be 16-byte aligned");
    int64_t raster_bytes, gil_bytes;
    if (!extent(L - 1, raster_token_stride, (int64_t)heads * d, eb, raster_bytes) ||
        !extent(heads - 1, gilbert_head_stride, rows * d, eb, gil_bytes))
        return fail(BSA_EINVAL, "tensor extent exceeds 2^48 bytes");
    const int64_t sb = inverse ? gil_bytes : raster_bytes, tb = inverse ? raster_bytes : gil_bytes;
    if (overlap(src, sb, dst, tb)) return fail(BSA_EINVAL, "src and dst overlap");
    return BSA_OK;
}

int validate_gilbert_perm_pool(const void* src, const void* dst, const int32_t* perm, int L, int heads, int d,
                               int block, int64_t raster_token_stride, int64_t gilbert_head_stride, int dtype,
                               const double* pool, int64_t pool_head_stride) {
    if (dst) {
        const int st = validate_gilbert_perm(src, dst, perm, L, heads, d, block, raster_token_stride,
                                             gilbert_head_stride, 0, dtype);
        if (st != BSA_OK) return st;
    } else {  // block means only: the source side of the permutation's checks
        if (!src || !perm) return fail(BSA_EINVAL, "src and perm must be non-NULL");
        if (dtype != BSA_BF16 && dtype != BSA_F32) return fail(BSA_EUNSUPPORTED, "dtype %d", dtype);
        if (!supported_dim(d)) return fail(BSA_EUNSUPPORTED, "d = %d (64 or 128)", d);
        if (!supported_dim(block)) return fail(BSA_EUNSUPPORTED, "block = %d (64 or 128)", block);
        if (L < 1 || heads < 1) return fail(BSA_EINVAL, "L = %d, heads = %d must be >= 1", L, heads);
        if (raster_token_stride < (int64_t)heads * d)
            return fail(BSA_EINVAL, "raster_token_stride %lld < heads*d = %lld", (long long)raster_token_stride,
                        (long long)heads * d);
        if (!aligned16(src) || !stride16(raster_token_stride, dtype_bytes(dtype)))
            return fail(BSA_EINVAL, "src and its token stride must be 16-byte aligned");
    }
    if (!pool) return fail(BSA_EINVAL, "pool must be non-NULL");
    if (heads > 65535) return fail(BSA_EINVAL, "heads = %d exceeds 65535", heads);
    if (reinterpret_cast<uintptr_t>(pool) & 7u) return fail(BSA_EINVAL, "pool must be 8-byte aligned");
    const int64_t nb = ceil_div(L, block);
    if (pool_head_stride < nb * d)
        return fail(BSA_EINVAL, "pool_head_stride %lld < n_blocks*d = %lld", (long long)pool_head_stride,
                    (long long)(nb * d));
    const int eb = dtype_bytes(dtype);
    int64_t pool_bytes, raster_bytes, gil_bytes = 0;
    if (!extent(heads - 1, pool_head_stride, nb * d, (int)sizeof(double), pool_bytes) ||
        !extent(L - 1, raster_token_stride, (int64_t)heads * d, eb, raster_bytes) ||
        (dst && !extent(heads - 1, gilbert_head_stride, nb * block * d, eb, gil_bytes)))
        return fail(BSA_EINVAL, "tensor extent exceeds 2^48 bytes");
    if (overlap(pool, pool_bytes, src, raster_bytes) || overlap(pool, pool_bytes, dst, gil_bytes))
        return fail(BSA_EINVAL, "pool overlaps src or dst");
    return BSA_OK;
}

int validate_gilbert_perm_pool_batch(const bsa_perm_job* jobs, int n_jobs, const int32_t* perm, int L, int heads,
                                     int d, int block, int dtype) {
    if (!jobs) return fail(BSA_EINVAL, "jobs must be non-NULL");
    if (n_jobs < 1 || n_jobs > BSA_MAX_PERM_JOBS)
        return fail(BSA_EINVAL, "n_jobs = %d outside [1, %d]", n_jobs, BSA_MAX_PERM_JOBS);
    if (heads > 65535) return fail(BSA_EINVAL, "heads = %d exceeds 65535", heads);
    struct Range {
        const char* p;
        int64_t n;
    };
    Range src[BSA_MAX_PERM_JOBS], out[BSA_MAX_PERM_JOBS][2];
    const int eb = dtype_bytes(dtype);
    for (int z = 0; z < n_jobs; ++z) {
        const bsa_perm_job& j = jobs[z];
        if (!j.dst && !j.pool) return fail(BSA_EINVAL, "job %d has neither dst nor pool", z);
        const int st = j.pool ? validate_gilbert_perm_pool(j.src, j.dst, perm, L, heads, d, block,
                                                           j.raster_token_stride, j.gilbert_head_stride, dtype,
                                                           j.pool, j.pool_head_stride)
                              : validate_gilbert_perm(j.src, j.dst, perm, L, heads, d, block, j.raster_token_stride,
                                                      j.gilbert_head_stride, 0, dtype);
        if (st != BSA_OK) {
            char why[sizeof(g_detail)];
            snprintf(why, sizeof(why), "%s", g_detail);
            return fail(st, "job %d: %s", z, why);
        }
        // every extent below was checked by the job's own validation
        const int64_t nb = ceil_div(L, block);
        src[z] = {static_cast<const char*>(j.src), ((int64_t)(L - 1) * j.raster_token_stride + (int64_t)heads * d) * eb};
        out[z][0] = {static_cast<const char*>(j.dst),
                     j.dst ? ((int64_t)(heads - 1) * j.gilbert_head_stride + nb * block * d) * eb : 0};
        out[z][1] = {reinterpret_cast<const char*>(j.pool),
                     j.pool ? ((int64_t)(heads - 1) * j.pool_head_stride + nb * d) * (int64_t)sizeof(double) : 0};
    }
    auto hit = [](const Range& a, const Range& b) { return overlap(a.p, a.n, b.p, b.n); };
    for (int z = 0; z < n_jobs; ++z)
        for (int y = 0; y < n_jobs; ++y) {
            if (y == z) continue;
            for (int o = 0; o < 2; ++o)
                if (hit(out[z][o], src[y]) || hit(out[z][o], out[y][0]) || hit(out[z][o], out[y][1]))
                    return fail(BSA_EINVAL, "job %d's %s overlaps job %d's buffers", z, o ? "pool" : "dst", y);
        }
    return BSA_OK;
}

int validate_raster_out(const AttnProblem& p) {
    if (!p.o_map) return fail(BSA_EINVAL, "row_map must be non-NULL");
    if (p.o_map_len < 1 || (int64_t)p.o_map_len > (int64_t)p.nqb * p.block)
        return fail(BSA_EINVAL, "rows %d outside [1, nqb*block]", p.o_map_len);
    if (p.o_ts < (int64_t)p.heads * p.d)
        return fail(BSA_EINVAL, "o_token_stride %lld < heads*d = %lld", (long long)p.o_ts,
                    (long long)p.heads * p.d);
    const int eb = dtype_bytes(p.dtype);
    int64_t bytes;
    if (!stride16(p.o_ts, eb)) return fail(BSA_EINVAL, "o_token_stride must be 16-byte aligned");
    if (!extent(p.o_map_len - 1, p.o_ts, (int64_t)p.heads * p.d, eb, bytes))
        return fail(BSA_EINVAL, "raster output extent exceeds 2^48 bytes");
    if (p.q_map) {
        if (p.q_ts < (int64_t)p.heads * p.d)
            return fail(BSA_EINVAL, "raster q_stride %lld < heads*d = %lld", (long long)p.q_ts,
                        (long long)p.heads * p.d);
        if (!stride16(p.q_ts, eb)) return fail(BSA_EINVAL, "raster q_stride must be 16-byte aligned");
        if (!extent(p.q_map_len > 0 ? p.q_map_len - 1 : 0, p.q_ts, (int64_t)p.heads * p.d, eb, bytes))
            return fail(BSA_EINVAL, "raster query extent exceeds 2^48 bytes");
    }
    return BSA_OK;
}

int validate_attn(const AttnProblem& p, bool dense) {
    if (!p.q || !p.k || !p.v || !p.o) return fail(BSA_EINVAL, "q, k, v and o must be non-NULL");
    if (!dense && (!p.row_ptr || !p.col_idx)) return fail(BSA_EINVAL, "row_ptr and col_idx must be non-NULL");
    if (p.dtype != BSA_BF16 && p.dtype != BSA_F32) return fail(BSA_EUNSUPPORTED, "dtype %d", p.dtype);
    if (!supported_dim(p.d)) return fail(BSA_EUNSUPPORTED, "d = %d (64 or 128)", p.d);
    if (!supported_dim(p.block)) return fail(BSA_EUNSUPPORTED, "block = %d (64 or 128)", p.block);
    if (p.heads < 1 || p.nqb < 1 || p.nkb < 1)
        return fail(BSA_EINVAL, "heads %d, nqb %d, nkb %d must be >= 1", p.heads, p.nqb, p.nkb);
    if ((int64_t)p.heads * p.nqb > INT32_MAX / 2) return fail(BSA_EINVAL, "heads*nqb too large");
    if (!dense && p.col_len < 0) return fail(BSA_EINVAL, "col_len %lld < 0", (long long)p.col_len);
    const int64_t qrows = (int64_t)p.nqb * p.block, krows = (int64_t)p.nkb * p.block;
    if (p.q_hs < qrows * p.d || p.o_hs < qrows * p.d)
        return fail(BSA_EINVAL, "q/o head stride below nqb*block*d = %lld", (long long)(qrows * p.d));
    if (p.k_hs < krows * p.d || p.v_hs < krows * p.d)
        return fail(BSA_EINVAL, "k/v head stride below nkb*block*d = %lld", (long long)(krows * p.d));
    const int eb = dtype_bytes(p.dtype);
    if (!aligned16(p.q) || !aligned16(p.k) || !aligned16(p.v) || !aligned16(p.o) || !stride16(p.q_hs, eb) ||
        !stride16(p.k_hs, eb) || !stride16(p.v_hs, eb) || !stride16(p.o_hs, eb))
        return fail(BSA_EINVAL, "tensor pointers and head strides must be 16-byte aligned");
    int64_t bytes;
    if (!extent(p.heads - 1, p.q_hs, qrows * p.d, eb, bytes) || !extent(p.heads - 1, p.o_hs, qrows * p.d, eb, bytes) ||
        !extent(p.heads - 1, p.k_hs, krows * p.d, eb, bytes) || !extent(p.heads - 1, p.v_hs, krows * p.d, eb, bytes))
        return fail(BSA_EINVAL, "tensor extent exceeds 2^48 bytes");
    if (!(p.scale > 0.0f) || p.scale > 3.0e38f) return fail(BSA_EINVAL, "scale must be finite and > 0");
    return BSA_OK;
}

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

size_t route_layout(const bsa_route_args* a, RouteLayout* lay) {
    const int n_cand = a->nkb - a->n_dense_tail_blocks;
    size_t off = 0;
    lay->n_cand = n_cand;
    lay->qbar = off;
    off = align256(off + sizeof(double) * (size_t)a->heads * a->nqb * a->d);
    lay->kbar_in_ws = a->kpool == nullptr;
    lay->kbar = off;
    if (lay->kbar_in_ws) off = align256(off + sizeof(double) * (size_t)a->heads * n_cand * a->d);
    lay->keys_in_ws = a->sel_keys == nullptr;
    lay->keys = off;
    if (lay->keys_in_ws) off = align256(off + sizeof(double) * (size_t)a->heads * a->nqb * n_cand);
    lay->keff = off;
    off = align256(off + sizeof(int32_t) * ((size_t)a->heads * a->nqb + 8));
    lay->flags = off;
    off = align256(off + sizeof(int32_t) * ((size_t)a->nqb + 8));
    lay->bitmap = lay->counts = off;
    // two-level selection: the segments' top-K pairs
    lay->n_seg = n_cand > kSegCandidates ? (int)ceil_div(n_cand, kSegCandidates) : 1;
    int kcap = a->k_per_row ? a->k_max : a->k_fixed;
    kcap = kcap < 0 ? 0 : (kcap > kSegCandidates ? kSegCandidates : kcap);
    lay->seg_cap = lay->n_seg > 1 ? kcap : 0;
    lay->seg_key = lay->seg_idx = lay->seg_cnt = off;
    if (lay->n_seg > 1) {
        const size_t pairs = (size_t)a->heads * a->nqb * lay->n_seg * (size_t)lay->seg_cap;
        lay->seg_key = off;
        off = align256(off + sizeof(unsigned long long) * pairs);
        lay->seg_idx = off;
        off = align256(off + sizeof(int32_t) * pairs);
        lay->seg_cnt = off;
        off = align256(off + sizeof(int32_t) * (size_t)a->heads * a->nqb * lay->n_seg);
    }
    lay->total = off;
    return off;
}

int validate_route(const bsa_route_args* a, RouteLayout* lay) {
    if (!a) return fail(BSA_EINVAL, "args is NULL");
    if (a->struct_size != sizeof(bsa_route_args))
        return fail(BSA_EINVAL, "struct_size %zu != sizeof(bsa_route_args) %zu", a->struct_size,
                    sizeof(bsa_route_args));
    if ((!a->q && !a->qpool) || !a->k) return fail(BSA_EINVAL, "k and one of q, qpool must be non-NULL");
    if (!a->row_ptr || !a->col_idx) return fail(BSA_EINVAL, "row_ptr and col_idx must be non-NULL");
    if (a->dtype != BSA_BF16 && a->dtype != BSA_F32) return fail(BSA_EUNSUPPORTED, "dtype %d", a->dtype);
    if (!supported_dim(a->d)) return fail(BSA_EUNSUPPORTED, "d = %d (64 or 128)", a->d);
    if (!supported_dim(a->block)) return fail(BSA_EUNSUPPORTED, "block = %d (64 or 128)", a->block);
    if (a->heads < 1 || a->nqb < 1 || a->nkb < 1)
        return fail(BSA_EINVAL, "heads %d, nqb %d, nkb %d must be >= 1", a->heads, a->nqb, a->nkb);
    if (a->n_dense_tail_blocks < 0 || a->n_dense_tail_blocks > a->nkb)
        return fail(BSA_EINVAL, "n_dense_tail_blocks %d outside [0, nkb]", a->n_dense_tail_blocks);
    const int n_cand = a->nkb - a->n_dense_tail_blocks;
    if (n_cand > kMaxCandidates)
        return fail(BSA_EUNSUPPORTED, "%d candidate blocks exceed the selection limit %d", n_cand, kMaxCandidates);
    if ((int64_t)a->heads * a->nqb > (1 << 24)) return fail(BSA_EINVAL, "heads*nqb too large");
    const int64_t qrows = (int64_t)a->nqb * a->block, krows = (int64_t)a->nkb * a->block;
    if (a->q && a->q_head_stride < qrows * a->d) return fail(BSA_EINVAL, "q_head_stride below nqb*block*d");
    if (a->k_head_stride < krows * a->d) return fail(BSA_EINVAL, "k_head_stride below nkb*block*d");
    const int eb = dtype_bytes(a->dtype);
    if (!aligned16(a->q) || !aligned16(a->k) || !stride16(a->q_head_stride, eb) || !stride16(a->k_head_stride, eb))
        return fail(BSA_EINVAL, "q/k pointers and head strides must be 16-byte aligned");
    int64_t bytes;
    if ((a->q && !extent(a->heads - 1, a->q_head_stride, qrows * a->d, eb, bytes)) ||
        !extent(a->heads - 1, a->k_head_stride, krows * a->d, eb, bytes))
        return fail(BSA_EINVAL, "q/k extent exceeds 2^48 bytes");
    if (a->qpool) {
        if (!aligned16(a->qpool) || a->qpool_head_stride % 2)
            return fail(BSA_EINVAL, "qpool and its head stride must be 16-byte aligned");
        if (a->qpool_head_stride < (int64_t)a->nqb * a->d) return fail(BSA_EINVAL, "qpool_head_stride below nqb*d");
        if (!extent(a->heads - 1, a->qpool_head_stride, (int64_t)a->nqb * a->d, 8, bytes))
            return fail(BSA_EINVAL, "qpool extent exceeds 2^48 bytes");
    }
    if (!(a->scale > 0.0) || a->scale > 1.0e300) return fail(BSA_EINVAL, "scale must be finite and > 0");
    if (a->overlap) {
        if (a->overlap_row_stride < n_cand) return fail(BSA_EINVAL, "overlap_row_stride below the candidate count");
        if (!(a->g_ref > 0.0)) return fail(BSA_EINVAL, "g_ref must be > 0");
        if (!(a->lambda >= 0.0)) return fail(BSA_EINVAL, "lambda must be >= 0");
        if (!(a->tau == a->tau)) return fail(BSA_EINVAL, "tau is NaN");
    }
    int kcap;
    if (a->k_per_row) {
        if (a->k_max < 0) return fail(BSA_EINVAL, "k_max %d < 0", a->k_max);
        kcap = a->k_max;
    } else {
        if (a->k_fixed < 0) return fail(BSA_EINVAL, "k_fixed %d < 0", a->k_fixed);
        kcap = a->k_fixed;
    }
    if (kcap > n_cand) kcap = n_cand;
    if (a->kpool && (a->kpool_valid_blocks < 0 || a->kpool_valid_blocks > n_cand))
        return fail(BSA_EINVAL, "kpool_valid_blocks %d outside [0, %d]", a->kpool_valid_blocks, n_cand);
    if (a->kpool && a->kpool_head_blocks != 0 && a->kpool_head_blocks < n_cand)
        return fail(BSA_EINVAL, "kpool_head_blocks %d below the candidate count %d", a->kpool_head_blocks, n_cand);
    if (n_cand > kSegCandidates && ceil_div(n_cand, kSegCandidates) * (int64_t)kcap > kSegCandidates)
        return fail(BSA_EUNSUPPORTED,
                    "%d candidates in %lld segments with a budget cap of %d: segments x cap must be <= %d", n_cand,
                    (long long)ceil_div(n_cand, kSegCandidates), kcap, kSegCandidates);
    const int64_t need = (int64_t)a->heads * a->nqb * ((int64_t)kcap + a->n_dense_tail_blocks);
    if (a->col_capacity < need)
        return fail(BSA_EINVAL, "col_capacity %lld < heads*nqb*(k cap + dense tail) = %lld",
                    (long long)a->col_capacity, (long long)need);
    route_layout(a, lay);
    return BSA_OK;
}

int validate_materialize(const bsa_route_args* a, const bsa_materialize_args* m, RouteLayout* lay) {
    if (!a) return fail(BSA_EINVAL, "args is NULL");
    if (!m) return fail(BSA_EINVAL, "materialize args is NULL");
    if (m->struct_size != sizeof(bsa_materialize_args))
        return fail(BSA_EINVAL, "struct_size %zu != sizeof(bsa_materialize_args) %zu", m->struct_size,
                    sizeof(bsa_materialize_args));
    if (a->struct_size == sizeof(bsa_route_args)) {
        if (a->k_per_row) return fail(BSA_EINVAL, "k_per_row must be NULL: the budgets are k_cov and k_unc");
        if (a->n_dense_tail_blocks != 0)
            return fail(BSA_EINVAL, "n_dense_tail_blocks must be 0: every KV block is a candidate");
        if (a->fallback_counts) return fail(BSA_EINVAL, "fallback_counts must be NULL (not produced)");
    }
    if (a->nkb > kMaxMaterializeBlocks)
        return fail(BSA_EUNSUPPORTED, "%d KV blocks exceed the materialisation limit %d", a->nkb,
                    kMaxMaterializeBlocks);
    // the router's own checks, with the top-K budget out of the way
    bsa_route_args base = *a;
    base.k_fixed = 0;
    base.k_max = 0;
    const int st = validate_route(&base, lay);
    if (st != BSA_OK) return st;
    if (m->k_cov < 0) return fail(BSA_EINVAL, "k_cov %d < 0", m->k_cov);
    if (m->k_unc < 0 || m->k_unc > kMaxUncovered)
        return fail(m->k_unc < 0 ? BSA_EINVAL : BSA_EUNSUPPORTED, "k_unc %d outside [0, %d]", m->k_unc,
                    kMaxUncovered);
    if (!(m->eta_cov == m->eta_cov)) return fail(BSA_EINVAL, "eta_cov is NaN");
    if (!(m->mass == m->mass)) return fail(BSA_EINVAL, "mass is NaN");
    if (m->prev_begin < 0 || m->prev_end < m->prev_begin)
        return fail(BSA_EINVAL, "previous-chunk range [%d, %d) invalid", m->prev_begin, m->prev_end);
    if (m->ref_begin < 0 || m->ref_end < m->ref_begin)
        return fail(BSA_EINVAL, "reference range [%d, %d) invalid", m->ref_begin, m->ref_end);
    if (m->window && (!m->window_len || m->window_stride < 0))
        return fail(BSA_EINVAL, "window needs window_len and window_stride >= 0");
    const int nkb = a->nkb;
    auto clip = [nkb](int x) { return x < nkb ? x : nkb; };
    const int64_t n_prev = clip(m->prev_end) - clip(m->prev_begin);
    const int64_t n_ref = clip(m->ref_end) - clip(m->ref_begin);
    int64_t per_row = n_prev;
    if (m->k_cov > per_row) per_row = m->k_cov;
    if (m->k_unc > per_row) per_row = m->k_unc;
    per_row += (m->window ? m->window_stride : 0) + n_ref;
    if (per_row > nkb) per_row = nkb;
    const int64_t need = (int64_t)a->heads * a->nqb * per_row;
    if (a->col_capacity < need)
        return fail(BSA_EINVAL,
                    "col_capacity %lld < heads*nqb*min(nkb, max(prev, k_cov, k_unc) + window_stride + ref) = %lld",
                    (long long)a->col_capacity, (long long)need);
    size_t off = lay->total;
    lay->bitmap = off;
    off = align256(off + sizeof(uint32_t) * (size_t)a->heads * a->nqb * ceil_div(nkb, 32));
    lay->counts = off;
    off = align256(off + sizeof(int32_t) * ((size_t)a->heads * a->nqb + 8));
    lay->total = off;
    return BSA_OK;
}

int validate_block_window(const int32_t* perm, const int32_t* inv, int T, int H, int W, int block, int q_chunk,
                          const int32_t* window, const int32_t* window_len, int window_stride) {
    if (T < 1 || H < 1 || W < 1) return fail(BSA_EINVAL, "grid %d x %d x %d: dimensions must be >= 1", T, H, W);
    if (!cells_fit(T, H, W)) return fail(BSA_EINVAL, "grid %d x %d x %d exceeds 2^31-1 cells", T, H, W);
    const int64_t L = (int64_t)T * H * W;
    if (!perm || !inv || !window || !window_len)
        return fail(BSA_EINVAL, "perm, inv, window and window_len must be non-NULL");
    if (block < 1) return fail(BSA_EINVAL, "block %d < 1", block);
    if (q_chunk < 0) return fail(BSA_EINVAL, "q_chunk %d < 0", q_chunk);
    const int64_t nbc = ceil_div(L, block);
    if (nbc > kMaxWindowChunkBlocks)
        return fail(BSA_EUNSUPPORTED, "%lld blocks per chunk exceed %d", (long long)nbc, kMaxWindowChunkBlocks);
    if (window_stride < 2 * nbc)
        return fail(BSA_EINVAL, "window_stride %d < 2 * blocks per chunk (%lld)", window_stride, (long long)(2 * nbc));
    if (((int64_t)q_chunk + 1) * nbc > INT32_MAX) return fail(BSA_EINVAL, "block indices exceed 2^31-1");
    return BSA_OK;
}

int validate_tile_index(int T, int H, int W, int tt, int th, int tw, const int32_t* row_cell, const int32_t* block_len) {
    if (T < 1 || H < 1 || W < 1) return fail(BSA_EINVAL, "grid %d x %d x %d: dimensions must be >= 1", T, H, W);
    if (tt < 1 || th < 1 || tw < 1) return fail(BSA_EINVAL, "tile %d x %d x %d: dimensions must be >= 1", tt, th, tw);
    if (!row_cell || !block_len) return fail(BSA_EINVAL, "row_cell and block_len must be non-NULL");
    if (!cells_fit(T, H, W)) return fail(BSA_EINVAL, "grid cells exceed 2^31-1");
    // padded rows = (tiles along each axis) x (cells per tile), overflow-checked
    const int64_t f[6] = {ceil_div(T, tt), ceil_div(H, th), ceil_div(W, tw), tt, th, tw};
    int64_t rows = 1;
    for (int64_t x : f)
        if (__builtin_mul_overflow(rows, x, &rows) || rows > INT32_MAX)
            return fail(BSA_EINVAL, "tiled rows exceed 2^31-1");
    return BSA_OK;
}

int validate_tile_perm(const void* src, const void* dst, const int32_t* row_cell, int n_rows, int L, int heads, int d,
                       int64_t raster_token_stride, int64_t tiled_head_stride, int inverse, int dtype) {
    if (!src || !dst || !row_cell) return fail(BSA_EINVAL, "src, dst and row_cell must be non-NULL");
    if (dtype != BSA_BF16 && dtype != BSA_F32) return fail(BSA_EUNSUPPORTED, "dtype %d", dtype);
    if (!supported_dim(d)) return fail(BSA_EUNSUPPORTED, "d = %d (64 or 128)", d);
    if (n_rows < 1 || L < 1 || heads < 1)
        return fail(BSA_EINVAL, "n_rows = %d, L = %d, heads = %d must be >= 1", n_rows, L, heads);
    if (inverse != 0 && inverse != 1) return fail(BSA_EINVAL, "inverse = %d (0 or 1)", inverse);
    if (raster_token_stride < (int64_t)heads * d)
        return fail(BSA_EINVAL, "raster_token_stride %lld < heads*d = %lld", (long long)raster_token_stride,
                    (long long)heads * d);
    if (tiled_head_stride < (int64_t)n_rows * d)
        return fail(BSA_EINVAL, "tiled_head_stride %lld < n_rows*d = %lld", (long long)tiled_head_stride,
                    (long long)n_rows * d);
    const int eb = dtype_bytes(dtype);
    if (!aligned16(src) || !aligned16(dst) || !stride16(raster_token_stride, eb) || !stride16(tiled_head_stride, eb))
        return fail(BSA_EINVAL, "pointers and strides must be 16-byte aligned");
    int64_t raster_bytes, tiled_bytes;
    if (!extent(L - 1, raster_token_stride, (int64_t)heads * d, eb, raster_bytes) ||
        !extent(heads - 1, tiled_head_stride, (int64_t)n_rows * d, eb, tiled_bytes))
        return fail(BSA_EINVAL, "tensor extent exceeds 2^48 bytes");
    const int64_t sb = inverse ? tiled_bytes : raster_bytes, tb = inverse ? raster_bytes : tiled_bytes;
    if (overlap(src, sb, dst, tb)) return fail(BSA_EINVAL, "src and dst overlap");
    return BSA_OK;
}

int validate_tile_block_window(const int32_t* row_cell, const int32_t* cell_row, int n_rows, int T, int H, int W,
                               int block, int q_chunk, const int32_t* window, const int32_t* window_len,
                               int window_stride) {
    if (T < 1 || H < 1 || W < 1) return fail(BSA_EINVAL, "grid %d x %d x %d: dimensions must be >= 1", T, H, W);
    if (!cells_fit(T, H, W)) return fail(BSA_EINVAL, "grid exceeds 2^31-1 cells");
    if (!row_cell || !cell_row || !window || !window_len)
        return fail(BSA_EINVAL, "row_cell, cell_row, window and window_len must be non-NULL");
    if (block < 1 || n_rows < 1 || n_rows % block)
        return fail(BSA_EINVAL, "n_rows %d must be a positive multiple of block %d", n_rows, block);
    if (q_chunk < 0) return fail(BSA_EINVAL, "q_chunk %d < 0", q_chunk);
    const int nbc = n_rows / block;
    if (nbc > kMaxWindowChunkBlocks)
        return fail(BSA_EUNSUPPORTED, "%d blocks per chunk exceed %d", nbc, kMaxWindowChunkBlocks);
    if (window_stride < 2 * nbc)
        return fail(BSA_EINVAL, "window_stride %d < 2 * blocks per chunk (%d)", window_stride, 2 * nbc);
    if (((int64_t)q_chunk + 1) * nbc > INT32_MAX) return fail(BSA_EINVAL, "block indices exceed 2^31-1");
    return BSA_OK;
}

int validate_slab_overlap(const double* cams, int n_cams, const int32_t* q_ptr, const int32_t* q_cam,
                          const double* q_geom, int nqb, int n_q, const int32_t* h_ptr, const int32_t* h_cam,
                          const double* h_geom, int nkb, int n_h, int grid_n, const float* overlap, int64_t stride) {
    if (!cams || n_cams < 1) return fail(BSA_EINVAL, "cams must be non-NULL with n_cams >= 1");
    if (nqb < 1 || nkb < 1) return fail(BSA_EINVAL, "nqb %d and nkb %d must be >= 1", nqb, nkb);
    if (nqb > 65535) return fail(BSA_EUNSUPPORTED, "nqb %d > 65535", nqb);
    if (!q_ptr || !h_ptr || !overlap) return fail(BSA_EINVAL, "q_slab_ptr, h_slab_ptr and overlap must be non-NULL");
    if (n_q < 0 || n_h < 0) return fail(BSA_EINVAL, "slab counts must be >= 0");
    if ((n_q > 0 && (!q_cam || !q_geom)) || (n_h > 0 && (!h_cam || !h_geom)))
        return fail(BSA_EINVAL, "slab cameras and geometry must be non-NULL when slabs are given");
    if (grid_n < 1 || grid_n > 64) return fail(BSA_EINVAL, "grid_n %d outside [1, 64]", grid_n);
    if (stride < nkb) return fail(BSA_EINVAL, "overlap_row_stride %lld < nkb %d", (long long)stride, nkb);
    return BSA_OK;
}

int validate_slab_coverage(const double* cams, int n_cams, const int32_t* perm, int T, int H, int W, int block,
                           const int32_t* frame_cam, const float* depth, const int32_t* h_cam, const double* h_geom,
                           int n_h, const float* coverage) {
    if (!cams || n_cams < 1) return fail(BSA_EINVAL, "cams must be non-NULL with n_cams >= 1");
    if (T < 1 || H < 1 || W < 1) return fail(BSA_EINVAL, "grid %d x %d x %d: dimensions must be >= 1", T, H, W);
    if (!cells_fit(T, H, W)) return fail(BSA_EINVAL, "grid exceeds 2^31-1 cells");
    if (block < 1) return fail(BSA_EINVAL, "block %d < 1", block);
    if (!perm || !frame_cam || !depth || !coverage)
        return fail(BSA_EINVAL, "perm, frame_cam, depth and coverage must be non-NULL");
    if (n_h < 0 || (n_h > 0 && (!h_cam || !h_geom)))
        return fail(BSA_EINVAL, "historical slabs: count >= 0, cameras and geometry non-NULL when given");
    if (n_h > 65535 * 128) return fail(BSA_EUNSUPPORTED, "%d historical slabs exceed %d", n_h, 65535 * 128);
    return BSA_OK;
}

}  // namespace bsa

extern "C" {

int bsa_version(void) { return 100; }  // 0.1.0

const char* bsa_strerror(int status) {
    switch (status) {
        case BSA_OK: return "ok";
        case BSA_EINVAL: return "invalid argument";
        case BSA_EUNSUPPORTED: return "unsupported configuration";
        case BSA_EWORKSPACE: return "workspace missing or too small";
        case BSA_EHIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char* bsa_last_error_detail(void) { return bsa::last_detail(); }

size_t bsa_route_workspace_size(const bsa_route_args* args) {
    bsa::RouteLayout lay;
    if (bsa::validate_route(args, &lay) != BSA_OK) return 0;
    return lay.total;
}

size_t bsa_route_materialize_workspace_size(const bsa_route_args* args, const bsa_materialize_args* margs) {
    bsa::RouteLayout lay;
    if (bsa::validate_materialize(args, margs, &lay) != BSA_OK) return 0;
    return lay.total;
}

size_t bsa_slab_coverage_workspace_size(int T, int H, int W) {
    if (T < 1 || H < 1 || W < 1 || !bsa::cells_fit(T, H, W)) return 0;
    return sizeof(uint32_t) * (size_t)bsa::ceil_div((int64_t)T * H * W, 32);
}

}  // extern "C"
