// Host-only driver of the C ABI's argument validation (csrc/validate.cpp),
// built with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_sanitize_validate.py: valid arguments, every error path, and
// extreme sizes and strides, which must come back as errors with no
// undefined behaviour (no signed overflow, no pointer wrap-around, no
// out-of-bounds access).  Prints "validate driver: N checks passed".
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "common.h"

using namespace bsa;

static int g_checks = 0;

static void expect(int got, int want, const char* what) {
    ++g_checks;
    if (got != want) {
        std::fprintf(stderr, "FAIL %s: got %d want %d (%s)\n", what, got, want, last_detail());
        std::exit(1);
    }
}

int main() {
    alignas(16) static char buf_a[1 << 16], buf_b[1 << 16];
    alignas(16) static double pool[1 << 12];
    static int32_t ints[1 << 12];
    const int64_t big = INT64_MAX / 2, huge = INT64_MAX;

    // Gilbert index
    expect(validate_gilbert_index(3, 30, 52, ints), BSA_OK, "index ok");
    expect(validate_gilbert_index(0, 30, 52, ints), BSA_EINVAL, "index T=0");
    expect(validate_gilbert_index(65536, 65536, 2, ints), BSA_EINVAL, "index > 2^31 cells");
    expect(validate_gilbert_index(3, 30, 52, nullptr), BSA_EINVAL, "index null perm");

    // permutation
    expect(validate_gilbert_perm(buf_a, buf_b, ints, 100, 2, 64, 64, 128, 128 * 64, 0, BSA_BF16), BSA_OK, "perm ok");
    expect(validate_gilbert_perm(buf_a, buf_b, ints, 100, 2, 64, 64, 128, 128 * 64, 2, BSA_BF16), BSA_EINVAL,
           "perm inverse=2");
    expect(validate_gilbert_perm(buf_a, buf_a + 64, ints, 100, 2, 64, 64, 128, 128 * 64, 0, BSA_BF16), BSA_EINVAL,
           "perm overlap");
    expect(validate_gilbert_perm(buf_a, buf_b, ints, 100, 2, 96, 64, 192, 128 * 96, 0, BSA_BF16), BSA_EUNSUPPORTED,
           "perm d=96");
    expect(validate_gilbert_perm(buf_a, buf_b, ints, 100, 2, 64, 64, 129, 128 * 64, 0, BSA_BF16), BSA_EINVAL,
           "perm stride unaligned");
    for (int64_t s : {big, huge, (int64_t)1 << 62})
        expect(validate_gilbert_perm(buf_a, buf_b, ints, 100, 2, 64, 64, s, 128 * 64, 0, BSA_BF16), BSA_EINVAL,
               "perm huge token stride");
    for (int64_t s : {big, huge})
        expect(validate_gilbert_perm(buf_a, buf_b, ints, INT32_MAX, 2, 64, 64, 128, s, 1, BSA_F32), BSA_EINVAL,
               "perm huge head stride");

    // permutation + pooling
    expect(validate_gilbert_perm_pool(buf_a, buf_b, ints, 100, 2, 64, 64, 128, 128 * 64, BSA_BF16, pool, 2 * 64),
           BSA_OK, "pool ok");
    expect(validate_gilbert_perm_pool(buf_a, nullptr, ints, 100, 2, 64, 64, 128, 0, BSA_F32, pool, 2 * 64), BSA_OK,
           "pool only ok");
    expect(validate_gilbert_perm_pool(buf_a, nullptr, ints, 100, 2, 64, 64, 128, 0, BSA_F32,
                                      reinterpret_cast<const double*>(buf_a), 2 * 64),
           BSA_EINVAL, "pool overlaps src");
    expect(validate_gilbert_perm_pool(buf_a, buf_b, ints, 100, 2, 64, 64, 128, 128 * 64, BSA_BF16, pool, 64),
           BSA_EINVAL, "pool stride short");
    for (int64_t s : {big, huge})
        expect(validate_gilbert_perm_pool(buf_a, nullptr, ints, 1000, 70000, 64, 64, 1 << 23, 0, BSA_F32, pool, s),
               BSA_EINVAL, "pool huge heads/stride");
    for (int64_t s : {big, huge})
        expect(validate_gilbert_perm_pool(buf_a, nullptr, ints, 1000, 2, 64, 64, s, 0, BSA_F32, pool, 1 << 20),
               BSA_EINVAL, "pool-only huge token stride");

    // batched permutation + pooling
    bsa_perm_job jobs[3];
    std::memset(jobs, 0, sizeof(jobs));
    jobs[0] = {buf_a, buf_b, 128, 128 * 64, nullptr, 0};
    jobs[1] = {buf_a, nullptr, 128, 0, pool, 2 * 64};
    expect(validate_gilbert_perm_pool_batch(jobs, 2, ints, 100, 2, 64, 64, BSA_BF16), BSA_OK, "batch ok");
    jobs[1].pool = reinterpret_cast<double*>(buf_b);
    expect(validate_gilbert_perm_pool_batch(jobs, 2, ints, 100, 2, 64, 64, BSA_BF16), BSA_EINVAL, "batch overlap");
    expect(validate_gilbert_perm_pool_batch(jobs, 0, ints, 100, 2, 64, 64, BSA_BF16), BSA_EINVAL, "batch n=0");
    expect(validate_gilbert_perm_pool_batch(jobs, BSA_MAX_PERM_JOBS + 1, ints, 100, 2, 64, 64, BSA_BF16), BSA_EINVAL,
           "batch n too large");
    jobs[1] = {buf_a, nullptr, huge, 0, pool, 2 * 64};
    expect(validate_gilbert_perm_pool_batch(jobs, 2, ints, 100, 2, 64, 64, BSA_BF16), BSA_EINVAL,
           "batch huge stride");
    {   // a long error detail is truncated, never overrun
        char name[2048];
        std::memset(name, 'x', sizeof(name) - 1);
        name[sizeof(name) - 1] = 0;
        fail(BSA_EINVAL, "%s", name);
        expect((int)(std::strlen(last_detail()) < 512), 1, "detail truncated");
        expect(validate_gilbert_perm_pool_batch(jobs, 2, ints, 100, 2, 64, 64, BSA_BF16), BSA_EINVAL,
               "batch nested detail");
    }

    // attention
    AttnProblem p;
    std::memset(&p, 0, sizeof(p));
    p.q = p.k = p.v = buf_a;
    p.o = buf_b;
    p.dtype = BSA_BF16;
    p.heads = 2, p.d = 128, p.block = 128, p.nqb = 3, p.nkb = 5;
    p.q_hs = p.o_hs = 3 * 128 * 128;
    p.k_hs = p.v_hs = 5 * 128 * 128;
    p.row_ptr = ints, p.col_idx = ints, p.col_len = 10, p.scale = 0.1f;
    expect(validate_attn(p, false), BSA_OK, "attn ok");
    expect(validate_attn(p, true), BSA_OK, "dense ok");
    AttnProblem r = p;
    r.scale = 0.0f;
    expect(validate_attn(r, false), BSA_EINVAL, "attn scale 0");
    r = p;
    r.col_len = -1;
    expect(validate_attn(r, false), BSA_EINVAL, "attn col_len < 0");
    r = p;
    r.heads = 1 << 20, r.nqb = 1 << 20;
    expect(validate_attn(r, false), BSA_EINVAL, "attn heads*nqb overflow");
    for (int64_t s : {big, huge}) {
        r = p;
        r.q_hs = s;
        expect(validate_attn(r, false), BSA_EINVAL, "attn huge q stride");
        r = p;
        r.k_hs = s;
        expect(validate_attn(r, true), BSA_EINVAL, "attn huge k stride");
    }
    r = p;
    r.nkb = INT32_MAX, r.nqb = INT32_MAX / 4;
    expect(validate_attn(r, false), BSA_EINVAL, "attn huge nkb");
    r = p;
    r.o_map = ints, r.o_map_len = 300, r.o_ts = 2 * 128;
    expect(validate_raster_out(r), BSA_OK, "raster ok");
    r.o_map_len = 3 * 128 + 1;
    expect(validate_raster_out(r), BSA_EINVAL, "raster rows > nqb*block");
    r.o_map_len = 300;
    for (int64_t s : {big, huge}) {
        r.o_ts = s;
        expect(validate_raster_out(r), BSA_EINVAL, "raster huge o stride");
    }
    r.o_ts = 2 * 128, r.q_map = ints, r.q_map_len = 300, r.q_ts = huge;
    expect(validate_raster_out(r), BSA_EINVAL, "raster huge q stride");

    // router
    bsa_route_args a;
    std::memset(&a, 0, sizeof(a));
    a.struct_size = sizeof(a);
    a.q = a.k = buf_a;
    a.row_ptr = ints, a.col_idx = ints;
    a.dtype = BSA_BF16, a.heads = 2, a.d = 128, a.block = 128, a.nqb = 3, a.nkb = 6;
    a.q_head_stride = 3 * 128 * 128, a.k_head_stride = 6 * 128 * 128;
    a.scale = 0.1, a.k_fixed = 4, a.col_capacity = 2 * 3 * 4;
    RouteLayout lay;
    expect(validate_route(&a, &lay), BSA_OK, "route ok");
    expect((int)(bsa_route_workspace_size(&a) == lay.total), 1, "workspace size");
    bsa_route_args b = a;
    b.struct_size = 1;
    expect(validate_route(&b, &lay), BSA_EINVAL, "route struct_size");
    b = a;
    b.col_capacity = 5;
    expect(validate_route(&b, &lay), BSA_EINVAL, "route capacity");
    b = a;
    b.nkb = 70000, b.k_head_stride = (int64_t)70000 * 128 * 128, b.col_capacity = 1 << 20;
    expect(validate_route(&b, &lay), BSA_EUNSUPPORTED, "route too many candidates");
    b = a;
    b.nkb = 9000, b.k_head_stride = (int64_t)9000 * 128 * 128, b.k_fixed = 3000, b.col_capacity = 1 << 20;
    expect(validate_route(&b, &lay), BSA_EUNSUPPORTED, "route segments x cap");
    b.k_fixed = 1000;
    expect(validate_route(&b, &lay), BSA_OK, "route two-level ok");
    expect((int)(lay.n_seg == 3 && lay.seg_cap == 1000), 1, "route two-level layout");
    for (int64_t s : {big, huge}) {
        b = a;
        b.k_head_stride = s;
        expect(validate_route(&b, &lay), BSA_EINVAL, "route huge k stride");
        b = a;
        b.col_capacity = s;
        b.k_fixed = INT32_MAX;
        b.heads = 1 << 12, b.nqb = 1 << 12;
        expect(validate_route(&b, &lay), BSA_EINVAL, "route huge heads*nqb");
    }
    b = a;
    b.scale = 1e308;
    expect(validate_route(&b, &lay), BSA_EINVAL, "route scale");
    bsa_materialize_args m;
    std::memset(&m, 0, sizeof(m));
    m.struct_size = sizeof(m);
    m.k_cov = 4, m.k_unc = 5, m.eta_cov = 0.9, m.mass = 0.9, m.prev_begin = 0, m.prev_end = 3;
    b = a;
    b.k_fixed = 0, b.col_capacity = 2 * 3 * 6;
    expect(validate_materialize(&b, &m, &lay), BSA_OK, "materialize ok");
    bsa_materialize_args n = m;
    n.prev_end = -1;
    expect(validate_materialize(&b, &n, &lay), BSA_EINVAL, "materialize prev range");
    n = m;
    n.window = ints, n.window_len = ints, n.window_stride = INT32_MAX;
    b.col_capacity = huge;
    expect(validate_materialize(&b, &n, &lay), BSA_OK, "materialize big window stride");

    // windows, tiles, slabs
    expect(validate_block_window(ints, ints, 3, 30, 52, 128, 47, ints, ints, 74), BSA_OK, "window ok");
    expect(validate_block_window(ints, ints, 3, 30, 52, 128, INT32_MAX, ints, ints, 74), BSA_EINVAL,
           "window q_chunk huge");
    expect(validate_tile_index(3, 30, 52, 1, 8, 16, ints, ints), BSA_OK, "tile index ok");
    expect(validate_tile_index(INT32_MAX, INT32_MAX, INT32_MAX, 1, 1, 1, ints, ints), BSA_EINVAL, "tile index huge");
    expect(validate_tile_perm(buf_a, buf_b, ints, 256, 200, 2, 64, 128, 256 * 64, 0, BSA_BF16), BSA_OK,
           "tile perm ok");
    for (int64_t s : {big, huge})
        expect(validate_tile_perm(buf_a, buf_b, ints, 256, INT32_MAX, 2, 64, s, 256 * 64, 0, BSA_BF16), BSA_EINVAL,
               "tile perm huge stride");
    expect(validate_tile_block_window(ints, ints, 256, 3, 30, 52, 128, 2, ints, ints, 4), BSA_OK,
           "tile window ok");
    expect(validate_slab_overlap(pool, 1, ints, ints, pool, 3, 1, ints, ints, pool, 5, 1, 8,
                                 reinterpret_cast<const float*>(buf_b), 5),
           BSA_OK, "slab overlap ok");
    expect(validate_slab_overlap(pool, 1, ints, ints, pool, 3, 1, ints, ints, pool, 5, 1, 65,
                                 reinterpret_cast<const float*>(buf_b), 5),
           BSA_EINVAL, "slab grid_n");
    expect(validate_slab_coverage(pool, 1, ints, 3, 30, 52, 128, ints, reinterpret_cast<const float*>(buf_a), ints,
                                  pool, 2, reinterpret_cast<const float*>(buf_b)),
           BSA_OK, "slab coverage ok");

    // error strings for every status
    for (int st = -2; st <= 8; ++st) expect((int)(bsa_strerror(st) != nullptr), 1, "strerror");
    expect((int)(bsa_slab_coverage_workspace_size(3, 30, 52) > 0), 1, "coverage workspace");
    std::printf("validate driver: %d checks passed\n", g_checks);
    return 0;
}
